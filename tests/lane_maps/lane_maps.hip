// Test-only kernel: runs the decode's and the append's wave-level building
// blocks (kvq_wave.h, kvq_quant.h) on one wave of known inputs and writes
// every lane's results, so that the test can compare each lane map and
// conversion with its definition. Not part of libkvq.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_quant.h"
#include "kvq_wave.h"

namespace {

constexpr int kOut = 30;  // results per lane

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Lane l's inputs: x = ((37 l) mod 64) + 0.25 (distinct, exact in fp32 sums),
// s = ((37 l) mod 64) - 31.5 (signed, distinct).
__global__ __launch_bounds__(64) void lane_maps(uint32_t* __restrict__ out) {
  const int l = threadIdx.x;
  const float x = float((37 * l) % 64) + 0.25f;
  const float sx = float((37 * l) % 64) - 31.5f;
  uint32_t r[kOut];
  r[0] = fbits(kvq::add_ror8(x));
  r[1] = fbits(kvq::max_ror8(x));
  r[2] = fbits(kvq::max_rows(x));
  r[3] = fbits(kvq::sum_rows(x));
  r[4] = kvq::max_lanes32_bits(fbits(x));
  r[5] = kvq::swap8_into<0xc>(1000u + l, 2000u + l);
  r[6] = kvq::swap8_into<0x3>(1000u + l, 2000u + l);
  r[7] = fbits(kvq::run_absmax<8>(x));
  r[8] = fbits(kvq::run_absmax<16>(x));
  {
    uint32_t kmin = kvq::float_key(sx), kmax = kmin;
    kvq::run_minmax_keys<4>(kmin, kmax);
    r[9] = fbits(kvq::key_float(kmin));
    r[10] = fbits(kvq::key_float(kmax));
    kmin = kvq::float_key(sx);
    kmax = kmin;
    kvq::run_minmax_keys<8>(kmin, kmax);
    r[11] = fbits(kvq::key_float(kmin));
    r[12] = fbits(kvq::key_float(kmax));
  }
  r[13] = kvq::quad_swap2(1000u + l);
  {
    // in[j] byte e = 16 j + 4 e + (l mod 4)
    uint32_t in[4], t[4];
    for (int j = 0; j < 4; ++j) {
      in[j] = 0;
      for (int e = 0; e < 4; ++e) in[j] |= uint32_t(16 * j + 4 * e + (l & 3)) << (8 * e);
    }
    kvq::transpose4x4_bytes(in, t);
    for (int e = 0; e < 4; ++e) r[14 + e] = t[e];
  }
  {
    // every E4M3 byte: lane l holds bytes 4 l .. 4 l + 3
    const uint32_t w = uint32_t(4 * l) | uint32_t(4 * l + 1) << 8 | uint32_t(4 * l + 2) << 16 | uint32_t(4 * l + 3) << 24;
    r[18] = kvq::fp8x2_bf16<0>(w);
    r[19] = kvq::fp8x2_bf16<1>(w);
  }
  {
    // the integers 0..15 as bytes: lane l holds (l + k) mod 16, k = 0..3
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= uint32_t((l + k) % 16) << (8 * k);
    r[20] = kvq::e4m3_pair_f16<0>(w);
    r[21] = kvq::e4m3_pair_f16<1>(w);
  }
  r[22] = kvq::float_key(sx);
  r[23] = fbits(kvq::key_float(kvq::float_key(sx)));
  {
    // y - (a bf16 half of a pair) through the bf16 dot product with the
    // register units: pair = (bf16 truncations of y and of -y)
    const float y = x * 1.0078125f + 0.0009765625f;
    const uint32_t pair = (fbits(y) >> 16) | (fbits(-y) & 0xffff0000u);
    const kvq::Bf16Units u = kvq::bf16_units();
    r[24] = fbits(kvq::sub_bf16_half(pair, u.lo, y));
    r[25] = fbits(kvq::sub_bf16_half(pair, u.hi, -y));
  }
  {
    // 2-bit integers in the nibbles: byte k of lane l holds (l + k) mod 4
    // (low nibble) and (l + 2k + 1) mod 4 (high nibble)
    uint32_t w = 0;
    for (int k = 0; k < 4; ++k) w |= uint32_t(((l + k) % 4) | (((l + 2 * k + 1) % 4) << 4)) << (8 * k);
    r[26] = kvq::e2m1_pair_f16<0>(w);
    r[27] = kvq::e2m1_pair_f16<1>(w);
    r[28] = kvq::e2m1_pair_f16<2>(w);
    r[29] = kvq::e2m1_pair_f16<3>(w);
  }
  for (int i = 0; i < kOut; ++i) out[i * 64 + l] = r[i];
}

}  // namespace

// out: device, 30 * 64 uint32 (result i of lane l at i * 64 + l). Returns a
// hipError_t value.
extern "C" int kvq_test_lane_maps(uint32_t* out, void* stream) {
  lane_maps<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>(out);
  return int(hipGetLastError());
}
