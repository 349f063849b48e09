// Device helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

constexpr int kWave = 64;

// Element of an input/residual array as fp32 (bf16 widens exactly).
template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if constexpr (BF16) {
    const uint32_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float(b << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// KIVI flush boundary: tokens of a length-n sequence held in whole groups.
__device__ __forceinline__ int kivi_quantized(int n, int G, int R) {
  const int t = n - R;
  return t > 0 ? (t / G) * G : 0;
}

// Slot of channel c among the Value words of one token block: within each
// chunk of 16*W channels (W words per 16 bytes: 2 for 8-byte words, 4 for
// 4-byte words), slot W*m + x holds channel 16*x + m, so that one 16-byte
// load by lane m yields channel m of W consecutive 16-channel tiles.
template <int W>
__device__ __forceinline__ int value_slot(int c) {
  const int chunk = c / (16 * W), in = c % (16 * W);
  return chunk * 16 * W + W * (in % 16) + in / 16;
}

__device__ __forceinline__ size_t pair_index(const CacheView& cv, int b, int h) {
  return size_t(b) * cv.Hkv + h;
}

}  // namespace kvq
