// Append-time quantization steps shared by the append kernels and the fused
// append + decode kernel, so that both store the same codes, scales and
// zero-points bit for bit.
//
// Operations (cited by page title and section):
//  - per-token FP8 E4M3 / INT8: "KV Cache Quantization" (infra.bea.ai) §4
//    "FP8 KV Cache" (scale from the maximum absolute value, stored with the
//    data); "KV Cache Quantization in Production LLM Serving" (llms.blog)
//    "1. FP8 KV Cache" (OCP E4M3) and "2. INT8 and INT4 Uniform Group-Wise
//    Quantization" ([-127, 127]); n4n.ai "Step 3: Implement quantization
//    hooks" (x / scale, round half to even, clamp).
//  - KIVI group flush: infra.bea.ai §3 (Key per channel over a group of
//    tokens, Value per token over groups of channels, "Residual Cache for
//    Streaming"); llms.blog "3. KIVI" (tokens leaving the residual window
//    are quantized and packed).
//
// Arithmetic is fp32 with true IEEE division and round-half-even (rintf);
// the formulas hold no product that could fuse into an add, and every
// function also disables contraction, so the result does not depend on the
// flags of the file that includes it.
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr int kQuantThreads = 256;  // workgroup size the group-flush steps assume

// ---------------------------------------------------------------------------
// Per-token FP8 E4M3 / INT8: one wave quantizes one token row, CPL = D / 64
// channels per lane (channel lane * CPL + j in x[j]).
// ---------------------------------------------------------------------------
// Two floats to a bfloat16 pair, round to nearest even (x0 in the low half).
typedef __bf16 quant_bf16x2 __attribute__((ext_vector_type(2)));
typedef float quant_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair_rne(float x0, float x1) {
  const quant_f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, quant_bf16x2));
}

// Returns the lane's CPL codes (channel lane * CPL + j in byte j; BF16: in
// the 16-bit half j) and sets *scale to the row's scale (1 for BF16, whose
// codes are the bfloat16 values). Wave-collective for FP8/INT8.
template <int FMT, int CPL>
__device__ __forceinline__ uint32_t quantize_token_lane(const float (&x)[CPL], float* scale) {
#pragma clang fp contract(off)
  if constexpr (FMT == KVQ_FMT_BF16) {
    *scale = 1.0f;
    const uint32_t w = bf16_pair_rne(x[0], CPL == 2 ? x[CPL - 1] : 0.0f);
    return CPL == 2 ? w : (w & 0xffffu);
  }
  if constexpr (FMT == KVQ_FMT_FP8_STATIC) {
    // the static scale 1.0: E4M3 of the value, saturated to +-448
    *scale = 1.0f;
    const float y0 = fminf(fmaxf(x[0], -448.0f), 448.0f);
    const float y1 = CPL == 2 ? fminf(fmaxf(x[CPL - 1], -448.0f), 448.0f) : 0.0f;
    return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false)) & (CPL == 2 ? 0xffffu : 0xffu);
  }
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) a = fmaxf(a, fabsf(x[j]));
  a = wave_max(a);
  const float s = a / (FMT == KVQ_FMT_FP8_E4M3 ? 448.0f : 127.0f);
  uint32_t codes = 0;
  if constexpr (FMT == KVQ_FMT_INT8) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float qv = 0.0f;
      if (s > 0.0f) qv = fminf(fmaxf(rintf(x[j] / s), -127.0f), 127.0f);
      codes |= (uint32_t(int32_t(qv)) & 0xffu) << (8 * j);
    }
  } else {
    float y[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (s > 0.0f) y[j] = fminf(fmaxf(x[j] / s, -448.0f), 448.0f);
    }
    // OCP E4M3, round to nearest even; inputs are already within +-448.
    codes = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false)) & (CPL == 2 ? 0xffffu : 0xffu);
  }
  *scale = s;
  return codes;
}

// ---------------------------------------------------------------------------
// Cross-lane steps without LDS: DPP moves within 16-lane rows.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float v) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false);
  return fmaxf(v, __builtin_bit_cast(float, y));
}
// Maximum over each aligned run of L lanes (L = 8 or 16) of a non-negative
// float (an absolute maximum), left in every lane of the run: quad swaps,
// then the half-row mirror (lane k <-> 7 - k) and for 16 the row mirror
// (k <-> 15 - k), each pairing runs already reduced. Non-negative floats
// order as their bit patterns, so each step is one unsigned maximum with a
// DPP operand (no NaN canonicalization).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umax_step(uint32_t v) {
  return max(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xf, 0xf, true)));
}
template <int L>
__device__ __forceinline__ float run_absmax(float a) {
  static_assert(L == 8 || L == 16, "runs of 8 or 16 lanes");
  uint32_t v = __builtin_bit_cast(uint32_t, a);
  v = dpp_umax_step<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_umax_step<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_umax_step<0x141>(v);  // row_half_mirror
  if constexpr (L == 16) v = dpp_umax_step<0x140>(v);  // row_mirror
  return __builtin_bit_cast(float, v);
}
// ---------------------------------------------------------------------------
// Quotients rounded to nearest even without the full division sequence. For
// a divisor b in [2^-60, 2^60] (in_div_range), the reciprocal seed of the
// hardware (within 1 ulp of 1/b) is refined once by Newton's step, and the
// quotient a * y is corrected twice with exact fused-multiply-add residuals
// a - b q. These are the steps of the library's correctly rounded division
// once its range scaling is the identity, which it is for such b and any a
// whose quotient can change a code (|a / b| >= 2^-12: a and every residual
// stay normal); for smaller quotients the result is still within an ulp and
// carries the sign of a, which is all a code of such a value depends on. The
// reciprocal part depends on b alone and is shared by all quotients by b.
// ---------------------------------------------------------------------------
// Callers use it where every divisor of a wave is in range (a wave-uniform
// test) and take true divisions otherwise.
__device__ __forceinline__ bool in_div_range(float b) {
  return b >= 0x1p-60f && b <= 0x1p60f;
}
__device__ __forceinline__ float recip_refined(float b) {
  const float y0 = __builtin_amdgcn_rcpf(b);
  return __builtin_fmaf(__builtin_fmaf(-b, y0, 1.0f), y0, y0);
}
// SIGNED: also carry the sign of a onto the result (needed where the code of
// a tiny quotient keeps its sign, as E4M3's signed zero does; an integer
// code of a tiny quotient is 0 whatever its sign).
template <bool SIGNED = true>
__device__ __forceinline__ float div_refined(float a, float b, float y) {
#pragma clang fp contract(off)
  float q = a * y;
  float r = __builtin_fmaf(-b, q, a);
  q = __builtin_fmaf(r, y, q);
  r = __builtin_fmaf(-b, q, a);
  q = __builtin_fmaf(r, y, q);
  return SIGNED ? __builtin_copysignf(q, a) : q;
}

// Order-preserving map of a float to an unsigned integer (finite values;
// -0 sorts just below +0) and its inverse, so that run minima and maxima of
// signed values are single unsigned DPP steps.
__device__ __forceinline__ uint32_t float_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __builtin_bit_cast(float, k ^ (uint32_t(int32_t(~k) >> 31) | 0x80000000u));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_umin_step(uint32_t v) {
  return min(v, uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xf, 0xf, true)));
}
// Minimum and maximum keys over each aligned run of L lanes (L = 4 or 8).
template <int L>
__device__ __forceinline__ void run_minmax_keys(uint32_t& kmin, uint32_t& kmax) {
  static_assert(L == 4 || L == 8, "runs of 4 or 8 lanes");
  kmin = dpp_umin_step<0xb1>(kmin);
  kmax = dpp_umax_step<0xb1>(kmax);
  kmin = dpp_umin_step<0x4e>(kmin);
  kmax = dpp_umax_step<0x4e>(kmax);
  if constexpr (L == 8) {
    kmin = dpp_umin_step<0x141>(kmin);
    kmax = dpp_umax_step<0x141>(kmax);
  }
}

// a / c for a >= 0 and a constant divisor c in [2^-60, 2^60] (a scale from a
// range or an absolute maximum): the refined-reciprocal quotient where a is
// zero or at least 2^-90 (a, the quotient and every residual stay normal),
// a true division for the rest (lanes that take it branch around it).
__device__ __forceinline__ float quot_nonneg(float a, float c, float rc) {
  float q;
  if (a == 0.0f || a >= 0x1p-90f) q = div_refined<false>(a, c, rc);
  else q = a / c;
  return q;
}

// The value of lane l ^ 2 (the other half of each quad).
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4e, 0xf, 0xf, false));
}

// 4x4 byte transpose: out[e] byte j = in[j] byte e.
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t (&in)[4], uint32_t (&out)[4]) {
  const uint32_t p0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // in0.b0 in1.b0 in0.b1 in1.b1
  const uint32_t p1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // in0.b2 in1.b2 in0.b3 in1.b3
  const uint32_t q0 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t q1 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(q0, p0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(q0, p0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(q1, p1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(q1, p1, 0x07060302u);
}

// Stores one lane's codes and (lane 0) the scale of token t of pair `pair`:
// Key rows token-major, Value codes in 8-token blocks with one 8-byte word
// per (permuted) channel slot; BF16: 2-byte codes, 16-byte Value words in
// channel order, no scale.
template <int FMT, int CPL>
__device__ __forceinline__ void store_token_codes(const CacheView& cv, size_t pair, int t, bool value, int lane,
                                                  uint32_t codes, float s) {
  constexpr int D = CPL * kWave;
  if constexpr (FMT == KVQ_FMT_BF16) {
    if (!value) {
      uint8_t* dst = cv.k_codes + ((pair * cv.cap + t) * D + lane * CPL) * 2;
      if constexpr (CPL == 2) *reinterpret_cast<uint32_t*>(dst) = codes;
      else *reinterpret_cast<uint16_t*>(dst) = uint16_t(codes);
    } else {
      uint8_t* blk = cv.v_codes + (pair * (cv.cap / 8) + t / 8) * (size_t(D) * 16) + (t & 7) * 2;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        *reinterpret_cast<uint16_t*>(blk + size_t(lane * CPL + j) * 16) = uint16_t(codes >> (16 * j));
    }
    return;
  }
  if (!value) {
    uint8_t* dst = cv.k_codes + (pair * cv.cap + t) * D + lane * CPL;
    if constexpr (CPL == 2) *reinterpret_cast<uint16_t*>(dst) = uint16_t(codes);
    else *dst = uint8_t(codes);
    if (FMT != KVQ_FMT_FP8_STATIC && lane == 0) cv.k_scale[pair * cv.cap + t] = s;
  } else {
    uint8_t* blk = cv.v_codes + (pair * (cv.cap / 8) + t / 8) * (size_t(D) * 8) + (t & 7);
#pragma unroll
    for (int j = 0; j < CPL; ++j) blk[size_t(value_slot<2>(lane * CPL + j)) * 8] = uint8_t(codes >> (8 * j));
    if (FMT != KVQ_FMT_FP8_STATIC && lane == 0) cv.v_scale[pair * cv.cap + t] = s;
  }
}

// ---------------------------------------------------------------------------
// Group-wise symmetric INT4 ("KV Cache Quantization in Production LLM
// Serving", llms.blog, "2. INT8 and INT4 Uniform Group-Wise Quantization"):
// per token and per group of G channels, s = max|x| / 7, code =
// clamp(rint(x / s), -8, 7) (within [-7, 7]), stored as the nibble code + 8.
// One wave quantizes one token row, CPL = D / 64 channels per lane.
// ---------------------------------------------------------------------------
// Returns the lane's nibbles (channel lane * CPL + j in bits [4j, 4j + 4))
// and sets *scale to the scale of the lane's channel group. Wave-collective.
template <int G, int CPL>
__device__ __forceinline__ uint32_t quantize_token_int4(const float (&x)[CPL], float* scale) {
#pragma clang fp contract(off)
  constexpr int LPG = G / CPL;  // lanes per channel group: an aligned power-of-two run
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) a = fmaxf(a, fabsf(x[j]));
#pragma unroll
  for (int o = 1; o < LPG; o <<= 1) a = fmaxf(a, __shfl_xor(a, o, kWave));
  const float s = a / 7.0f;
  uint32_t u = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float qv = 0.0f;
    if (s > 0.0f) qv = fminf(fmaxf(rintf(x[j] / s), -8.0f), 7.0f);
    u |= uint32_t(int32_t(qv) + 8) << (4 * j);
  }
  *scale = s;
  return u;
}

// Unnormalized fast Walsh-Hadamard transform of one row held by a wave
// (channel lane * CPL + j in x[j]; d = 64 * CPL): stages h = 1, 2, 4, ...,
// the pair (i, i + h) becoming (a + b, a - b). Each output is one fp32 add
// or subtract of the same two inputs in any evaluation order, so the result
// is reproducible bit for bit ("KV Cache Quantization in Production LLM
// Serving", llms.blog, "5. QuaRot and RotateKV": online fast transforms).
template <int CPL>
__device__ __forceinline__ void fwht_wave(float (&x)[CPL]) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x % kWave;
  if constexpr (CPL == 2) {
    const float a = x[0], b = x[1];
    x[0] = a + b;
    x[1] = a - b;
  }
  // the remaining channel bits are the lane's bits 0..5
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const int m = 1 << k;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const float y = __shfl_xor(x[j], m, kWave);
      x[j] = (lane & m) ? y - x[j] : x[j] + y;
    }
  }
}

// Byte of a Key row (d nibbles) that holds channel c: rows are stored in
// chunks of 8 channels, chunk (kk, r) = channels [32 kk + 8 r, 32 kk + 8 r + 8)
// at byte (d / 8) r + 4 kk, channel 32 kk + 8 r + e in nibble e of the chunk.
template <int D>
__device__ __forceinline__ int int4_key_byte(int c) {
  return (D / 8) * ((c % 32) / 8) + 4 * (c / 32) + (c % 8) / 2;
}

// Stores one lane's Key nibbles of token t and (each group's first lane) the
// token's Key scales. With CPL = 1 neighbouring lanes share a byte.
template <int G, int CPL>
__device__ __forceinline__ void store_int4_key(const CacheView& cv, size_t pair, int t, int lane, uint32_t u,
                                               float s) {
  constexpr int D = CPL * kWave;
  uint8_t* row = cv.k_codes + (pair * cv.cap + t) * (D / 2);
  if constexpr (CPL == 2) {
    row[int4_key_byte<D>(2 * lane)] = uint8_t(u);
  } else {
    const uint32_t other = uint32_t(__shfl_xor(int(u), 1, kWave));
    if ((lane & 1) == 0) row[int4_key_byte<D>(lane)] = uint8_t(u | (other << 4));
  }
  if (lane % (G / CPL) == 0) cv.k_scale[(pair * cv.cap + t) * (D / G) + (lane * CPL) / G] = s;
}

// Value word of channel c in the 8-token block holding token t (the KIVI
// INT4 layout: one 32-bit word per permuted channel slot, token t % 8 in
// bits [4 (t % 8), 4 (t % 8) + 4)).
template <int D>
__device__ __forceinline__ uint32_t* int4_value_word(const CacheView& cv, size_t pair, int t, int c) {
  return reinterpret_cast<uint32_t*>(cv.v_codes) + (pair * (cv.cap / 8) + t / 8) * D + value_slot<4>(c);
}

// ---------------------------------------------------------------------------
// KIVI group flush, one workgroup of kQuantThreads threads per group. The G
// tokens are staged in LDS as fp32; Key statistics run down each channel,
// Value statistics along each token's channel groups.
// ---------------------------------------------------------------------------
template <int G, int D>
struct FlushSmem {
  float xs[G][D + 1];
  float red_mn[kQuantThreads], red_mx[kQuantThreads];
  float sk[D], zk[D];              // Key scale, zero-point per channel
  float sv[G][D / G], zv[G][D / G];  // Value scale, zero-point per token and channel group
};

// Asymmetric code of one element: clamp(rint((x - mn) / s), 0, qmax), or 0
// for a degenerate group (s == 0).
__device__ __forceinline__ uint32_t asym_code(float x, float s, float mn, float qmax) {
#pragma clang fp contract(off)
  if (!(s > 0.0f)) return 0u;
  const float qv = fminf(fmaxf(rintf((x - mn) / s), 0.0f), qmax);
  return uint32_t(qv);
}

// 8 consecutive input elements (bf16 or fp32) from element i of p (i a
// multiple of 8, rows 16-byte aligned) as fp32, in 16-byte loads.
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, size_t i, float* x) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(a[k]);
      x[2 * k + 1] = bf16_hi(a[k]);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Stages tokens [grp*G, grp*G + G) of one pair: a token below n (already in
// the cache) comes from its residual ring slot, token t >= n from row t - n
// of the pair's T new input rows. Every thread issues all its 16-byte loads
// before it stores to LDS. No barrier.
template <bool BF16, int G, int D>
__device__ __forceinline__ void flush_stage(FlushSmem<G, D>& f, const CacheView& cv, size_t pair, int grp, int n,
                                            const void* in, int T, const uint8_t* ring) {
  constexpr int PER = G * D / (8 * kQuantThreads);  // 8-element loads per thread
  static_assert(PER * 8 * kQuantThreads == G * D, "staging tiles the group");
  float x[PER][8];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = (u * kQuantThreads + int(threadIdx.x)) * 8;
    const int i = e / D, c = e % D;
    const int t = grp * G + i;
    if (t < n) load8<BF16>(ring, (pair * cv.C + (t % cv.C)) * D + c, x[u]);
    else load8<BF16>(in, (pair * T + (t - n)) * D + c, x[u]);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = (u * kQuantThreads + int(threadIdx.x)) * 8;
    const int i = e / D, c = e % D;
#pragma unroll
    for (int k = 0; k < 8; ++k) f.xs[i][c + k] = x[u][k];
  }
}

// A scale or zero-point as stored: fp32, or rounded to binary16 (M16;
// nearest, ties to even), whose value the codes are then taken against.
// store_meta writes element i of a metadata array of either width.
template <bool M16>
__device__ __forceinline__ float stored_meta(float x) {
  if constexpr (M16) return float(_Float16(x)) + 0.0f;
  else return x;
}
template <bool M16>
__device__ __forceinline__ void store_meta(float* base, size_t i, float x) {
  if constexpr (M16) reinterpret_cast<_Float16*>(base)[i] = _Float16(x);
  else base[i] = x;
}

// Key half of a flush from the staged tile: per-channel scale and
// zero-point (stored, and kept in f.sk / f.zk) and the packed codes.
// Starts and ends with a barrier. M16: binary16 metadata.
template <int BITS, int G, int D, bool M16 = false>
__device__ __forceinline__ void flush_key(FlushSmem<G, D>& f, const CacheView& cv, size_t pair, int grp) {
#pragma clang fp contract(off)
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr int P = kQuantThreads / D;  // threads per channel
  const int tid = threadIdx.x;
  __syncthreads();
  {
    const int c = tid % D, part = tid / D;
    float mn = INFINITY, mx = -INFINITY;
    for (int i = part; i < G; i += P) {
      const float x = f.xs[i][c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    f.red_mn[tid] = mn;
    f.red_mx[tid] = mx;
  }
  __syncthreads();
  if (tid < D) {
    float mn = f.red_mn[tid], mx = f.red_mx[tid];
#pragma unroll
    for (int p = 1; p < P; ++p) {
      mn = fminf(mn, f.red_mn[p * D + tid]);
      mx = fmaxf(mx, f.red_mx[p * D + tid]);
    }
    const float s = stored_meta<M16>((mx - mn) / QMAX + 0.0f);
    const float z = stored_meta<M16>(mn + 0.0f);
    f.sk[tid] = s;
    f.zk[tid] = z;
    const size_t si = (pair * (cv.cap / G) + grp) * D + tid;
    store_meta<M16>(cv.k_scale, si, s);
    store_meta<M16>(cv.k_zero, si, z);
  }
  __syncthreads();
  {
    constexpr int CW = 32 / BITS;  // channels per 32-bit word
    constexpr int W = D / CW;      // words per token row
    uint32_t* rows = reinterpret_cast<uint32_t*>(cv.k_codes + (pair * cv.cap + size_t(grp) * G) * (D * BITS / 8));
    for (int w = tid; w < G * W; w += kQuantThreads) {
      const int i = w / W, c0 = (w % W) * CW;
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < CW; ++j)
        word |= asym_code(f.xs[i][c0 + j], f.sk[c0 + j], f.zk[c0 + j], QMAX) << (j * BITS);
      rows[w] = word;
    }
  }
  __syncthreads();
}

// Value half of a flush from the staged tile: per-token, per-channel-group
// scale and zero-point (stored, and kept in f.sv / f.zv) and the codes in
// blocks of TB tokens (8 for INT4, 16 for INT2), one 32-bit word per
// permuted channel slot. Starts and ends with a barrier. M16: binary16
// metadata.
template <int BITS, int G, int D, bool M16 = false>
__device__ __forceinline__ void flush_value(FlushSmem<G, D>& f, const CacheView& cv, size_t pair, int grp) {
#pragma clang fp contract(off)
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr int NVG = D / G;              // Value channel groups per token
  constexpr int TP = kQuantThreads / D;   // threads per (token, channel group)
  constexpr int CPT = G / TP;             // channels per thread in a Value group
  static_assert(G * NVG == D, "value groups tile head_dim");
  const int tid = threadIdx.x;
  __syncthreads();
  {
    const int pr = tid / TP, part = tid % TP;
    const int i = pr / NVG, j = pr % NVG;
    float mn = INFINITY, mx = -INFINITY;
    for (int k = 0; k < CPT; ++k) {
      const float x = f.xs[i][j * G + part * CPT + k];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int o = 1; o < TP; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    }
    if (part == 0) {
      const float s = stored_meta<M16>((mx - mn) / QMAX + 0.0f);
      const float z = stored_meta<M16>(mn + 0.0f);
      f.sv[i][j] = s;
      f.zv[i][j] = z;
      const size_t vi = (pair * cv.cap + size_t(grp) * G + i) * NVG + j;
      store_meta<M16>(cv.v_scale, vi, s);
      store_meta<M16>(cv.v_zero, vi, z);
    }
  }
  __syncthreads();
  {
    constexpr int TB = BITS == 2 ? 16 : 8;
    constexpr int NB = G / TB;
    uint32_t* blocks = reinterpret_cast<uint32_t*>(cv.v_codes) + (pair * (cv.cap / TB) + size_t(grp) * NB) * D;
    for (int w = tid; w < NB * D; w += kQuantThreads) {
      const int blk = w / D, c = w % D, j = c / G;
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        const int i = blk * TB + k;
        word |= asym_code(f.xs[i][c], f.sv[i][j], f.zv[i][j], QMAX) << (k * BITS);
      }
      blocks[blk * D + value_slot<4>(c)] = word;
    }
  }
  __syncthreads();
}

}  // namespace kvq
