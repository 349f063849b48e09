// Append-time quantization kernels for libkvq (gfx950).
//
// Operations (cited by page title and section):
//  - per-token FP8 E4M3: "KV Cache Quantization" (infra.bea.ai) §4 "FP8 KV
//    Cache" (scale from the maximum absolute value, stored with the data);
//    "KV Cache Quantization in Production LLM Serving" (llms.blog) "1. FP8
//    KV Cache" (OCP E4M3).
//  - per-token symmetric INT8: llms.blog "2. INT8 and INT4 Uniform Group-Wise
//    Quantization" ([-127, 127], one scale per group); n4n.ai "Step 3:
//    Implement quantization hooks" (x / scale, round half to even, clamp).
//  - KIVI: infra.bea.ai §3 (Key per channel, Value per token, "Residual
//    Cache for Streaming"); llms.blog "3. KIVI" (tokens leaving the residual
//    window are quantized and packed into memory blocks).
//
// Quantization arithmetic is fp32 with true IEEE division, round-half-even
// (rintf) and, because this file is compiled with -ffp-contract=off, no
// fused multiply-add, so codes, scales and zero-points are reproducible bit
// for bit. An append is two launches on the caller's stream: the first
// quantizes (per-token formats) or flushes whole groups (KIVI); the second,
// one workgroup per sequence, writes the tokens that stay in the KIVI
// residual ring and then advances seq_lens. Stream order makes every read
// of old ring slots and of seq_lens happen before they are overwritten.
#include <hip/hip_runtime.h>

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 32;  // tokens per workgroup in the per-token kernel

typedef float float2_t __attribute__((ext_vector_type(2)));

// Length checks shared by the append kernels: a sequence whose append would
// be malformed or overflow the capacity is left unchanged.
__device__ __forceinline__ bool append_range(const CacheView& cv, const int32_t* seq_lens,
                                             const int32_t* append_lens, int T, int b, int* n, int* tb) {
  *n = seq_lens[b];
  *tb = append_lens ? append_lens[b] : T;
  return *n >= 0 && *tb >= 0 && *tb <= T && int64_t(*n) + *tb <= cv.max_tokens;
}

// ---------------------------------------------------------------------------
// Per-token FP8 E4M3 / INT8: one wave per token row, D/64 channels per lane.
// ---------------------------------------------------------------------------
template <int FMT, int D, bool BF16>
__global__ __launch_bounds__(kThreads) void append_per_token(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                            const void* __restrict__ kin,
                                                            const void* __restrict__ vin, int T,
                                                            const int32_t* __restrict__ append_lens) {
  constexpr int CPL = D / kWave;  // channels per lane
  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const size_t pair = pair_index(cv, b, h);
  const int i_end = min(tb, int(blockIdx.x + 1) * kTokPerBlock);
  for (int i = int(blockIdx.x) * kTokPerBlock + wave; i < i_end; i += kThreads / kWave) {
    const int t = n + i;  // absolute token position in the sequence
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const void* src = which ? vin : kin;
      const size_t in_base = (pair * T + i) * D + lane * CPL;
      float x[CPL];
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        x[j] = load_elem<BF16>(src, in_base + j);
        a = fmaxf(a, fabsf(x[j]));
      }
      a = wave_max(a);
      const float s = a / (FMT == KVQ_FMT_FP8_E4M3 ? 448.0f : 127.0f);
      uint32_t codes = 0;  // CPL bytes, channel lane*CPL + j in byte j
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
      if (which == 0) {
        uint8_t* dst = cv.k_codes + (pair * cv.cap + t) * D + lane * CPL;
        if constexpr (CPL == 2) {
          *reinterpret_cast<uint16_t*>(dst) = uint16_t(codes);
        } else {
          *dst = uint8_t(codes);
        }
        if (lane == 0) cv.k_scale[pair * cv.cap + t] = s;
      } else {
        // Value codes: 8-token blocks, one 8-byte word per channel slot.
        uint8_t* blk = cv.v_codes + (pair * (cv.cap / 8) + t / 8) * (size_t(D) * 8) + (t & 7);
#pragma unroll
        for (int j = 0; j < CPL; ++j) blk[size_t(value_slot<2>(lane * CPL + j)) * 8] = uint8_t(codes >> (8 * j));
        if (lane == 0) cv.v_scale[pair * cv.cap + t] = s;
      }
    }
  }
}

// Asymmetric code of one element: clamp(rint((x - mn) / s), 0, qmax), or 0
// for a degenerate group (s == 0).
__device__ __forceinline__ uint32_t asym_code(float x, float s, float mn, float qmax) {
  if (!(s > 0.0f)) return 0u;
  const float qv = fminf(fmaxf(rintf((x - mn) / s), 0.0f), qmax);
  return uint32_t(qv);
}

// ---------------------------------------------------------------------------
// KIVI group flush: one workgroup per (group slot, kv head, sequence). The G
// tokens of a group are staged in LDS as fp32 (old ones from the residual
// ring, new ones from the input); Key statistics run down each channel,
// Value statistics along each token's channel groups.
// ---------------------------------------------------------------------------
template <int BITS, int G, int D, bool BF16>
__global__ __launch_bounds__(kThreads) void kivi_flush(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                      const void* __restrict__ kin, const void* __restrict__ vin,
                                                      int T, const int32_t* __restrict__ append_lens) {
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr int P = kThreads / D;  // threads per channel for Key statistics
  constexpr int NVG = D / G;       // Value channel groups per token
  constexpr int TP = kThreads / D; // threads per (token, channel group)
  constexpr int CPT = G / TP;      // channels per thread in a Value group
  static_assert(G * NVG == D, "value groups tile head_dim");

  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int q0 = kivi_quantized(n, G, cv.R);
  const int q1 = kivi_quantized(n + tb, G, cv.R);
  const int grp = q0 / G + int(blockIdx.x);
  if ((grp + 1) * G > q1) return;

  __shared__ float xs[G][D + 1];
  __shared__ float red_mn[kThreads], red_mx[kThreads];
  __shared__ float sk[D], zk[D];
  __shared__ float sv[G][NVG], zv[G][NVG];

  const int tid = threadIdx.x;
  const size_t pair = pair_index(cv, b, h);

  auto load_tile = [&](const void* in, const uint8_t* ring) {
    for (int e = tid; e < G * D; e += kThreads) {
      const int i = e / D, c = e % D;
      const int t = grp * G + i;
      xs[i][c] = t < n ? load_elem<BF16>(ring, (pair * cv.C + (t % cv.C)) * D + c)
                       : load_elem<BF16>(in, (pair * T + (t - n)) * D + c);
    }
  };

  // ---- Key: per channel over the G tokens ----
  load_tile(kin, cv.k_resid);
  __syncthreads();
  {
    const int c = tid % D, part = tid / D;
    float mn = INFINITY, mx = -INFINITY;
    for (int i = part; i < G; i += P) {
      const float x = xs[i][c];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
    red_mn[tid] = mn;
    red_mx[tid] = mx;
  }
  __syncthreads();
  if (tid < D) {
    float mn = red_mn[tid], mx = red_mx[tid];
#pragma unroll
    for (int p = 1; p < P; ++p) {
      mn = fminf(mn, red_mn[p * D + tid]);
      mx = fmaxf(mx, red_mx[p * D + tid]);
    }
    const float s = (mx - mn) / QMAX + 0.0f;
    const float z = mn + 0.0f;
    sk[tid] = s;
    zk[tid] = z;
    const size_t si = (pair * (cv.cap / G) + grp) * D + tid;
    cv.k_scale[si] = s;
    cv.k_zero[si] = z;
  }
  __syncthreads();
  {
    constexpr int CW = 32 / BITS;  // channels per 32-bit word
    constexpr int W = D / CW;      // words per token row
    uint32_t* rows = reinterpret_cast<uint32_t*>(cv.k_codes + (pair * cv.cap + size_t(grp) * G) * (D * BITS / 8));
    for (int w = tid; w < G * W; w += kThreads) {
      const int i = w / W, c0 = (w % W) * CW;
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < CW; ++j) word |= asym_code(xs[i][c0 + j], sk[c0 + j], zk[c0 + j], QMAX) << (j * BITS);
      rows[w] = word;
    }
  }
  __syncthreads();

  // ---- Value: per token over each group of G channels ----
  load_tile(vin, cv.v_resid);
  __syncthreads();
  {
    const int pr = tid / TP, part = tid % TP;
    const int i = pr / NVG, j = pr % NVG;
    float mn = INFINITY, mx = -INFINITY;
    for (int k = 0; k < CPT; ++k) {
      const float x = xs[i][j * G + part * CPT + k];
      mn = fminf(mn, x);
      mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int o = 1; o < TP; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    }
    if (part == 0) {
      const float s = (mx - mn) / QMAX + 0.0f;
      const float z = mn + 0.0f;
      sv[i][j] = s;
      zv[i][j] = z;
      const size_t vi = (pair * cv.cap + size_t(grp) * G + i) * NVG + j;
      cv.v_scale[vi] = s;
      cv.v_zero[vi] = z;
    }
  }
  __syncthreads();
  {
    // Blocks of TB tokens (8 for INT4, 16 for INT2): one 32-bit word per
    // channel slot holds the block's codes of that channel, token k in bits
    // [k * BITS, (k + 1) * BITS).
    constexpr int TB = BITS == 2 ? 16 : 8;
    constexpr int NB = G / TB;
    uint32_t* blocks = reinterpret_cast<uint32_t*>(cv.v_codes) + (pair * (cv.cap / TB) + size_t(grp) * NB) * D;
    for (int w = tid; w < NB * D; w += kThreads) {
      const int blk = w / D, c = w % D, j = c / G;
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < TB; ++k) {
        const int i = blk * TB + k;
        word |= asym_code(xs[i][c], sv[i][j], zv[i][j], QMAX) << (k * BITS);
      }
      blocks[blk * D + value_slot<4>(c)] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// Second launch: one workgroup per sequence. KIVI: copy the tokens that end
// in the residual window into their ring slots (bit copy, 16-byte vectors).
// Then advance seq_lens[b] once every thread has read it.
// ---------------------------------------------------------------------------
template <bool KIVI>
__global__ __launch_bounds__(kThreads) void append_finish(CacheView cv, int32_t* __restrict__ seq_lens,
                                                         const void* __restrict__ kin,
                                                         const void* __restrict__ vin, int T,
                                                         const int32_t* __restrict__ append_lens) {
  const int b = blockIdx.x;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int n1 = n + tb;
  if constexpr (KIVI) {
    const int q1 = kivi_quantized(n1, cv.G, cv.R);
    const int start = max(n, q1);
    const int rows = n1 - start;
    const int row_bytes = cv.D * (cv.bf16 ? 2 : 4);
    const int vec_per_row = row_bytes / 16;
    const int total = cv.Hkv * rows * vec_per_row;
    for (int e = threadIdx.x; e < total; e += kThreads) {
      const int v = e % vec_per_row;
      const int r = (e / vec_per_row) % rows;
      const int h = e / (vec_per_row * rows);
      const int t = start + r;
      const size_t pair = pair_index(cv, b, h);
      const size_t src = (pair * T + (t - n)) * row_bytes + size_t(v) * 16;
      const size_t dst = (pair * cv.C + (t % cv.C)) * row_bytes + size_t(v) * 16;
      *reinterpret_cast<uint4*>(cv.k_resid + dst) = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(kin) + src);
      *reinterpret_cast<uint4*>(cv.v_resid + dst) = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(vin) + src);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) seq_lens[b] = n1;
}

template <int FMT, int D, bool BF16>
void launch_per_token(const CacheView& cv, int32_t* seq_lens, const void* k, const void* v, int T,
                      const int32_t* al, hipStream_t st) {
  const dim3 grid((T + kTokPerBlock - 1) / kTokPerBlock, cv.Hkv, cv.B);
  append_per_token<FMT, D, BF16><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
}

template <int BITS, int G, int D, bool BF16>
void launch_flush(const CacheView& cv, int32_t* seq_lens, const void* k, const void* v, int T,
                  const int32_t* al, hipStream_t st) {
  const dim3 grid(T / G + 1, cv.Hkv, cv.B);
  kivi_flush<BITS, G, D, BF16><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
}

template <int FMT, bool BF16>
void per_token_d(const CacheView& cv, int32_t* sl, const void* k, const void* v, int T, const int32_t* al,
                 hipStream_t st) {
  if (cv.D == 128) launch_per_token<FMT, 128, BF16>(cv, sl, k, v, T, al, st);
  else launch_per_token<FMT, 64, BF16>(cv, sl, k, v, T, al, st);
}

template <int BITS, bool BF16>
void flush_gd(const CacheView& cv, int32_t* sl, const void* k, const void* v, int T, const int32_t* al,
              hipStream_t st) {
  if (cv.G == 32) {
    if (cv.D == 128) launch_flush<BITS, 32, 128, BF16>(cv, sl, k, v, T, al, st);
    else launch_flush<BITS, 32, 64, BF16>(cv, sl, k, v, T, al, st);
  } else {
    if (cv.D == 128) launch_flush<BITS, 64, 128, BF16>(cv, sl, k, v, T, al, st);
    else launch_flush<BITS, 64, 64, BF16>(cv, sl, k, v, T, al, st);
  }
}

}  // namespace

hipError_t launch_append(const CacheView& cv, int32_t* seq_lens, const void* k_new, const void* v_new, int T,
                         const int32_t* append_lens, hipStream_t stream) {
  if (cv.fmt == KVQ_FMT_KIVI) {
    if (cv.bits == 4) {
      if (cv.bf16) flush_gd<4, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else flush_gd<4, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else {
      if (cv.bf16) flush_gd<2, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else flush_gd<2, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    }
    append_finish<true><<<cv.B, kThreads, 0, stream>>>(cv, seq_lens, k_new, v_new, T, append_lens);
  } else {
    if (cv.fmt == KVQ_FMT_FP8_E4M3) {
      if (cv.bf16) per_token_d<KVQ_FMT_FP8_E4M3, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_FP8_E4M3, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else {
      if (cv.bf16) per_token_d<KVQ_FMT_INT8, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_INT8, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    }
    append_finish<false><<<cv.B, kThreads, 0, stream>>>(cv, seq_lens, k_new, v_new, T, append_lens);
  }
  return hipGetLastError();
}

}  // namespace kvq
