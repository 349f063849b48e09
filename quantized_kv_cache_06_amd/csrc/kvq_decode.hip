// Decode attention over the quantized cache (gfx950): split-K partials and
// the cross-split merge.
//
// Operation: one query token per sequence attends to every cached token
// while the codes are dequantized in registers — "KV cache quantization"
// (guide.dupenodi.dev) "Key takeaways": the attention kernel must read the
// quantized cache; "How KV cache quantization reduces GPU memory" (n4n.ai)
// "Step 5": a separate dequantize pass gives the bandwidth savings away;
// "KV Cache Quantization in Production LLM Serving" (llms.blog) "Serving
// Economics": decode is bound by memory bandwidth.
//
// decode_split: one workgroup per (split, kv head, sequence). The split's
// tokens are processed in chunks of 256: one thread per token computes the
// g query heads' scores, an online softmax keeps (running max m, running sum
// l) per head, and threads laid out over (channel, token part) accumulate the
// unnormalized output. KIVI's last split also covers the residual ring.
// decode_merge: per (query head, sequence), rescales the splits' partial
// states to a common maximum and normalizes.
#include <hip/hip_runtime.h>

#include "kvq_device.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;

typedef float float2_t __attribute__((ext_vector_type(2)));

// Dequantized value of code k (KIVI: code * s + z).
__device__ __forceinline__ float kivi_value(uint32_t code, float s, float z) { return fmaf(float(code), s, z); }

template <int FMT, int BITS, int D, int NH, bool BF16>
__global__ __launch_bounds__(kThreads) void decode_split(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                        const void* __restrict__ q, float sm_scale, DecodeWork wk) {
  constexpr bool KIVI = FMT == KVQ_FMT_KIVI;
  constexpr int P = kThreads / D;           // token parts in the PV phase
  constexpr int RB = D * BITS / 8;          // bytes per Key code row
  constexpr int KGRP = kChunk / 32;         // Key groups per chunk at the smallest group (32)
  constexpr int NVG_MAX = D / 32;           // Value groups per token at the smallest group
  static_assert(P * D == kThreads, "thread layout");

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = cv.g;
  const int G = cv.G;
  int n = seq_lens[b];
  n = min(max(n, 0), cv.max_tokens);
  const int nq = KIVI ? kivi_quantized(n, G, cv.R) : n;
  const int L = wk.L;
  if (s > nq / L) return;
  const int t0 = s * L;
  const int t1 = min(t0 + L, nq);
  const bool has_resid = KIVI && (s == nq / L) && (n > nq);
  const size_t pair = pair_index(cv, b, h);

  __shared__ float qs[NH][D];
  __shared__ float sc[NH > 8 ? NH : 8][kChunk];   // scores -> probabilities; reused for the final reduction
  __shared__ float pv[NH][kChunk];                  // probability x Value scale (per-token formats)
  __shared__ float st_m[NH], st_l[NH], st_a[NH];
  __shared__ float kss[KIVI ? KGRP : 1][D], kzs[KIVI ? KGRP : 1][D];
  __shared__ float vss[KIVI ? kChunk : 1][NVG_MAX], vzs[KIVI ? kChunk : 1][NVG_MAX];

  for (int e = tid; e < NH * D; e += kThreads) {
    const int j = e / D, c = e % D;
    qs[j][c] = j < g ? load_elem<BF16>(q, (size_t(b) * cv.Hq + size_t(h) * g + j) * D + c) : 0.0f;
  }
  if (tid < NH) {
    st_m[tid] = -INFINITY;
    st_l[tid] = 0.0f;
    st_a[tid] = 1.0f;
  }
  const int c = tid % D, part = tid / D;
  float acc[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) acc[j] = 0.0f;
  __syncthreads();

  // Online-softmax update over the nt scores of one chunk (waves take heads).
  auto softmax_chunk = [&](int nt, int cs) {
    for (int j = wave; j < NH; j += kThreads / kWave) {
      if (j >= g) continue;
      float mx = -INFINITY;
      for (int i = lane; i < nt; i += kWave) mx = fmaxf(mx, sc[j][i]);
      mx = wave_max(mx);
      const float m_old = st_m[j];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = __expf(m_old - m_new);
      float sum = 0.0f;
      for (int i = lane; i < nt; i += kWave) {
        const float p = __expf(sc[j][i] - m_new);
        sc[j][i] = p;
        sum += p;
        if constexpr (!KIVI) pv[j][i] = p * cv.v_scale[pair * cv.cap + cs + i];
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        st_m[j] = m_new;
        st_l[j] = st_l[j] * alpha + sum;
        st_a[j] = alpha;
      }
    }
  };

  // ---------------- quantized tokens ----------------
  for (int cs = t0; cs < t1; cs += kChunk) {
    const int nt = min(kChunk, t1 - cs);
    if constexpr (KIVI) {
      const int g0 = cs / G, ng = (nt + G - 1) / G, nvg = D / G;
      for (int e = tid; e < ng * D; e += kThreads) {
        const int gi = e / D, cc = e % D;
        const size_t si = (pair * (cv.cap / G) + g0 + gi) * D + cc;
        kss[gi][cc] = cv.k_scale[si];
        kzs[gi][cc] = cv.k_zero[si];
      }
      for (int e = tid; e < nt * nvg; e += kThreads) {
        const size_t vi = (pair * cv.cap + cs) * nvg + e;
        vss[e / nvg][e % nvg] = cv.v_scale[vi];
        vzs[e / nvg][e % nvg] = cv.v_zero[vi];
      }
      __syncthreads();
    }
    // QK: one thread per token.
    if (tid < nt) {
      const int t = cs + tid;
      float sco[NH];
#pragma unroll
      for (int j = 0; j < NH; ++j) sco[j] = 0.0f;
      const uint4* row = reinterpret_cast<const uint4*>(cv.k_codes + (pair * cv.cap + t) * RB);
      const int gl = KIVI ? tid / G : 0;
#pragma unroll
      for (int vi = 0; vi < RB / 16; ++vi) {
        const uint4 w4 = row[vi];
        const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          constexpr int CPW = 32 / BITS;
#pragma unroll
          for (int k = 0; k < CPW; k += (FMT == KVQ_FMT_FP8_E4M3 ? 2 : 1)) {
            const int ch = (vi * 4 + wi) * CPW + k;
            float x0, x1 = 0.0f;
            if constexpr (KIVI) {
              const uint32_t code = (words[wi] >> (k * BITS)) & ((1u << BITS) - 1u);
              x0 = kivi_value(code, kss[gl][ch], kzs[gl][ch]);
            } else if constexpr (FMT == KVQ_FMT_INT8) {
              x0 = float(int8_t(uint8_t(words[wi] >> (8 * k))));
            } else {
              const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(int(words[wi] >> (8 * k)), false);
              x0 = f[0];
              x1 = f[1];
            }
#pragma unroll
            for (int j = 0; j < NH; ++j) {
              sco[j] = fmaf(qs[j][ch], x0, sco[j]);
              if constexpr (FMT == KVQ_FMT_FP8_E4M3) sco[j] = fmaf(qs[j][ch + 1], x1, sco[j]);
            }
          }
        }
      }
      const float ks = KIVI ? 1.0f : cv.k_scale[pair * cv.cap + t];
#pragma unroll
      for (int j = 0; j < NH; ++j) sc[j][tid] = sco[j] * ks * sm_scale;
    }
    __syncthreads();
    softmax_chunk(nt, cs);
    __syncthreads();
    // PV: thread (channel c, part) walks 8-token blocks part, part+P, ...
#pragma unroll
    for (int j = 0; j < NH; ++j) acc[j] *= st_a[j];
    const int nblk = (nt + 7) / 8;
    for (int blk = part; blk < nblk; blk += P) {
      const size_t tb0 = size_t(cs) + size_t(blk) * 8;
      const uint8_t* wp = cv.v_codes + ((pair * (cv.cap / 8) + tb0 / 8) * D + c) * BITS;
      uint32_t w0, w1 = 0;
      if constexpr (BITS == 8) {
        const uint2 w = *reinterpret_cast<const uint2*>(wp);
        w0 = w.x;
        w1 = w.y;
      } else if constexpr (BITS == 4) {
        w0 = *reinterpret_cast<const uint32_t*>(wp);
      } else {
        w0 = *reinterpret_cast<const uint16_t*>(wp);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = blk * 8 + k;
        if (i < nt) {
          if constexpr (KIVI) {
            const uint32_t code = (w0 >> (k * BITS)) & ((1u << BITS) - 1u);
            const float v = kivi_value(code, vss[i][c / G], vzs[i][c / G]);
#pragma unroll
            for (int j = 0; j < NH; ++j) acc[j] = fmaf(sc[j][i], v, acc[j]);
          } else {
            const uint32_t wd = k < 4 ? w0 : w1;
            float v;
            if constexpr (FMT == KVQ_FMT_INT8) {
              v = float(int8_t(uint8_t(wd >> (8 * (k & 3)))));
            } else {
              const float2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(int(wd >> (8 * (k & 2))), false);
              v = f[k & 1];
            }
#pragma unroll
            for (int j = 0; j < NH; ++j) acc[j] = fmaf(pv[j][i], v, acc[j]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---------------- residual ring (KIVI, last split only) ----------------
  if constexpr (KIVI) {
    if (has_resid) {
      const int C = cv.C;
      for (int cs = nq; cs < n; cs += kChunk) {
        const int nt = min(kChunk, n - cs);
        if (tid < nt) {
          const int t = cs + tid;
          const size_t rbase = (pair * C + (t % C)) * D;
          float sco[NH];
#pragma unroll
          for (int j = 0; j < NH; ++j) sco[j] = 0.0f;
          for (int ch = 0; ch < D; ++ch) {
            const float x = load_elem<BF16>(cv.k_resid, rbase + ch);
#pragma unroll
            for (int j = 0; j < NH; ++j) sco[j] = fmaf(qs[j][ch], x, sco[j]);
          }
#pragma unroll
          for (int j = 0; j < NH; ++j) sc[j][tid] = sco[j] * sm_scale;
        }
        __syncthreads();
        softmax_chunk(nt, cs);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NH; ++j) acc[j] *= st_a[j];
        for (int i = part; i < nt; i += P) {
          const int t = cs + i;
          const float v = load_elem<BF16>(cv.v_resid, (pair * C + (t % C)) * D + c);
#pragma unroll
          for (int j = 0; j < NH; ++j) acc[j] = fmaf(sc[j][i], v, acc[j]);
        }
        __syncthreads();
      }
    }
  }

  // ---------------- combine token parts, write the partial state --------------
  float* red = &sc[0][0];  // P * NH * D <= 8 * kChunk floats
#pragma unroll
  for (int j = 0; j < NH; ++j) red[(part * NH + j) * D + c] = acc[j];
  __syncthreads();
  if (part == 0) {
    for (int j = 0; j < g; ++j) {
      float o = 0.0f;
#pragma unroll
      for (int p = 0; p < P; ++p) o += red[(p * NH + j) * D + c];
      wk.o[((size_t(b) * cv.Hq + size_t(h) * g + j) * wk.S + s) * D + c] = o;
    }
  }
  if (tid < g) {
    const size_t mi = (size_t(b) * cv.Hq + size_t(h) * g + tid) * wk.S + s;
    wk.m[mi] = st_m[tid];
    wk.l[mi] = st_l[tid];
  }
}

// One workgroup (D threads) per (query head, sequence).
template <bool KIVI>
__global__ void decode_merge(CacheView cv, const int32_t* __restrict__ seq_lens, float* __restrict__ out,
                             DecodeWork wk) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  int n = seq_lens[b];
  n = min(max(n, 0), cv.max_tokens);
  const int nq = KIVI ? kivi_quantized(n, cv.G, cv.R) : n;
  const int ns = min(nq / wk.L + 1, wk.S);
  const size_t row = (size_t(b) * cv.Hq + hq) * wk.S;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, wk.m[row + s]);
  float o = 0.0f;
  if (M != -INFINITY) {
    float lsum = 0.0f, acc = 0.0f;
    for (int s = 0; s < ns; ++s) {
      const float w = __expf(wk.m[row + s] - M);
      lsum = fmaf(wk.l[row + s], w, lsum);
      acc = fmaf(wk.o[(row + s) * cv.D + c], w, acc);
    }
    o = acc / lsum;
  }
  out[(size_t(b) * cv.Hq + hq) * cv.D + c] = o;
}

template <int FMT, int BITS, int D, bool BF16>
void launch_split_nh(const CacheView& cv, const int32_t* sl, const void* q, float sm, const DecodeWork& wk,
                     hipStream_t st) {
  const dim3 grid(wk.S, cv.Hkv, cv.B);
  if (cv.g > 4) decode_split<FMT, BITS, D, 8, BF16><<<grid, kThreads, 0, st>>>(cv, sl, q, sm, wk);
  else decode_split<FMT, BITS, D, 4, BF16><<<grid, kThreads, 0, st>>>(cv, sl, q, sm, wk);
}

template <int FMT, int BITS, bool BF16>
void launch_split_d(const CacheView& cv, const int32_t* sl, const void* q, float sm, const DecodeWork& wk,
                    hipStream_t st) {
  if (cv.D == 128) launch_split_nh<FMT, BITS, 128, BF16>(cv, sl, q, sm, wk, st);
  else launch_split_nh<FMT, BITS, 64, BF16>(cv, sl, q, sm, wk, st);
}

template <bool BF16>
void launch_split(const CacheView& cv, const int32_t* sl, const void* q, float sm, const DecodeWork& wk,
                  hipStream_t st) {
  switch (cv.fmt) {
    case KVQ_FMT_FP8_E4M3: launch_split_d<KVQ_FMT_FP8_E4M3, 8, BF16>(cv, sl, q, sm, wk, st); break;
    case KVQ_FMT_INT8: launch_split_d<KVQ_FMT_INT8, 8, BF16>(cv, sl, q, sm, wk, st); break;
    default:
      if (cv.bits == 4) launch_split_d<KVQ_FMT_KIVI, 4, BF16>(cv, sl, q, sm, wk, st);
      else launch_split_d<KVQ_FMT_KIVI, 2, BF16>(cv, sl, q, sm, wk, st);
  }
}

}  // namespace

hipError_t launch_decode(const CacheView& cv, const int32_t* seq_lens, const void* q, float sm_scale, float* out,
                         const DecodeWork& work, hipStream_t stream) {
  if (cv.bf16) launch_split<true>(cv, seq_lens, q, sm_scale, work, stream);
  else launch_split<false>(cv, seq_lens, q, sm_scale, work, stream);
  const dim3 mgrid(cv.Hq, cv.B);
  if (cv.fmt == KVQ_FMT_KIVI) decode_merge<true><<<mgrid, cv.D, 0, stream>>>(cv, seq_lens, out, work);
  else decode_merge<false><<<mgrid, cv.D, 0, stream>>>(cv, seq_lens, out, work);
  return hipGetLastError();
}

}  // namespace kvq
