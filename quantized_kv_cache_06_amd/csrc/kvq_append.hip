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

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 32;  // tokens per workgroup in the per-token kernel

// Length checks shared by the append kernels: a sequence whose append would
// be malformed or overflow the capacity is left unchanged.
__device__ __forceinline__ bool append_range(const CacheView& cv, const int32_t* seq_lens,
                                             const int32_t* append_lens, int T, int b, int* n, int* tb) {
  *n = seq_lens[b];
  *tb = append_lens ? append_lens[b] : T;
  return *n >= 0 && *tb >= 0 && *tb <= T && int64_t(*n) + *tb <= cv.max_tokens;
}

// ---------------------------------------------------------------------------
// Per-token FP8 E4M3 / INT8 (and the unquantized BF16 cache): one wave per
// token row, D/64 channels per lane.
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
#pragma unroll
      for (int j = 0; j < CPL; ++j) x[j] = load_elem<BF16>(src, in_base + j);
      float s;
      const uint32_t codes = quantize_token_lane<FMT, CPL>(x, &s);
      store_token_codes<FMT, CPL>(cv, pair, t, which != 0, lane, codes, s);
    }
  }
}

// ---------------------------------------------------------------------------
// Group-wise symmetric INT4: one wave per 8-token Value block. The wave
// quantizes the block's new tokens one row at a time (Key and Value),
// stores the Key nibbles and the scales as it goes, and collects the Value
// nibbles of its lanes' channels; it then rewrites each channel's block word
// once, keeping the nibbles of tokens it does not own. Each block word has
// one writer per call, so the read-modify-write is race-free.
// ---------------------------------------------------------------------------
template <int D, int G, bool BF16, bool ROT>
__global__ __launch_bounds__(kThreads) void append_int4(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                       const void* __restrict__ kin, const void* __restrict__ vin,
                                                       int T, const int32_t* __restrict__ append_lens) {
  constexpr int CPL = D / kWave;
  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  if (tb == 0) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const size_t pair = pair_index(cv, b, h);
  const int blk = n / 8 + int(blockIdx.x) * (kThreads / kWave) + wave;
  const int t_lo = max(n, 8 * blk), t_hi = min(n + tb, 8 * blk + 8);
  if (t_lo >= t_hi) return;
  uint32_t vw[CPL], vm[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) vw[j] = vm[j] = 0u;
  for (int t = t_lo; t < t_hi; ++t) {
    const size_t in_base = (pair * T + (t - n)) * D + lane * CPL;
    float xk[CPL], xv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      xk[j] = load_elem<BF16>(kin, in_base + j);
      xv[j] = load_elem<BF16>(vin, in_base + j);
    }
    if constexpr (ROT) fwht_wave<CPL>(xk);  // Keys are stored rotated
    float sk, sv;
    const uint32_t uk = quantize_token_int4<G, CPL>(xk, &sk);
    const uint32_t uv = quantize_token_int4<G, CPL>(xv, &sv);
    store_int4_key<G, CPL>(cv, pair, t, lane, uk, sk);
    if (lane % (G / CPL) == 0) cv.v_scale[(pair * cv.cap + t) * (D / G) + (lane * CPL) / G] = sv;
    const int sh = 4 * (t % 8);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      vw[j] |= ((uv >> (4 * j)) & 0xFu) << sh;
      vm[j] |= 0xFu << sh;
    }
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    uint32_t* w = int4_value_word<D>(cv, pair, t_lo, lane * CPL + j);
    *w = (*w & ~vm[j]) | vw[j];
  }
}

// ---------------------------------------------------------------------------
// KIVI group flush: one workgroup per (group slot, kv head, sequence). The
// steps (staging, Key half, Value half) are shared with the fused append +
// decode kernel.
// ---------------------------------------------------------------------------
template <int BITS, int G, int D, bool BF16, bool M16>
__global__ __launch_bounds__(kThreads) void kivi_flush(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                      const void* __restrict__ kin, const void* __restrict__ vin,
                                                      int T, const int32_t* __restrict__ append_lens) {
  static_assert(kThreads == kQuantThreads, "flush steps assume this workgroup size");
  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int q0 = kivi_quantized(n, G, cv.R);
  const int q1 = kivi_quantized(n + tb, G, cv.R);
  const int grp = q0 / G + int(blockIdx.x);
  if ((grp + 1) * G > q1) return;

  __shared__ FlushSmem<G, D> f;
  const size_t pair = pair_index(cv, b, h);
  flush_stage<BF16, G, D>(f, cv, pair, grp, n, kin, T, cv.k_resid);
  flush_key<BITS, G, D, M16>(f, cv, pair, grp);
  flush_stage<BF16, G, D>(f, cv, pair, grp, n, vin, T, cv.v_resid);
  flush_value<BITS, G, D, M16>(f, cv, pair, grp);
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
                                                         const int32_t* __restrict__ append_lens,
                                                         int32_t* __restrict__ skipped) {
  const int b = blockIdx.x;
  int n, tb;
  const bool ok = append_range(cv, seq_lens, append_lens, T, b, &n, &tb);
  if (skipped != nullptr && threadIdx.x == 0) skipped[b] = ok ? 0 : 1;
  if (!ok) return;
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

template <int D, int G, bool BF16, bool ROT>
void launch_int4(const CacheView& cv, int32_t* seq_lens, const void* k, const void* v, int T, const int32_t* al,
                 hipStream_t st) {
  // blocks touched by T tokens starting anywhere: at most T / 8 + 2
  const int nblk = T / 8 + 2;
  const dim3 grid((nblk + kThreads / kWave - 1) / (kThreads / kWave), cv.Hkv, cv.B);
  append_int4<D, G, BF16, ROT><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
}

template <bool BF16, bool ROT>
void int4_dg(const CacheView& cv, int32_t* sl, const void* k, const void* v, int T, const int32_t* al,
             hipStream_t st) {
  if (cv.D == 128) {
    if (cv.G == 32) launch_int4<128, 32, BF16, ROT>(cv, sl, k, v, T, al, st);
    else if (cv.G == 64) launch_int4<128, 64, BF16, ROT>(cv, sl, k, v, T, al, st);
    else launch_int4<128, 128, BF16, ROT>(cv, sl, k, v, T, al, st);
  } else {
    if (cv.G == 32) launch_int4<64, 32, BF16, ROT>(cv, sl, k, v, T, al, st);
    else launch_int4<64, 64, BF16, ROT>(cv, sl, k, v, T, al, st);
  }
}

template <int BITS, int G, int D, bool BF16>
void launch_flush(const CacheView& cv, int32_t* seq_lens, const void* k, const void* v, int T,
                  const int32_t* al, hipStream_t st) {
  const dim3 grid(T / G + 1, cv.Hkv, cv.B);
  if (cv.fmt == KVQ_FMT_KIVI_F16)
    kivi_flush<BITS, G, D, BF16, true><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
  else
    kivi_flush<BITS, G, D, BF16, false><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
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
                         const int32_t* append_lens, int32_t* skipped, hipStream_t stream) {
  if (cv.fmt == KVQ_FMT_KIVI || cv.fmt == KVQ_FMT_KIVI_F16) {
    if (cv.bits == 4) {
      if (cv.bf16) flush_gd<4, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else flush_gd<4, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else {
      if (cv.bf16) flush_gd<2, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else flush_gd<2, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    }
    append_finish<true><<<cv.B, kThreads, 0, stream>>>(cv, seq_lens, k_new, v_new, T, append_lens, skipped);
  } else {
    if (cv.fmt == KVQ_FMT_FP8_E4M3) {
      if (cv.bf16) per_token_d<KVQ_FMT_FP8_E4M3, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_FP8_E4M3, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else if (cv.fmt == KVQ_FMT_FP8_STATIC) {
      if (cv.bf16) per_token_d<KVQ_FMT_FP8_STATIC, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_FP8_STATIC, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else if (cv.fmt == KVQ_FMT_INT4) {
      if (cv.bf16) int4_dg<true, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else int4_dg<false, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else if (cv.fmt == KVQ_FMT_INT4_HADAMARD) {
      if (cv.bf16) int4_dg<true, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else int4_dg<false, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else if (cv.fmt == KVQ_FMT_BF16) {
      if (cv.bf16) per_token_d<KVQ_FMT_BF16, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_BF16, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    } else {
      if (cv.bf16) per_token_d<KVQ_FMT_INT8, true>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
      else per_token_d<KVQ_FMT_INT8, false>(cv, seq_lens, k_new, v_new, T, append_lens, stream);
    }
    append_finish<false><<<cv.B, kThreads, 0, stream>>>(cv, seq_lens, k_new, v_new, T, append_lens, skipped);
  }
  return hipGetLastError();
}

}  // namespace kvq
