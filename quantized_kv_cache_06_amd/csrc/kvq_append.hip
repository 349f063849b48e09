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
// for bit. An append is a few launches on the caller's stream: the first
// quantizes (per-token formats) or flushes whole groups (KIVI); for KIVI a
// second writes the tokens that stay in the residual ring; the last
// advances seq_lens. Stream order makes every read of old ring slots and of
// seq_lens happen before they are overwritten.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kvq_quant.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
// Tuning knobs of the per-token tile append (compile-time; the defaults are
// the measured best on MI355X): the cache policy of its input loads (2:
// non-temporal, each input byte is read once) and whether both tensors'
// rows are requested before either is quantized.
#ifndef KVQ_APPEND_LOAD_AUX
#define KVQ_APPEND_LOAD_AUX 2
#endif
#ifndef KVQ_APPEND_PRELOAD
#define KVQ_APPEND_PRELOAD 1
#endif
// Workgroups per compute unit the register allocation of the KIVI flush
// (d = 128, bf16 inputs) must allow.
#ifndef KVQ_FLUSH_WG_PER_CU
#define KVQ_FLUSH_WG_PER_CU 3
#endif

// Length checks shared by the append kernels: a sequence whose append would
// be malformed or overflow the capacity is left unchanged.
__device__ __forceinline__ bool append_range(const CacheView& cv, const int32_t* seq_lens,
                                             const int32_t* append_lens, int T, int b, int* n, int* tb) {
  *n = seq_lens[b];
  *tb = append_lens ? append_lens[b] : T;
  return *n >= 0 && *tb >= 0 && *tb <= T && int64_t(*n) + *tb <= cv.max_tokens;
}

// ---------------------------------------------------------------------------
// Per-token FP8 E4M3 / INT8 / static FP8 and the unquantized BF16 cache:
// one wave per tile of whole 8-token Value blocks, aligned to absolute token
// positions (TPW = 32 tokens at d = 128, 64 at d = 64). Lane l takes block
// i = l / LPR of the tile and channels [8 g, 8 g + 8), g = l % LPR, LPR =
// d / 8: load j (j = 0..7) fetches token 8 i + j of every block, so each
// input row is read by LPR consecutive lanes in 16-byte pieces, and each
// lane ends up holding an 8 x 8 (token, channel) tile of its block:
//  - the row maximum is a DPP maximum over the LPR lanes of the row;
//  - Key rows are stored as 8-byte (bf16: 16-byte) pieces of each row;
//  - Value words (one per channel, the block's 8 tokens) come from a byte
//    transpose in registers; lanes g and g ^ 2 then swap half of their
//    words so that each writes 64 contiguous bytes of the permuted slots.
// A block that already holds tokens below the sequence length (an append
// that starts inside a block) keeps their bytes with a read-modify-write of
// its words; each word has one writer per call. Positions past the new
// length are written with codes of zero rows; no reader looks at them.
// ---------------------------------------------------------------------------
template <int FMT, int D, bool BF16>
__global__ __launch_bounds__(kThreads, 3) void append_tiles(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                        const void* __restrict__ kin, const void* __restrict__ vin,
                                                        int T, const int32_t* __restrict__ append_lens) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 8;              // lanes per token row
  constexpr int TPW = 8 * (kWave / LPR);  // tokens per wave tile
  constexpr bool CACHE16 = FMT == KVQ_FMT_BF16;
  constexpr bool SCALED = FMT == KVQ_FMT_FP8_E4M3 || FMT == KVQ_FMT_INT8;
  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  if (tb == 0) return;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int tile = n / TPW + int(blockIdx.x) * (kThreads / kWave) + wave;
  if (tile * TPW >= n + tb) return;  // wave-uniform
  const int i = lane / LPR, g = lane % LPR;
  const int tblk = tile * TPW + 8 * i;               // first token of the lane's block
  const int v_lo = max(n - tblk, 0);                 // tokens [v_lo, v_hi) of the block are new
  const int v_hi = min(n + tb - tblk, 8);
  const bool any = v_lo < v_hi;                      // uniform over the LPR lanes of the block
  const size_t pair = pair_index(cv, b, h);
  const size_t in_row0 = pair * size_t(T);           // the pair's first input row

  uint32_t kcode[8][CACHE16 ? 4 : 2];  // [token][dword]: the lane's 8 channels of each token
  uint32_t vcode[8][CACHE16 ? 4 : 2];
  float kscale[8], vscale[8];
  // bf16 inputs: both tensors' rows are loaded before either is quantized,
  // so the Value loads are in flight while the Keys are computed. The loads
  // go through buffer resources over the tile's new input rows: a row
  // outside them (before the old length or past the new one) lies outside
  // the resource, reads as zero and fetches nothing, so every load is
  // issued unconditionally and the waits stay exact.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t raw[2][8];
  if constexpr (BF16) {
    const int r0 = max(tile * TPW, n);                       // the tile's first new token
    const int nrows = min((tile + 1) * TPW, n + tb) - r0;    // its new tokens (>= 1)
    const uint32_t rbytes = uint32_t(nrows) * D * 2;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const uint16_t* base = static_cast<const uint16_t*>(which ? vin : kin) + (in_row0 + size_t(r0 - n)) * D;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, int(rbytes), 0x00020000);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // a row before r0 gets an offset at the top of the 32-bit range
        // (never a wrapped negative one); a row past the new length lies
        // past the resource's end
        const int rel = tblk + j - r0;
        const uint32_t off = rel < 0 ? 0xfffffff0u : uint32_t(rel) * uint32_t(D * 2) + uint32_t(16 * g);
        raw[which][j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, KVQ_APPEND_LOAD_AUX);
      }
      if constexpr (KVQ_APPEND_PRELOAD == 0) {
        if (which == 0) asm volatile("" ::: "memory");
      }
    }
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void* src = which ? vin : kin;
    uint32_t (&code)[8][CACHE16 ? 4 : 2] = which ? vcode : kcode;
    float (&scale)[8] = which ? vscale : kscale;
    float x[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool live = j >= v_lo && j < v_hi;
      const size_t row = in_row0 + size_t(tblk + j - n);
      if constexpr (BF16) {
        (void)live;
        (void)row;
        const uint32_t a[4] = {raw[which][j][0], raw[which][j][1], raw[which][j][2], raw[which][j][3]};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[j][2 * k] = bf16_lo(a[k]);
          x[j][2 * k + 1] = bf16_hi(a[k]);
        }
        if constexpr (CACHE16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) code[j][k] = a[k];  // bf16 inputs are stored as they are
        }
      } else {
        float4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
        if (live) {
          const float* r = static_cast<const float*>(src) + row * D + 8 * g;
          p0 = *reinterpret_cast<const float4*>(r);
          p1 = *reinterpret_cast<const float4*>(r + 4);
        }
        x[j][0] = p0.x; x[j][1] = p0.y; x[j][2] = p0.z; x[j][3] = p0.w;
        x[j][4] = p1.x; x[j][5] = p1.y; x[j][6] = p1.z; x[j][7] = p1.w;
        if constexpr (CACHE16) {
#pragma unroll
          for (int k = 0; k < 4; ++k) code[j][k] = bf16_pair_rne(x[j][2 * k], x[j][2 * k + 1]);
        }
      }
    }
    if constexpr (!CACHE16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float sc = 1.0f;
        if constexpr (SCALED) {
          float a = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[j][e]));
          a = run_absmax<LPR>(a);
          // a / 448 (or / 127)
          constexpr float kDen = FMT == KVQ_FMT_FP8_E4M3 ? 448.0f : 127.0f;
          sc = quot_nonneg(a, kDen, recip_refined(kDen));
        }
        scale[j] = sc;
        // divide by a positive stand-in where the scale is 0 and select the 0
        // code afterwards: no branch around each division. The quotient is
        // the refined-reciprocal one when every scale of the wave is in
        // range (a wave-uniform test), else a true division.
        const bool pos = sc > 0.0f;
        const float den = pos ? sc : 1.0f;
        const bool fast = __all(in_div_range(den));
        const float rden = recip_refined(den);
        // FP8 keeps the quotient's sign (E4M3 has a signed zero); an INT8 code
        // of a tiny quotient is 0 whatever its sign
        constexpr bool SIGNED = FMT == KVQ_FMT_FP8_E4M3;
        auto quot = [&](float xv) { return fast ? div_refined<SIGNED>(xv, den, rden) : xv / den; };
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float xv = x[j][4 * k + e];
            if constexpr (FMT == KVQ_FMT_FP8_STATIC) {
              y[e] = fminf(fmaxf(xv, -448.0f), 448.0f);
            } else if constexpr (FMT == KVQ_FMT_FP8_E4M3) {
              const float q = __builtin_amdgcn_fmed3f(quot(xv), -448.0f, 448.0f);
              y[e] = pos ? q : 0.0f;
            } else {
              // a zero scale means a zero row: its quotients are zeros, code 0
              y[e] = __builtin_amdgcn_fmed3f(rintf(quot(xv)), -127.0f, 127.0f);
            }
          }
          uint32_t w;
          if constexpr (FMT == KVQ_FMT_INT8) {
            w = (uint32_t(int32_t(y[0])) & 0xffu) | ((uint32_t(int32_t(y[1])) & 0xffu) << 8) |
                ((uint32_t(int32_t(y[2])) & 0xffu) << 16) | (uint32_t(int32_t(y[3])) << 24);
          } else {
            // OCP E4M3, round to nearest even; inputs are already within +-448
            w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false));
            w = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], int(w), true));
          }
          code[j][k] = w;
        }
      }
    }
  }
  if (!any) return;  // nothing of this lane's block is appended (after every DPP step)

  // ---- Key rows and per-token scales ----
  constexpr int RB = CACHE16 ? 2 * D : D;  // bytes per Key row
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < v_lo || j >= v_hi) continue;
    uint8_t* dst = cv.k_codes + (pair * cv.cap + size_t(tblk + j)) * RB + (CACHE16 ? 16 : 8) * g;
    if constexpr (CACHE16)
      *reinterpret_cast<uint4*>(dst) = make_uint4(kcode[j][0], kcode[j][1], kcode[j][2], kcode[j][3]);
    else *reinterpret_cast<uint2*>(dst) = make_uint2(kcode[j][0], kcode[j][1]);
  }
  if constexpr (SCALED) {
    // lane g < 8 of the block stores token g's scales (picked without an
    // indexed register access)
    if (g < 8 && g >= v_lo && g < v_hi) {
      float ks = kscale[0], vs = vscale[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) {
        ks = g == j ? kscale[j] : ks;
        vs = g == j ? vscale[j] : vs;
      }
      cv.k_scale[pair * cv.cap + size_t(tblk + g)] = ks;
      cv.v_scale[pair * cv.cap + size_t(tblk + g)] = vs;
    }
  }

  // ---- Value words: one per channel, the block's 8 tokens ----
  const size_t blk = size_t(tblk / 8);
  if constexpr (CACHE16) {
    // word of channel 8 g + e: 16 bytes, token pair p in dword p; no slot
    // permutation (one word per 16-byte load)
    uint4* dst = reinterpret_cast<uint4*>(cv.v_codes + (pair * (cv.cap / 8) + blk) * (size_t(D) * 16)) + 8 * g;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t w[4];
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low half of each token's dword
#pragma unroll
      for (int p = 0; p < 4; ++p) w[p] = __builtin_amdgcn_perm(vcode[2 * p + 1][e >> 1], vcode[2 * p][e >> 1], sel);
      if (v_lo > 0) {
        // keep the halves of tokens below the old length
        const uint4 old = dst[e];
        const uint32_t o[4] = {old.x, old.y, old.z, old.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t keep = (2 * p < v_lo ? 0x0000ffffu : 0u) | (2 * p + 1 < v_lo ? 0xffff0000u : 0u);
          w[p] = (o[p] & keep) | (w[p] & ~keep);
        }
      }
      dst[e] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    // word of channel 8 g + e: token j in byte j (tokens 0-3 in the low
    // dword); lo[e], hi[e]
    uint32_t lo[8], hi[8];
    {
      uint32_t a[4], t[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {      // channels 4 half .. 4 half + 3
#pragma unroll
        for (int q = 0; q < 2; ++q) {             // tokens 4 q .. 4 q + 3
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = vcode[4 * q + r][half];
          transpose4x4_bytes(a, t);
#pragma unroll
          for (int e = 0; e < 4; ++e) (q ? hi : lo)[4 * half + e] = t[e];
        }
      }
    }
    // Slots: channel 8 g + e lies in slot 2 e + odd of the lane's run of 16
    // slots (odd = bit 1 of g; the run starts at slot 32 (g / 4) + 16 (g & 1)).
    // The even lane writes slots [0, 8) of the run (its words e < 4 and the
    // partner's), the odd lane slots [8, 16) (words e >= 4).
    const bool odd = (g & 2) != 0;
    uint32_t mine[8], theirs[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // send the words the partner writes: the even lane its e >= 4, the odd lane its e < 4
      const uint32_t slo = odd ? lo[k] : lo[4 + k];
      const uint32_t shi = odd ? hi[k] : hi[4 + k];
      theirs[2 * k] = quad_swap2(slo);
      theirs[2 * k + 1] = quad_swap2(shi);
      mine[2 * k] = odd ? lo[4 + k] : lo[k];
      mine[2 * k + 1] = odd ? hi[4 + k] : hi[k];
    }
    const int run = 32 * (g / 4) + 16 * (g & 1) + (odd ? 8 : 0);
    uint4* dst = reinterpret_cast<uint4*>(cv.v_codes + (pair * (cv.cap / 8) + blk) * (size_t(D) * 8) + size_t(run) * 8);
    // 16-byte piece k: slots 2k, 2k + 1 of the half-run = (even word, odd word) of channel e = k (+4)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t w[4];
      if (odd) {
        w[0] = theirs[2 * k]; w[1] = theirs[2 * k + 1]; w[2] = mine[2 * k]; w[3] = mine[2 * k + 1];
      } else {
        w[0] = mine[2 * k]; w[1] = mine[2 * k + 1]; w[2] = theirs[2 * k]; w[3] = theirs[2 * k + 1];
      }
      if (v_lo > 0) {
        // keep the bytes of tokens below the old length (bytes 0..v_lo-1 of each word)
        const uint4 old = dst[k];
        const uint32_t o[4] = {old.x, old.y, old.z, old.w};
        const uint32_t klo = v_lo >= 4 ? 0xffffffffu : (1u << (8 * v_lo)) - 1u;
        const uint32_t khi = v_lo <= 4 ? 0u : (1u << (8 * (v_lo - 4))) - 1u;
        const uint32_t keep[4] = {klo, khi, klo, khi};
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (o[q] & keep[q]) | (w[q] & ~keep[q]);
      }
      dst[k] = make_uint4(w[0], w[1], w[2], w[3]);
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
// KIVI group flush for head_dim 128 and bf16 inputs (the benchmark shapes):
// two waves per 64 flushed tokens (one group of 64, or two of 32), the even
// wave of a pair of waves the Keys, the odd one the Values, no LDS and no
// barrier. Lane l takes quarter q = l / 16 of the tokens (16 consecutive
// rows, whole Value blocks) and channels [8 g, 8 g + 8), g = l % 16: load j
// fetches row 16 q + j of every quarter in 16-byte pieces, from the residual
// ring (tokens below the old length) or the new input. A wave holds one
// tensor's rows, so it issues all its loads at once.
//  - Key: per-channel minimum and maximum over the lane's 16 rows, combined
//    across the quarters of the group with lane exchanges;
//  - Value: per-token, per-channel-group minimum and maximum over the
//    G / 8 lanes of the group within the row, by DPP steps;
//  - codes from the refined-reciprocal quotient (div_refined) where every
//    scale of the wave is in_div_range (else true divisions), packed in
//    registers into Key row pieces and whole Value words.
// The arithmetic of each code, scale and zero-point is that of flush_key /
// flush_value (and of the oracle): fp32, true quotients, round half to even.
// ---------------------------------------------------------------------------
template <int BITS, int G, bool M16>
__global__ __launch_bounds__(kThreads, KVQ_FLUSH_WG_PER_CU) void kivi_flush_waves(
    CacheView cv, const int32_t* __restrict__ seq_lens, const void* __restrict__ kin, const void* __restrict__ vin,
    int T, const int32_t* __restrict__ append_lens) {
#pragma clang fp contract(off)
  constexpr int D = 128;
  constexpr float QMAX = float((1 << BITS) - 1);
  constexpr int NVG = D / G;   // Value channel groups per token
  constexpr int LPG = G / 8;   // lanes of one Value channel group within a row
  constexpr int QPG = G / 16;  // quarters (16-row lane groups) of one Key group
  constexpr int TB = BITS == 2 ? 16 : 8;  // tokens per Value word
  const int b = blockIdx.z, h = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int q0 = kivi_quantized(n, G, cv.R);
  const int q1 = kivi_quantized(n + tb, G, cv.R);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const bool values = (wave & 1) != 0;  // the tensor this wave flushes (wave-uniform)
  const int T0 = q0 + 64 * (int(blockIdx.x) * (kThreads / kWave / 2) + wave / 2);
  if (T0 >= q1) return;  // wave-uniform
  const int q = lane / 16, g = lane % 16;
  const int tq = T0 + 16 * q;                              // the lane's first token
  const int gstart = T0 + 16 * (q - q % QPG);             // first token of the lane's Key group
  const bool ok = gstart + G <= q1;                        // the group is flushed by this call
  const size_t pair = pair_index(cv, b, h);
  const int C = cv.C;

  // ---- loads: 16 rows of Key (then Value), 8 channels each ----
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  auto load_rows = [&](const uint8_t* ring, const void* in, u32x4_t (&r)[16]) {
    if (T0 >= n) {
      // every row is new input: one scalar base for the wave, and the
      // lane's rows at fixed 256-byte steps from its offset
      const uint8_t* base = static_cast<const uint8_t*>(in) + (pair * T + size_t(T0 - n)) * (D * 2);
      const uint32_t lo = uint32_t(16 * q * D * 2 + 16 * g);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        r[j] = u32x4_t{0u, 0u, 0u, 0u};
        if (ok) r[j] = *reinterpret_cast<const u32x4_t*>(base + lo + j * (D * 2));
      }
    } else {
      // the first flushed tokens of a call: rows from the residual ring
      // (tokens below the old length) and from the input
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int t = tq + j;
        const uint16_t* p = t < n ? reinterpret_cast<const uint16_t*>(ring) + (pair * C + size_t(t % C)) * D + 8 * g
                                  : static_cast<const uint16_t*>(in) + (pair * T + size_t(t - n)) * D + 8 * g;
        r[j] = u32x4_t{0u, 0u, 0u, 0u};
        if (ok) r[j] = *reinterpret_cast<const u32x4_t*>(p);
      }
    }
  };
  auto elem = [](const u32x4_t& w, int e) { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); };
  // clamp(rint(q), 0, qmax) for a finite q, carried in the low bits of the
  // pattern of q' + 1.5 * 2^23 with q' = med3(q, -0.49, qmax + 0.49): the
  // addition rounds q' to the nearest integer, ties to even (the same as
  // rint, and q' only moves q within the interval that rounds to the same
  // clamped code), and leaves it in the mantissa above kRoundBits. Codes are
  // packed by adding such patterns shifted into place; the sum of the
  // shifted kRoundBits is taken off once per word (pack_offset).
  constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
  constexpr uint32_t kRoundBits = 0x4B400000u;
  auto code_bits = [](float qv) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(qv, -0.49f, QMAX + 0.49f) + kRound);
  };
  auto pack_offset = [](int count) {
    uint32_t o = 0;
    for (int i = 0; i < count; ++i) o += kRoundBits << (BITS * i);
    return o;
  };
  // A zero scale (a degenerate group) has code 0. With fp32 metadata it
  // means max == min, so every difference x - z is 0 and its quotient by the
  // stand-in divisor 1 is already 0; a binary16 zero-point need not equal
  // the minimum, so there the code is selected.
  auto degen = [](float s_, uint32_t c) { return (!M16 || s_ > 0.0f) ? c : kRoundBits; };
  constexpr int KRB = D * BITS / 8;  // Key row bytes
  if (!values) {
    u32x4_t kr[16];
    load_rows(cv.k_resid, kin, kr);

    // ---- Key: per-channel statistics over the group ----
    float ks[8], kz[8];
    {
      float kmn[8], kmx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kmn[e] = INFINITY;
        kmx[e] = -INFINITY;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = elem(kr[j], e);
          kmn[e] = fminf(kmn[e], x);
          kmx[e] = fmaxf(kmx[e], x);
        }
#pragma unroll
      for (int o = 16; o < 16 * QPG; o <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kmn[e] = fminf(kmn[e], __shfl_xor(kmn[e], o, kWave));
          kmx[e] = fmaxf(kmx[e], __shfl_xor(kmx[e], o, kWave));
        }
      const float rq = recip_refined(QMAX);
      // the rows are widened again for the codes rather than held widened
      // through the statistics (128 registers)
#pragma unroll
      for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(kr[j]));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ks[e] = stored_meta<M16>(quot_nonneg(kmx[e] - kmn[e], QMAX, rq) + 0.0f);
        kz[e] = stored_meta<M16>(kmn[e] + 0.0f);
      }
    }
    if (ok && q % QPG == 0) {
      const size_t si = (pair * (cv.cap / G) + size_t(gstart / G)) * D + 8 * g;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        store_meta<M16>(cv.k_scale, si + e, ks[e]);
        store_meta<M16>(cv.k_zero, si + e, kz[e]);
      }
    }

    // ---- Key codes and stores ----
    {
      // divisor stand-in 1 for a degenerate channel (s == 0), whose code is 0
      float kdv[8], ky[8];
      bool fast = true;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kdv[e] = ks[e] > 0.0f ? ks[e] : 1.0f;
        fast = fast && in_div_range(kdv[e]);
        ky[e] = recip_refined(kdv[e]);
      }
      fast = __all(fast);  // wave-uniform
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t w = 0;
        if (fast) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            w += degen(ks[e], code_bits(div_refined<false>(elem(kr[j], e) - kz[e], kdv[e], ky[e]))) << (BITS * e);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            w += degen(ks[e], code_bits((elem(kr[j], e) - kz[e]) / kdv[e])) << (BITS * e);
        }
        w -= pack_offset(8);
        if (ok) {
          uint8_t* row = cv.k_codes + (pair * cv.cap + size_t(tq + j)) * KRB;
          if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(row + 4 * g) = w;
          else *reinterpret_cast<uint16_t*>(row + 2 * g) = uint16_t(w);
        }
      }
    }
    return;
  }

  // ---- Value: per-token statistics over each channel group, codes ----
  u32x4_t vr[16];
  load_rows(cv.v_resid, vin, vr);
  uint32_t vword[16 / TB][8];  // [block][channel]
#pragma unroll
  for (int k = 0; k < 16 / TB; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) vword[k][e] = 0u;
  float vsc[16], vzr[16], vdv[16];
  bool vfast = true;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float mn = elem(vr[j], 0), mx = mn;
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      mn = fminf(mn, elem(vr[j], e));
      mx = fmaxf(mx, elem(vr[j], e));
    }
    uint32_t kmin = float_key(mn), kmax = float_key(mx);
    run_minmax_keys<LPG>(kmin, kmax);
    mn = key_float(kmin);
    mx = key_float(kmax);
    vsc[j] = stored_meta<M16>(quot_nonneg(mx - mn, QMAX, recip_refined(QMAX)) + 0.0f);
    vzr[j] = stored_meta<M16>(mn + 0.0f);
    vdv[j] = vsc[j] > 0.0f ? vsc[j] : 1.0f;
    vfast = vfast && in_div_range(vdv[j]);
    if (ok && g % LPG == 0) {
      const size_t vi = (pair * cv.cap + size_t(tq + j)) * NVG + g / LPG;
      store_meta<M16>(cv.v_scale, vi, vsc[j]);
      store_meta<M16>(cv.v_zero, vi, vzr[j]);
    }
  }
  // the rows are widened again for the codes (as for the Keys)
#pragma unroll
  for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(vr[j]));
  if (__all(vfast)) {  // wave-uniform
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float vy = recip_refined(vdv[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vword[j / TB][e] +=
            degen(vsc[j], code_bits(div_refined<false>(elem(vr[j], e) - vzr[j], vdv[j], vy))) << (BITS * (j % TB));
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vword[j / TB][e] += degen(vsc[j], code_bits((elem(vr[j], e) - vzr[j]) / vdv[j])) << (BITS * (j % TB));
  }
#pragma unroll
  for (int k = 0; k < 16 / TB; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) vword[k][e] -= pack_offset(TB);
  if (!ok) return;

  uint32_t* vblocks = reinterpret_cast<uint32_t*>(cv.v_codes);
#pragma unroll
  for (int k = 0; k < 16 / TB; ++k) {
    const size_t blk = size_t((tq + k * TB) / TB);
#pragma unroll
    for (int e = 0; e < 8; ++e) vblocks[(pair * (cv.cap / TB) + blk) * D + value_slot<4>(8 * g + e)] = vword[k][e];
  }
}

// ---------------------------------------------------------------------------
// KIVI, second launch: one workgroup per (kv head, sequence) copies the new
// tokens that stay in the residual window into their ring slots (bit copy,
// 16-byte vectors, four in flight per thread). It runs after the flush
// launch, whose reads of old ring slots it may overwrite.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void ring_copy(CacheView cv, const int32_t* __restrict__ seq_lens,
                                                     const void* __restrict__ kin, const void* __restrict__ vin,
                                                     int T, const int32_t* __restrict__ append_lens) {
  const int h = blockIdx.x, b = blockIdx.y;
  int n, tb;
  if (!append_range(cv, seq_lens, append_lens, T, b, &n, &tb)) return;
  const int n1 = n + tb;
  const int start = max(n, kivi_quantized(n1, cv.G, cv.R));
  const int row_bytes = cv.D * (cv.bf16 ? 2 : 4);
  const int vpr = row_bytes / 16;              // 16-byte vectors per row
  const int total = (n1 - start) * vpr;
  const size_t pair = pair_index(cv, b, h);
  constexpr int U = 4;
  for (int e0 = int(threadIdx.x); e0 < total; e0 += U * kThreads) {
    uint4 kx[U], vx[U];
    size_t dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = min(e0 + u * kThreads, total - 1);  // a clamped index re-copies the last vector
      const int t = start + e / vpr, v = e % vpr;
      const size_t src = (pair * T + size_t(t - n)) * row_bytes + size_t(v) * 16;
      dst[u] = (pair * cv.C + size_t(t % cv.C)) * row_bytes + size_t(v) * 16;
      kx[u] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(kin) + src);
      vx[u] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(vin) + src);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      *reinterpret_cast<uint4*>(cv.k_resid + dst[u]) = kx[u];
      *reinterpret_cast<uint4*>(cv.v_resid + dst[u]) = vx[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Last launch: one thread per sequence advances seq_lens[b] (every earlier
// launch of the append has read it) and reports a skipped sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void append_finish(CacheView cv, int32_t* __restrict__ seq_lens, int T,
                                                   const int32_t* __restrict__ append_lens,
                                                   int32_t* __restrict__ skipped) {
  const int b = int(blockIdx.x) * 64 + int(threadIdx.x);
  if (b >= cv.B) return;
  int n, tb;
  const bool ok = append_range(cv, seq_lens, append_lens, T, b, &n, &tb);
  if (skipped != nullptr) skipped[b] = ok ? 0 : 1;
  if (ok) seq_lens[b] = n + tb;
}

template <int FMT, int D, bool BF16>
void launch_per_token(const CacheView& cv, int32_t* seq_lens, const void* k, const void* v, int T,
                      const int32_t* al, hipStream_t st) {
  // tiles touched by T tokens starting anywhere: at most T / TPW + 2
  constexpr int TPW = 8 * (kWave / (D / 8));
  const int ntile = T / TPW + 2;
  const dim3 grid((ntile + kThreads / kWave - 1) / (kThreads / kWave), cv.Hkv, cv.B);
  append_tiles<FMT, D, BF16><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
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
  if constexpr (D == 128 && BF16) {
    // two waves per 64 flushed tokens: at most T + G flushed tokens per pair
    const int chunks = (T + G + 63) / 64;
    constexpr int kChunksPerWg = kThreads / kWave / 2;
    const dim3 grid((chunks + kChunksPerWg - 1) / kChunksPerWg, cv.Hkv, cv.B);
    if (cv.fmt == KVQ_FMT_KIVI_F16)
      kivi_flush_waves<BITS, G, true><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
    else
      kivi_flush_waves<BITS, G, false><<<grid, kThreads, 0, st>>>(cv, seq_lens, k, v, T, al);
    return;
  }
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
    ring_copy<<<dim3(cv.Hkv, cv.B), kThreads, 0, stream>>>(cv, seq_lens, k_new, v_new, T, append_lens);
    append_finish<<<(cv.B + 63) / 64, 64, 0, stream>>>(cv, seq_lens, T, append_lens, skipped);
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
    append_finish<<<(cv.B + 63) / 64, 64, 0, stream>>>(cv, seq_lens, T, append_lens, skipped);
  }
  return hipGetLastError();
}

}  // namespace kvq
