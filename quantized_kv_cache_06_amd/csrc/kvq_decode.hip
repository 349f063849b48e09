// Decode attention over the quantized cache (gfx950): split-K partials on
// the matrix cores and the cross-split merge.
//
// Operation: one query token per sequence attends to every cached token
// while the codes are dequantized on the fly — "KV cache quantization"
// (guide.dupenodi.dev) "Key takeaways": the attention kernel must read the
// quantized cache; "How KV cache quantization reduces GPU memory" (n4n.ai)
// "Step 5": a separate dequantize pass gives the bandwidth savings away;
// "KV Cache Quantization in Production LLM Serving" (llms.blog) "Serving
// Economics": decode is bound by memory bandwidth.
//
// How the work maps onto CDNA4
// ----------------------------
// One workgroup (4 waves) per work item, a split of one (kv head,
// sequence) pair (see decode_item); the waves take the split's 32-token
// tiles (whole groups for KIVI) in turn, each keeping its own online
// softmax state, and are merged through LDS at the end. Per tile:
//
//  scores (QK): S^T[32 tokens x 16 cols] = K[32 x d] * Qt[d x 16] with
//    v_mfma_f32_16x16x32_bf16 (KIVI: _f16). Column c = 8 * term + head:
//    every query head of the GQA group (up to 8) appears twice, as the
//    "hi" part of its query and as the "lo" remainder, so the products keep
//    about 16 (bf16) or 22 (f16) significant bits of the fp32 query; the two
//    columns are added with one DPP row rotation. Codes enter the matrix
//    core exactly: E4M3 and INT8 codes convert to bf16 exactly; group-wise
//    INT4 nibbles (code + 8) become the bf16 128 + nibble by OR-ing them
//    under the bf16 pattern of 128 (136 * sum(q) comes off per channel
//    group); KIVI 4-bit codes are masked one per byte, where a byte
//    holding c <= 15 is the E4M3 pattern of c * 2^-9, and the scaled FP8
//    conversion (scale 2^9) turns two such bytes into the f16 pair c
//    exactly; KIVI 2-bit codes are masked one per nibble, the E2M1 pattern
//    of c / 2, and the scaled FP4 conversion (scale 2) turns a byte into
//    the f16 pair of its two codes. Per-token scales multiply the finished
//    scores; KIVI per-channel Key scales are folded into the query once per
//    group (score = sum_c (q_c s_c) code_c + sum_c q_c z_c).
//  softmax: running maximum and sum per head in the log2 domain (exp2).
//  values (PV): O^T[d x 16] += V^T[d x 32] * P^T[32 x 16], again with the
//    probabilities (times the per-token Value scale) split into bf16 hi and
//    lo columns. Value codes enter as the bf16 128 + c * 2^k (masked in
//    place under the bf16 pattern of 128; INT2 k = 0, 2 or 4 with 2^-k taken
//    into the staged Value scale); a second product with the constant -128
//    takes 128 * p' off in the same accumulator. The KIVI per-token
//    zero-points add sum_t p_t z_t per channel group on the vector ALU.
// The cache layout (include/kvq.h) is chosen so that every lane loads its
// operand bytes with 16-byte loads and no shuffles: Key rows token-major,
// Value words per channel in blocks of 8 (16 for INT2) tokens, channel words
// permuted so 16 consecutive lanes read 16 consecutive channels.
//
// KIVI residual tokens (full precision, fewer than R + G per sequence) are
// handled by one extra workgroup per (kv head, sequence) on the vector ALU,
// writing the last partial slot. The workgroup of a (sequence, kv head) that
// finishes last (an arrival counter in the workspace) combines every partial
// by the log-sum-exp rule and writes the normalized output: one launch per
// call.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "kvq_quant.h"
#include "kvq_wave.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTile = 32;        // tokens per wave iteration (two 16-token score tiles)
constexpr int kResidChunk = 64;   // KIVI residual tokens per chunk (one per lane in its softmax)
constexpr float kLazyLog2 = 8.0f;  // headroom of the lazy softmax rescale (log2 units)
constexpr int kMaxSplits = kMaxDecodeSplits;  // quantized splits per sequence (S - 1 <= this)
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kMagic128 = 0x43004300u;  // two bf16 128.0
// Tuning knobs (compile-time; the defaults are the measured best on MI355X):
// non-temporal loads for the streamed cache codes and for the per-token
// scales and zero-points (each byte is read once per call; KIVI's Key group
// parameters, re-read by every tile of a group, stay temporal), the 64-byte
// Key pieces of 8-bit codes at d = 128, and the prefetch ring depth.
#ifndef KVQ_DECODE_NT
#define KVQ_DECODE_NT 1
#endif
#ifndef KVQ_DECODE_NT_META
#define KVQ_DECODE_NT_META 0
#endif
#ifndef KVQ_DECODE_KSPLIT
#define KVQ_DECODE_KSPLIT 1
#endif
#ifndef KVQ_DECODE_INTERLEAVE
#define KVQ_DECODE_INTERLEAVE 1
#endif
#ifndef KVQ_DECODE_NPF
#define KVQ_DECODE_NPF 2
#endif
// Workgroups per compute unit the register allocation must allow (0 = the
// per-kernel default of min_wg_per_cu below).
#ifndef KVQ_DECODE_MIN_WG_PER_CU
#define KVQ_DECODE_MIN_WG_PER_CU 0
#endif
constexpr bool kStreamNT = KVQ_DECODE_NT != 0;
constexpr bool kMetaNT = KVQ_DECODE_NT_META != 0;
constexpr int kCodeAux = kStreamNT ? 2 : 0;  // cache policy of the code loads (2: non-temporal)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Two floats to an f16 pair, round to nearest even (x0 in the low half).
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {
  const f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[0]); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return float(__builtin_bit_cast(f16x2_t, w)[1]); }

// (x & m) | c in one instruction (a three-input bitwise op; its truth table
// is f(0xF0, 0xCC, 0xAA) = (0xF0 & 0xCC) | 0xAA).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(x, m, c, 0xEA);
}

// m ? a : b for a lane mask m (all ones or all zeros) as one bitwise op.
// Unlike a plain conditional between two elements of a register array, it
// cannot be rewritten into an array access with a lane-dependent index
// (which would move the array to scratch memory, whose loads wait behind
// every outstanding global load).
__device__ __forceinline__ float select_bits(uint32_t m, float a, float b) {
  return __builtin_bit_cast(float, __builtin_amdgcn_bitop3_b32(__builtin_bit_cast(uint32_t, a),
                                                               __builtin_bit_cast(uint32_t, b), m, 0xE4));
}

// -1.0 in a register the compiler cannot see through, so that x - f16 below
// stays a multiply-add with an f16 operand (one v_fma_mix instruction)
// instead of a convert and a subtract.
__device__ __forceinline__ float opaque_minus_one() {
  float v;
  asm volatile("v_mov_b32 %0, 0xbf800000" : "=v"(v));
  return v;
}
// f16 pair (x0 - hi.lo, x1 - hi.hi), each difference exact in fp32 and
// rounded once to f16: the lo term of the hi/lo split of (x0, x1) whose hi
// term is hi = pack_f16(x0, x1). m1 = opaque_minus_one().
__device__ __forceinline__ uint32_t f16_residual(uint32_t hi, float x0, float x1, float m1) {
  const f16x2_t h = __builtin_bit_cast(f16x2_t, hi);
  return pack_f16(__builtin_fmaf(float(h[0]), m1, x0), __builtin_fmaf(float(h[1]), m1, x1));
}

// Two floats to a bf16 pair, round to nearest even (x0 in the low half).
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  const f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// hi = bf16(x), lo = bf16(x - hi) for a pair of floats.
struct Split2 {
  uint32_t hi, lo;
};
__device__ __forceinline__ Split2 split_pair(float x0, float x1) {
  Split2 s;
  s.hi = pack_bf16(x0, x1);
  s.lo = pack_bf16(x0 - bf_lo(s.hi), x1 - bf_hi(s.hi));
  return s;
}
// The same split with each residual x - hi (exact) taken as one bf16 dot
// product (sub_bf16_half): two instructions fewer where both terms are
// kept. u = bf16_units().
__device__ __forceinline__ Split2 split_pair_dot(float x0, float x1, const Bf16Units& u) {
  Split2 s;
  s.hi = pack_bf16(x0, x1);
  s.lo = pack_bf16(sub_bf16_half(s.hi, u.lo, x0), sub_bf16_half(s.hi, u.hi, x1));
  return s;
}

// Signed INT8 byte pair to a bf16 pair, exact.
template <int SEL>
__device__ __forceinline__ uint32_t i8x2_bf16(uint32_t w) {
  return pack_bf16(float(int8_t(uint8_t(w >> (16 * SEL)))), float(int8_t(uint8_t(w >> (16 * SEL + 8)))));
}
// Byte pair SEL of w (8-bit formats) to a bf16 pair, exact.
template <int FMT, int SEL>
__device__ __forceinline__ uint32_t byte_pair_bf16(uint32_t w) {
  if constexpr (FMT == KVQ_FMT_FP8_E4M3 || FMT == KVQ_FMT_FP8_STATIC) return fp8x2_bf16<SEL>(w);
  else return i8x2_bf16<SEL>(w);
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (unrolled).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

// ---------------------------------------------------------------------------
// Index maps shared by the loads and the operands (see the file header).
//
// Channel of element i of k-step kk held by row group r in the score MFMA:
// lanes of row group r hold the contiguous channels [CPL*r, CPL*(r+1)), CPL =
// D/4, and element i of k-step kk is the following one of them.
// KIVI (KBYTE set) takes its Key codes in the order the conversions of
// key_operand produce them; group-wise INT4 pairs nibble j with nibble
// j + 4.
template <int BITS, bool KBYTE = false>
__device__ __forceinline__ constexpr int cperm(int kk, int i) {
  if constexpr (BITS >= 8) return 8 * kk + i;
  else if constexpr (BITS == 4 && KBYTE) return 8 * kk + 2 * (i & 3) + (i >> 2);
  else if constexpr (BITS == 2 && KBYTE)
    return 16 * (kk >> 1) + 8 * (kk & 1) + 4 * (i >> 2) + ((i >> 1) & 1) + 2 * (i & 1);
  else if constexpr (BITS == 4) return 8 * kk + (i >> 1) + 4 * (i & 1);
  else return 16 * (kk >> 1) + 4 * (kk & 1) + (i >> 1) + 8 * (i & 1);
}
// Token (within a 32-token tile) of score tile t, row 4r + j. The same
// token is element j (t = 0) / 4 + j (t = 1) of row group r in the value
// MFMA's K dimension, up to the per-format pairing of the operand halves.
template <int BITS>
__device__ __forceinline__ constexpr int tok(int t, int r, int j) {
  if constexpr (BITS == 2) return 16 * (r >> 1) + 8 * t + 4 * (r & 1) + j;
  else return 8 * r + 4 * t + j;
}

// Loads of NB bytes (4, 8, 16 or 32) into dwords. NT marks the load
// non-temporal (streamed once: the cache codes of a decode call).
template <typename V, bool NT>
__device__ __forceinline__ V load_vec(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}
template <int NB, bool NT = false>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* w) {
  if constexpr (NB == 32) {
    const u32x4 a = load_vec<u32x4, NT>(p);
    const u32x4 b = load_vec<u32x4, NT>(p + 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
  } else if constexpr (NB == 16) {
    const u32x4 a = load_vec<u32x4, NT>(p);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else if constexpr (NB == 8) {
    const u32x2 a = load_vec<u32x2, NT>(p);
    w[0] = a[0]; w[1] = a[1];
  } else {
    w[0] = load_vec<uint32_t, NT>(p);
  }
}

// N consecutive input elements (bf16 or fp32) starting at element i, as
// fp32, with 8/16-byte vector loads (i is a multiple of N).
template <bool BF16, int N>
__device__ __forceinline__ void load_elems(const void* p, size_t i, float* x) {
  if constexpr (BF16) {
    const uint16_t* s = static_cast<const uint16_t*>(p) + i;
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int v = 0; v < N / 8; ++v) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(s + 8 * v);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x[8 * v + 2 * k] = bf_lo(w[k]);
          x[8 * v + 2 * k + 1] = bf_hi(w[k]);
        }
      }
    } else if constexpr (N == 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(s);
      x[0] = bf_lo(w);
      x[1] = bf_hi(w);
    } else {
      static_assert(N % 4 == 0, "bf16 groups of 4");
#pragma unroll
      for (int v = 0; v < N / 4; ++v) {
        const u32x2 w = *reinterpret_cast<const u32x2*>(s + 4 * v);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          x[4 * v + 2 * k] = bf_lo(w[k]);
          x[4 * v + 2 * k + 1] = bf_hi(w[k]);
        }
      }
    }
  } else {
    const float* s = static_cast<const float*>(p) + i;
    static_assert(N % 2 == 0, "fp32 pairs");
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int v = 0; v < N / 4; ++v) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(s + 4 * v);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[4 * v + k] = w[k];
      }
    } else {
#pragma unroll
      for (int v = 0; v < N / 2; ++v) {
        const f32x2 w = *reinterpret_cast<const f32x2*>(s + 2 * v);
        x[2 * v] = w[0];
        x[2 * v + 1] = w[1];
      }
    }
  }
}

// Key operand (16 tokens x 32 channels) of k-step kk from the lane's raw
// Key bytes. 8-bit codes: bf16, exact. KIVI codes: f16, each element exactly
// the code: INT4 codes are masked one nibble per byte and two bytes at a
// time go through the scaled E4M3 conversion (e4m3_pair_f16); INT2 codes
// are masked two per byte, one per nibble (fields 0 and 2, then 1 and 3),
// and one byte at a time goes through the scaled E2M1 conversion
// (e2m1_pair_f16). The f16 results are normal numbers or zero, which the
// matrix cores multiply exactly.

template <int FMT, int BITS>
__device__ __forceinline__ u32x4 key_operand(const uint32_t* kw, int kk) {
  u32x4 a;
  if constexpr (FMT == KVQ_FMT_INT4 || FMT == KVQ_FMT_INT4_HADAMARD) {
    // group-wise INT4: chunk word kk holds the k-step's 8 nibbles (code + 8);
    // pair j = (nibble j, nibble j + 4) as bf16 128 + nibble, exact
    const uint32_t w = kw[kk];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = and_or(w >> (4 * j), 0x000F000Fu, kMagic128);
  } else if constexpr (BITS == 16) {
    // bf16 rows: 16-byte piece kk holds the k-step's 8 channels as they are
    a[0] = kw[4 * kk];
    a[1] = kw[4 * kk + 1];
    a[2] = kw[4 * kk + 2];
    a[3] = kw[4 * kk + 3];
  } else if constexpr (BITS == 8) {
    a[0] = byte_pair_bf16<FMT, 0>(kw[2 * kk]);
    a[1] = byte_pair_bf16<FMT, 1>(kw[2 * kk]);
    a[2] = byte_pair_bf16<FMT, 0>(kw[2 * kk + 1]);
    a[3] = byte_pair_bf16<FMT, 1>(kw[2 * kk + 1]);
  } else if constexpr (BITS == 4) {
    // even nibbles one per byte, then the odd ones: pairs (0, 2), (4, 6),
    // (1, 3), (5, 7) of the k-step's 8
    const uint32_t w = kw[kk], ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    a[0] = e4m3_pair_f16<0>(ev);
    a[1] = e4m3_pair_f16<1>(ev);
    a[2] = e4m3_pair_f16<0>(od);
    a[3] = e4m3_pair_f16<1>(od);
  } else {
    // word kk/2 holds 16 codes, 4 per byte (field f at bits 2f): m0 keeps
    // fields 0 and 2 of every byte, m1 fields 1 and 3, one per nibble; byte
    // b of each gives the pairs (field 0, 2) and (1, 3) of byte b, from
    // bytes 0-1 (even kk) or 2-3 (odd kk)
    const uint32_t w = kw[kk >> 1], m0 = w & 0x33333333u, m1 = (w >> 2) & 0x33333333u;
    if (kk & 1) {
      a[0] = e2m1_pair_f16<2>(m0); a[1] = e2m1_pair_f16<2>(m1);
      a[2] = e2m1_pair_f16<3>(m0); a[3] = e2m1_pair_f16<3>(m1);
    } else {
      a[0] = e2m1_pair_f16<0>(m0); a[1] = e2m1_pair_f16<0>(m1);
      a[2] = e2m1_pair_f16<1>(m0); a[3] = e2m1_pair_f16<1>(m1);
    }
  }
  return a;
}

// Value operand (16 channels x 32 tokens as bf16) of channel tile mt from
// the lane's raw Value words (row group r).
template <int FMT, int BITS>
__device__ __forceinline__ u32x4 value_operand(const uint32_t* vw, int mt, int r) {
  u32x4 a;
  if constexpr (BITS == 16) {
    // bf16: 16-byte load mt holds channel tile mt's 8 tokens as they are
    a[0] = vw[4 * mt];
    a[1] = vw[4 * mt + 1];
    a[2] = vw[4 * mt + 2];
    a[3] = vw[4 * mt + 3];
  } else if constexpr (BITS == 8) {
    // 16-byte load p holds the 8-byte words of channel tiles 2p, 2p+1
    const uint32_t* w = vw + 4 * (mt >> 1) + 2 * (mt & 1);
    a[0] = byte_pair_bf16<FMT, 0>(w[0]);
    a[1] = byte_pair_bf16<FMT, 1>(w[0]);
    a[2] = byte_pair_bf16<FMT, 0>(w[1]);
    a[3] = byte_pair_bf16<FMT, 1>(w[1]);
  } else if constexpr (BITS == 4) {
    const uint32_t w = vw[mt];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = and_or(w >> (4 * j), 0x000F000Fu, kMagic128);
  } else {
    // fields 0-2 of the lane's byte in place (x1, x4, x16), field 3 shifted
    // down (x1); the Value scales of the tokens of pairs 1 and 2 are staged
    // times 1/4 and 1/16
    const uint32_t x = vw[mt] >> (8 * (r & 1));
    a[0] = and_or(x, 0x00030003u, kMagic128);
    a[1] = and_or(x, 0x000C000Cu, kMagic128);
    a[2] = and_or(x, 0x00300030u, kMagic128);
    a[3] = and_or(x >> 6, 0x00030003u, kMagic128);
  }
  return a;
}

// Probability operand (32 tokens x 16 columns) from p[t][j] (token tok(t,
// r, j)): the element order matches value_operand's token order. Each lane
// splits every value into bf16 hi + lo and keeps the term of its column.
template <int BITS>
__device__ __forceinline__ u32x4 prob_operand(const float (&p)[2][4], bool lo) {
  u32x4 b;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float x0, x1;
    if constexpr (BITS >= 8) {
      x0 = p[k >> 1][2 * (k & 1)];
      x1 = p[k >> 1][2 * (k & 1) + 1];
    } else {
      x0 = p[0][k];
      x1 = p[1][k];
    }
    const Split2 s = split_pair(x0, x1);
    b[k] = lo ? s.lo : s.hi;
  }
  return b;
}

// Zeroes the halves of a bf16 operand whose token index is >= valid, for the
// last, partial tile of a per-token format (8-bit order: element e is token
// 8r + e of the tile).
__device__ __forceinline__ u32x4 mask_tokens8(u32x4 a, int r, int valid) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 8 * r + 2 * k;
    const uint32_t keep = (e < valid ? 0x0000ffffu : 0u) | (e + 1 < valid ? 0xffff0000u : 0u);
    a[k] &= keep;
  }
  return a;
}

// LDS of one workgroup: the quantized-split path and the residual path use
// it differently; the larger of the two sizes it.
template <int D>
struct SmemQuant {
  float q[8][D];              // query of the GQA group (KIVI)
  // each wave's unnormalized output, maximum and sum; piece kWaves is the
  // new token of a fused step of a per-token format
  float o[kWaves + 1][8][D];
  float m[kWaves + 1][8];
  float l[kWaves + 1][8];
  float xn[2][D];             // the new token's dequantized Key and Value rows
  // per-wave staging of a tile's metadata: per-token scales (8-bit
  // formats: [K | V][32 tokens]); KIVI: Value [scale | zero][32 * D/32]
  // and Key group [scale | zero][D]
  float meta[kWaves][2][32 * (D / 32)];
  float kgrp[kWaves][2][D];
};
template <int D>
struct SmemResid {
  float q[8][D];
  float sc[8][kResidChunk];   // scores, then probabilities
  float st_m[8], st_l[8], st_a[8];
};
// The KIVI residual path of the fused append + decode step also flushes a
// completed group (staged in LDS) before attending over it.
template <int D, int G>
struct SmemResidFused : SmemResid<D> {
  FlushSmem<G, D> f;
};
template <int D, int G, bool FUSED>
using SmemResidT = std::conditional_t<FUSED && (G > 0), SmemResidFused<D, (G > 0 ? G : 32)>, SmemResid<D>>;
template <int D, int G, bool FUSED>
constexpr size_t smem_floats() {
  return (sizeof(SmemQuant<D>) > sizeof(SmemResidT<D, G, FUSED>) ? sizeof(SmemQuant<D>)
                                                                   : sizeof(SmemResidT<D, G, FUSED>)) /
         sizeof(float);
}

// Row of one partial state (unnormalized output, log2-domain maximum and
// sum) of query head j of kv head h in split slot s.
__device__ __forceinline__ size_t partial_row(const CacheView& cv, const DecodeWork& wk, int b, int h, int j,
                                              int s) {
  return (size_t(b) * cv.Hq + size_t(h) * cv.g + j) * wk.S + s;
}

// Partial states cross workgroups (and XCDs) inside one launch: they are
// written and read as relaxed device-scope atomics, which the compiler emits
// as plain coherent (sc1) stores and loads with no cache write-back.
__device__ __forceinline__ void put_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_partial(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resource over n bytes at p (raw addressing, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, int(n), 0x00020000);
}
// NB bytes (4, 8, 16 or 32) from buffer r at vector offset vo plus scalar
// offset so. Bytes outside the buffer's range read as 0 and are not fetched.
template <int NB, int AUX>
__device__ __forceinline__ void buffer_bytes(__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so, uint32_t* w) {
  if constexpr (NB == 32) {
    buffer_bytes<16, AUX>(r, vo, so, w);
    buffer_bytes<16, AUX>(r, vo + 16, so, w + 4);
  } else if constexpr (NB == 16) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, AUX);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  } else if constexpr (NB == 8) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, AUX);
    w[0] = a[0]; w[1] = a[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, vo, so, AUX);
  }
}
// 16-byte partial loads and stores with the same device-scope coherence as
// put_partial / get_partial (cache policy sc1).
constexpr int kCoherent = 16;
__device__ __forceinline__ f32x4 get_partial4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent);
}
__device__ __forceinline__ void put_partial4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kCoherent);
}

// x, as a value the compiler cannot relate to earlier expressions of x
// (emits no instruction). Used after the main loop so that addresses the
// epilogue shares with the prologue are recomputed instead of being held in
// registers across the loop.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Fused append + decode, per-token formats (FP8, INT8, INT4, static FP8,
// rotated INT4, bf16): the sequence's new token t (its length
// before the call) is quantized by the append's own steps (wave 0 the Key
// row, wave 1 the Value row) and stored at position t; it enters attention
// as one more piece of the workgroup's wave merge: maximum = its score, sum
// = 1, output = its dequantized Value row. Every load (the two new rows and
// the query) is issued before the first barrier. Workgroup-collective.
template <int FMT, int D, int G, bool BF16>
__device__ __forceinline__ void new_token_piece(const CacheView& cv, int b, int h, int t, const AppendIn& ap,
                                                const void* __restrict__ q, float sm_log2, SmemQuant<D>& sm) {
  constexpr int CPL = D / kWave;
  constexpr int CPT = D / 32;  // channels per thread in the dot products (32 threads per head)
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = cv.g;
  const size_t pair = pair_index(cv, b, h);
  constexpr bool INT4G = FMT == KVQ_FMT_INT4 || FMT == KVQ_FMT_INT4_HADAMARD;
  constexpr bool ROT = FMT == KVQ_FMT_INT4_HADAMARD;
  const int j = tid / 32, part = tid % 32;
  float qx[CPT];
  if constexpr (ROT) {
    // the rotated query q' = H q / d that the workgroup staged in LDS
#pragma unroll
    for (int k = 0; k < CPT; ++k) qx[k] = sm.q[j][part * CPT + k];
  } else {
    load_elems<BF16, CPT>(q, (size_t(b) * cv.Hq + size_t(h) * g + min(j, g - 1)) * D + part * CPT, qx);
  }
  if (wave < 2) {
    float x[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) x[e] = load_elem<BF16>(wave ? ap.v : ap.k, pair * D + lane * CPL + e);
    if constexpr (ROT) {
      if (wave == 0) fwht_wave<CPL>(x);  // Keys are stored rotated (wave-uniform branch)
    }
    float sc;
    uint32_t codes;
    if constexpr (INT4G) {
      codes = quantize_token_int4<G, CPL>(x, &sc);
      if (wave == 0) {
        store_int4_key<G, CPL>(cv, pair, t, lane, codes, sc);
      } else {
        if (lane % (G / CPL) == 0) cv.v_scale[(pair * cv.cap + t) * (D / G) + (lane * CPL) / G] = sc;
        // this workgroup is the only writer of the sequence's block words
        const int sh = 4 * (t % 8);
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
          uint32_t* w = int4_value_word<D>(cv, pair, t, lane * CPL + e);
          *w = (*w & ~(0xFu << sh)) | (((codes >> (4 * e)) & 0xFu) << sh);
        }
      }
    } else {
      codes = quantize_token_lane<FMT, CPL>(x, &sc);
      store_token_codes<FMT, CPL>(cv, pair, t, wave == 1, lane, codes, sc);
    }
    float c[2];  // the codes as values, exactly
    if constexpr (INT4G) {
      c[0] = float(int(codes & 0xFu) - 8);
      c[1] = float(int((codes >> 4) & 0xFu) - 8);
    } else if constexpr (FMT == KVQ_FMT_BF16) {
      c[0] = bf_lo(codes);
      c[1] = bf_hi(codes);
    } else if constexpr (FMT == KVQ_FMT_FP8_E4M3 || FMT == KVQ_FMT_FP8_STATIC) {
      const uint32_t w = fp8x2_bf16<0>(codes);
      c[0] = bf_lo(w);
      c[1] = bf_hi(w);
    } else {
      c[0] = float(int8_t(uint8_t(codes)));
      c[1] = float(int8_t(uint8_t(codes >> 8)));
    }
#pragma unroll
    for (int e = 0; e < CPL; ++e) sm.xn[wave][lane * CPL + e] = c[e] * sc;
  }
  __syncthreads();
  float dot = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) dot = fmaf(qx[k], sm.xn[0][part * CPT + k], dot);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) dot += __shfl_xor(dot, o, kWave);
#pragma unroll
  for (int k = 0; k < CPT; ++k) sm.o[kWaves][j][part * CPT + k] = sm.xn[1][part * CPT + k];
  if (part == 0) {
    sm.m[kWaves][j] = j < g ? dot * sm_log2 : -INFINITY;
    sm.l[kWaves][j] = 1.0f;
  }
}

// Element j of binary16 values packed two per 32-bit register, widened
// exactly.
template <int N>
__device__ __forceinline__ float half_at(const uint32_t (&w)[N], int j) {
  const uint32_t bits = w[j / 2];
  return float(__builtin_bit_cast(_Float16, uint16_t((j & 1) ? bits >> 16 : bits)));
}

// ---------------------------------------------------------------------------
// Quantized tokens [t0, t1) of one split: 4 waves on the matrix cores.
// Every global load of a tile (codes, scales, zero-points, and the Key
// group parameters when the tile opens a group) is issued one tile ahead in
// a single batch, so a wave always has the next tile in flight while it
// computes the current one; metadata is re-laid out through the wave's own
// LDS area.
// ---------------------------------------------------------------------------
// With FUSED and t_new >= 0 (the per-token formats), the fused step's new token t_new
// joins the wave merge as a fifth piece (new_token_piece).
template <int FMT, int BITS, int D, int G, bool BF16, bool FUSED>
__device__ __forceinline__ void split_quantized(const CacheView& cv, int b, int h, int s, int t0, int t1,
                                                const void* __restrict__ q, float sm_log2, const DecodeWork& wk,
                                                SmemQuant<D>& sm, int t_new, const AppendIn& ap) {
  constexpr bool KIVI = FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16;
  // KIVI with binary16 metadata: the raw halves ride in the ring (two per
  // register) and are widened when the tile is processed
  constexpr bool M16 = FMT == KVQ_FMT_KIVI_F16;
  constexpr bool KBYTE = KIVI;  // Key codes in the byte-wise conversion's order
  constexpr int CPL = D / 4;                  // channels per row group (score MFMA)
  // 8-bit codes at d = 128: row group r holds channels [16r, 16r+16) and
  // [64+16r, 64+16r+16), so each Key load instruction covers 64 contiguous
  // bytes of every row it touches (elements 8kk + i of the lane's 32 keep
  // their order: k-steps 0-1 take the first piece, 2-3 the second)
  constexpr bool KSPLIT = KVQ_DECODE_KSPLIT != 0 && BITS == 8 && D == 128;
  constexpr int NKK = D / 32;                 // k-steps of the score MFMA
  constexpr int NMT = D / 16;                 // channel tiles of the value MFMA
  constexpr int KB = D * BITS / 8;            // bytes per Key row
  constexpr int LKB = CPL * BITS / 8;         // Key bytes per lane per token
  constexpr int VWB = BITS == 16 ? 16 : BITS == 8 ? 8 : 4;  // bytes per Value word (one channel, one block)
  // per-token scales (FP8/INT8), KIVI metadata or INT4 group scales; none for
  // the bf16 cache and the static-scale FP8
  constexpr bool SCALED = FMT != KVQ_FMT_BF16 && FMT != KVQ_FMT_FP8_STATIC;
  // group-wise INT4: per-token scales of each channel group for Key and Value
  // (ROT: the Keys are stored Walsh-Hadamard rotated, the query is rotated
  // here the same way)
  constexpr bool INT4G = FMT == KVQ_FMT_INT4 || FMT == KVQ_FMT_INT4_HADAMARD;
  constexpr bool ROT = FMT == KVQ_FMT_INT4_HADAMARD;
  // KIVI and group-wise INT4: each lane takes the softmax of half of its
  // column's scores (see the scores below)
  constexpr bool HALF = KIVI || INT4G;
  constexpr int TB = BITS == 2 ? 16 : 8;      // tokens per Value block
  constexpr int VW = 16 / VWB;                // Value words per 16-byte load
  constexpr int NVL = D / (16 * VW);          // 16-byte Value loads per lane per tile
  constexpr int NVG = KIVI || INT4G ? D / (G > 0 ? G : 1) : 1;  // Value channel groups
  constexpr int MPG = KIVI || INT4G ? G / 16 : NMT;    // channel tiles per Value channel group
  constexpr int KPG = INT4G ? G / 32 : 1;     // INT4: score k-steps per channel group
  constexpr int KGL = D / 32;                 // Key group floats per lane (lanes 0-31 scale, 32-63 zero)
  constexpr int NPF = (KIVI && G == 32 && KVQ_DECODE_NPF > 2) ? 2 : KVQ_DECODE_NPF;  // ring slots (register budget)
  static_assert(KGL == 2 || KGL == 4, "group load width");

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: tile indices stay scalar
  const int m = lane & 15, r = lane >> 4;
  const int hh = m & 7;            // head within the GQA group for this column
  const bool lo_col = m >= 8;      // column holds the lo term
  const int g = cv.g;
  const size_t pair = pair_index(cv, b, h);

  // ---- this wave's tiles (whole KIVI groups) ----
  const int ntile = (t1 - t0 + kTile - 1) / kTile;
  constexpr int GG = KIVI ? G : kTile;         // group size (KIVI), else a harmless divisor
  constexpr int TPG = GG / kTile;
  // Work units of TPG tiles (one KIVI group, else one tile). With
  // KVQ_DECODE_INTERLEAVE the 4 waves take units round-robin (the workgroup
  // sweeps one contiguous region); otherwise each wave takes a contiguous
  // quarter. tile_of(k) is the k-th tile (0 <= k < nk) of this wave.
  const int nunit = (ntile + TPG - 1) / TPG;
  int nk, ua;
  if constexpr (KVQ_DECODE_INTERLEAVE != 0) {
    nk = wave < nunit ? (nunit - wave + kWaves - 1) / kWaves * TPG : 0;
    ua = wave;
  } else {
    const int upw = (nunit + kWaves - 1) / kWaves;
    ua = min(wave * upw, nunit);
    nk = (min(ua + upw, nunit) - ua) * TPG;
  }
  nk = min(nk, ntile - ua * TPG);  // a partial last unit (per-token formats have TPG = 1)
  auto tile_of = [&](int k) {
    if constexpr (KVQ_DECODE_INTERLEAVE != 0) return (ua + kWaves * (k / TPG)) * TPG + k % TPG;
    else return ua * TPG + k;
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4 o[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // KIVI: per channel group, sum_t p_t z_t (the zero-points). The Value
  // codes enter the matrix core as 128 + code, and a second product with
  // the constant -(128 + kCenter) leaves code * p' (group-wise INT4: the
  // codes are stored as code + 8, and the centre 8 takes that off too)
  constexpr float kCenter = INT4G ? 8.0f : 0.0f;
  const uint32_t cpair = pack_bf16(-(128.0f + kCenter), -(128.0f + kCenter));
  const u32x4 kCenterA = {cpair, cpair, cpair, cpair};
  float zb[NVG];
#pragma unroll
  for (int j = 0; j < NVG; ++j) zb[j] = 0.0f;
  float kbias = 0.0f, kscale = 1.0f;  // KIVI: score = (acc * kscale + kbias), log2 domain
  int kes = 0;                        // KIVI: exponent that scaled the open group's Key scales

  // Code loads: a scalar base that advances with the tile plus a per-lane
  // byte offset fixed for the split, so no per-lane address arithmetic is
  // done per tile.
  const uint8_t* kpair = cv.k_codes + pair * size_t(cv.cap) * KB;
  const uint8_t* vpair = cv.v_codes + pair * size_t(cv.cap / TB) * D * VWB;
  uint32_t koff[2];
  // bf16 rows: the lane's k-step kk is the 16-byte piece at 64 kk + 16 r, so
  // each load instruction covers 64 contiguous bytes of every row it touches
#pragma unroll
  for (int t = 0; t < 2; ++t)
    koff[t] = uint32_t(tok<BITS>(t, m >> 2, m & 3) * KB + (KSPLIT || BITS == 16 ? 16 * r : LKB * r));
  const uint32_t voff = uint32_t((size_t(BITS == 2 ? (r >> 1) : r) * D + VW * m) * VWB);
  // the pair's code regions as buffers; a tile past the wave's run loads
  // through an empty buffer (reads 0, fetches nothing), so the loads in
  // flight stay the same on every path without re-reading bytes
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(kpair, uint32_t(size_t(cv.cap) * KB));
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(vpair, uint32_t(size_t(cv.cap / TB) * D * VWB));
  const __amdgpu_buffer_rsrc_t none = buffer_rsrc(kpair, 0u);
  float* meta0 = sm.meta[wave][0];
  float* meta1 = sm.meta[wave][1];

  // Prefetch ring of NPF tile slots (codes, tile metadata, Key group
  // parameters). Slot u holds the wave's tiles u, u + NPF, ...; a slot is refilled with the
  // tile NPF ahead as soon as its tile is consumed, so NPF - 1 tiles are in
  // flight while one is computed. Slot indices are compile-time (the loop
  // over a round of NPF tiles is unrolled), so the ring lives in registers.
  struct Slot {
    uint32_t kw[2][LKB / 4], vw[NVL * 4];
    float mw[NVG], gw[KGL];
    // binary16 metadata (M16): raw halves, two per register
    uint32_t mh[(NVG + 1) / 2], gh[KGL / 2];
  };
  Slot ring[NPF];
  // Loads are issued unconditionally (a tile index past the wave's run is
  // clamped to its last tile, whose bytes are then re-read from cache) so
  // that the number of loads in flight does not depend on the path taken and
  // the waits before each slot's use stay exact.
  // uc: the ring slot (compile time). With NPF a multiple of TPG a slot
  // only ever holds the same tile of its group, so only the slots of a
  // group's first tile load the Key group parameters.
  auto load_tile = [&](Slot& sl, int ti, auto uc) {
    constexpr int U = decltype(uc)::value;
    constexpr bool kGroupLoad = NPF % TPG != 0 || U % TPG == 0;
    const int T0 = __builtin_amdgcn_readfirstlane(t0 + tile_of(min(ti, nk - 1)) * kTile);
    const bool live = ti < nk;  // uniform
    const __amdgpu_buffer_rsrc_t kr = live ? krs : none;
    const __amdgpu_buffer_rsrc_t vr = live ? vrs : none;
    const uint32_t ks = uint32_t(T0) * KB;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if constexpr (BITS == 16) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) buffer_bytes<16, kCodeAux>(kr, koff[t] + 64 * kk, ks, sl.kw[t] + 4 * kk);
      } else if constexpr (KSPLIT) {
        buffer_bytes<16, kCodeAux>(kr, koff[t], ks, sl.kw[t]);
        buffer_bytes<16, kCodeAux>(kr, koff[t] + 64, ks, sl.kw[t] + 4);
      } else {
        buffer_bytes<LKB, kCodeAux>(kr, koff[t], ks, sl.kw[t]);
      }
    }
    const uint32_t vs = uint32_t(T0 / TB) * D * VWB;
#pragma unroll
    for (int p = 0; p < NVL; ++p) buffer_bytes<16, kCodeAux>(vr, voff + uint32_t(p * 16 * VW * VWB), vs, sl.vw + 4 * p);
    // metadata: lanes 0-31 the Key (or Value scale) half, lanes 32-63 the
    // Value (or Value zero) half, NVG floats per lane
    const int part = lane >> 5, qi = lane & 31;
    if constexpr (!SCALED) {
      (void)part;
      (void)qi;
    } else if constexpr (INT4G) {
      const float* src = (part ? cv.v_scale : cv.k_scale) + (pair * cv.cap + T0 + qi) * NVG;
      if constexpr (NVG == 4) {
        const f32x4 x = load_vec<f32x4, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
        sl.mw[0] = x[0]; sl.mw[1] = x[1]; sl.mw[2] = x[2]; sl.mw[3] = x[3];
      } else if constexpr (NVG == 2) {
        const f32x2 x = load_vec<f32x2, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
        sl.mw[0] = x[0]; sl.mw[1] = x[1];
      } else {
        sl.mw[0] = load_vec<float, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
      }
    } else if constexpr (!KIVI) {
      sl.mw[0] = load_vec<float, kMetaNT>(
          reinterpret_cast<const uint8_t*>((part ? cv.v_scale : cv.k_scale) + (pair * cv.cap + T0 + qi)));
    } else if constexpr (M16) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(part ? cv.v_zero : cv.v_scale) +
                           (pair * cv.cap + T0 + qi) * NVG * 2;
      if constexpr (NVG == 4) {
        const u32x2 x = load_vec<u32x2, kMetaNT>(src);
        sl.mh[0] = x[0];
        sl.mh[1] = x[1];
      } else if constexpr (NVG == 2) {
        sl.mh[0] = load_vec<uint32_t, kMetaNT>(src);
      } else {
        sl.mh[0] = uint32_t(*reinterpret_cast<const uint16_t*>(src));
      }
      if constexpr (kGroupLoad) {
        const uint8_t* gsrc = reinterpret_cast<const uint8_t*>(part ? cv.k_zero : cv.k_scale) +
                              ((pair * (cv.cap / GG) + T0 / GG) * D + qi * KGL) * 2;
        if constexpr (KGL == 4) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(gsrc);
          sl.gh[0] = x[0];
          sl.gh[1] = x[1];
        } else {
          sl.gh[0] = *reinterpret_cast<const uint32_t*>(gsrc);
        }
      }
    } else {
      const float* src = (part ? cv.v_zero : cv.v_scale) + (pair * cv.cap + T0 + qi) * NVG;
      if constexpr (NVG == 4) {
        const f32x4 x = load_vec<f32x4, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
        sl.mw[0] = x[0]; sl.mw[1] = x[1]; sl.mw[2] = x[2]; sl.mw[3] = x[3];
      } else if constexpr (NVG == 2) {
        const f32x2 x = load_vec<f32x2, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
        sl.mw[0] = x[0]; sl.mw[1] = x[1];
      } else {
        sl.mw[0] = load_vec<float, kMetaNT>(reinterpret_cast<const uint8_t*>(src));
      }
      // the group parameters of the tile's group (used when it opens one)
      if constexpr (kGroupLoad) {
        const float* gsrc = (part ? cv.k_zero : cv.k_scale) + (pair * (cv.cap / GG) + T0 / GG) * D + qi * KGL;
        if constexpr (KGL == 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(gsrc);
          sl.gw[0] = x[0]; sl.gw[1] = x[1]; sl.gw[2] = x[2]; sl.gw[3] = x[3];
        } else {
          const f32x2 x = *reinterpret_cast<const f32x2*>(gsrc);
          sl.gw[0] = x[0]; sl.gw[1] = x[1];
        }
      }
    }
  };
  auto opens_group = [&](int k) { return KIVI && (k % TPG) == 0; };

  // ---- query, part 1: issue its loads (a clamped head; heads beyond the
  // GQA group read as 0). They go out before the first tiles' loads, so the
  // operand is built below while those tiles are in flight.
  u32x4 bq[NKK];
  constexpr int EPT = 8 * D / kThreads;  // KIVI: 4 (D = 128) or 2 (D = 64) elements per thread
  constexpr int NQX = KIVI ? EPT : CPL;
  float qx[NQX];
  if constexpr (KIVI) {
    const int e0 = tid * EPT, j = e0 / D, c = e0 % D;
    load_elems<BF16, EPT>(q, (size_t(b) * cv.Hq + size_t(h) * g + min(j, g - 1)) * D + c, qx);
  } else if constexpr (ROT) {
    // whole query rows of heads wave and wave + 4, CPL channels per lane,
    // rotated after the tiles' loads are issued
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = min(wave + 4 * u, g - 1);
      const size_t at = (size_t(b) * cv.Hq + size_t(h) * g + j) * D + lane * (D / kWave);
#pragma unroll
      for (int e = 0; e < D / kWave; ++e) qx[u * (D / kWave) + e] = load_elem<BF16>(q, at + e);
    }
  } else {
    const size_t qrow = (size_t(b) * cv.Hq + size_t(h) * g + min(hh, g - 1)) * D;
    if constexpr (BITS == 16 || INT4G) {
      // k-step kk of row group r: channels [32 kk + 8 r, 32 kk + 8 r + 8)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) load_elems<BF16, 8>(q, qrow + 32 * kk + 8 * r, qx + 8 * kk);
    } else if constexpr (KSPLIT) {
      load_elems<BF16, CPL / 2>(q, qrow + 16 * r, qx);
      load_elems<BF16, CPL / 2>(q, qrow + 64 + 16 * r, qx + CPL / 2);
    } else {
      load_elems<BF16, CPL>(q, qrow + CPL * r, qx);
    }
  }
  if (nk > 0) static_for<NPF>([&](auto uc) { load_tile(ring[decltype(uc)::value], decltype(uc)::value, uc); });

  // ---- query, part 2: KIVI stages q in LDS and keeps its share of the
  // normalized query (below); the others build the operand
  // KIVI Key-group fold layout: lane (m, r) computes both f16 terms of the
  // operand pairs of head hh, row group r, for the NKW k-steps from kk0 (the
  // hi lanes the first half, the lo lanes the second); the two lanes of a
  // (head, row group) then swap halves. qn = q * 2^eq for those elements,
  // eq putting the head's largest |q| in [64, 128).
  constexpr int NKW = NKK / 2;
  float qn[NKW][4][2];
  float kb4[NVG];  // group-wise INT4: 136 * the query sum of each channel group
  int eq = 0, fbase = 0;
  const float m1 = KIVI ? opaque_minus_one() : -1.0f;
  const Bf16Units bu = bf16_units();  // the probability split's dot-product units
  if constexpr (KIVI) {
    const int e0 = tid * EPT, j = e0 / D, c = e0 % D;
#pragma unroll
    for (int i = 0; i < EPT; ++i) sm.q[j][c + i] = j < g ? qx[i] : 0.0f;
    __syncthreads();
    const int kk0 = lo_col ? NKW : 0;
    fbase = CPL * r + cperm<BITS, KBYTE>(kk0, 0);  // the lane's elements sit at fbase + cperm(kw, i)
    float mx = 0.0f;
#pragma unroll
    for (int kw = 0; kw < NKW; ++kw)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int i = 2 * e + h2;
          const float v = sm.q[hh][fbase + cperm<BITS, KBYTE>(kw, i)];
          qn[kw][e][h2] = v;
          mx = fmaxf(mx, fabsf(v));
        }
    mx = max_rows(max_ror8(mx));
    eq = mx > 0.0f ? 7 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
    for (int kw = 0; kw < NKW; ++kw)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) qn[kw][e][h2] = __builtin_amdgcn_ldexpf(qn[kw][e][h2], eq);
  } else {
    if constexpr (ROT) {
      // q' = H q / d in LDS (H H = d I, so q' . (H k) = q . k); then the
      // lane's k-step channels as for the unrotated format
      constexpr int QPL = D / kWave;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float row[QPL];
#pragma unroll
        for (int e = 0; e < QPL; ++e) row[e] = qx[u * QPL + e];
        fwht_wave<QPL>(row);
        const int j = wave + 4 * u;
#pragma unroll
        for (int e = 0; e < QPL; ++e) sm.q[j][lane * QPL + e] = j < g ? row[e] * (1.0f / float(D)) : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qx[8 * kk + e] = sm.q[hh][32 * kk + 8 * r + e];
    }
    // group-wise INT4: the Key codes enter as 128 + (code + 8), so 136 times
    // the query sum of each channel group comes off its dot product. The sum
    // is taken over the hi + lo values the matrix core multiplies (exact in
    // fp32), so the offset cancels exactly.
    float qs[NVG];
#pragma unroll
    for (int gi = 0; gi < NVG; ++gi) qs[gi] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = hh < g ? qx[cperm<BITS>(kk, 2 * e)] : 0.0f;
        const float x1 = hh < g ? qx[cperm<BITS>(kk, 2 * e + 1)] : 0.0f;
        const Split2 sp = split_pair(x0, x1);
        bq[kk][e] = lo_col ? sp.lo : sp.hi;
        if constexpr (INT4G) {
          qs[kk / KPG] += (bf_lo(sp.hi) + bf_lo(sp.lo)) + (bf_hi(sp.hi) + bf_hi(sp.lo));
        }
      }
    }
    if constexpr (INT4G) {
#pragma unroll
      for (int gi = 0; gi < NVG; ++gi) kb4[gi] = sum_rows(qs[gi]) * 136.0f;
    }
  }

  auto process = [&](Slot& sl, int ti) {
    const int T0 = t0 + tile_of(ti) * kTile;
    const bool grp_open = opens_group(ti);
    const uint32_t (&kc)[2][LKB / 4] = sl.kw;
    const uint32_t* vc = sl.vw;
    {
      const int part = lane >> 5, qi = lane & 31;
      float* mdst = (part ? meta1 : meta0) + qi * NVG;
      // KIVI-2: token qi is element qi % 4 of its Value operand pair, whose
      // codes enter the matrix core times 1, 4, 16 or 1
      const float fq = (KIVI && BITS == 2 && part == 0) ? ((qi & 3) == 1 ? 0.25f : (qi & 3) == 2 ? 0.0625f : 1.0f)
                                                        : 1.0f;
      if constexpr (M16) {
#pragma unroll
        for (int j = 0; j < NVG; ++j) mdst[j] = KIVI && BITS == 2 ? half_at(sl.mh, j) * fq : half_at(sl.mh, j);
      } else if constexpr (KIVI && BITS == 2) {
#pragma unroll
        for (int j = 0; j < NVG; ++j) mdst[j] = sl.mw[j] * fq;
      } else if constexpr (SCALED) {
#pragma unroll
        for (int j = 0; j < NVG; ++j) mdst[j] = sl.mw[j];
      }
      if constexpr (KIVI) {
        if (grp_open) {
          // Key scales (lanes 0-31; >= 0) scaled by 2^kes so that the
          // group's largest lies in [64, 128); zero-points as they are
          float gv[KGL];
#pragma unroll
          for (int j = 0; j < KGL; ++j) {
            if constexpr (M16) gv[j] = half_at(sl.gh, j);
            else gv[j] = sl.gw[j];
          }
          // the largest scale's bit pattern (scales are >= 0, so the
          // unsigned order of the patterns is theirs); kes = 7 - its
          // binary exponent e (largest in [2^(e-1), 2^e)), 0 for all zero
          uint32_t mb = 0u;
#pragma unroll
          for (int j = 0; j < KGL; ++j) {
            const uint32_t u = __builtin_bit_cast(uint32_t, gv[j]);
            mb = mb > u ? mb : u;
          }
          mb = max_lanes32_bits(mb);
          if (mb >= 0x00800000u) kes = 133 - int(mb >> 23);     // normal: e = biased exponent - 126
          else kes = mb != 0u ? 124 + __builtin_clz(mb) : 0;  // subnormal: e = 32 - clz - 149
          const int kl = part ? 0 : kes;
          float* gdst = sm.kgrp[wave][part] + qi * KGL;
#pragma unroll
          for (int j = 0; j < KGL; ++j) gdst[j] = __builtin_amdgcn_ldexpf(gv[j], kl);
        }
      }
    }
    wave_lds_sync();

    // ---- KIVI: fold this group's per-channel Key scales into the query ----
    // x_c = qn_c * s'_c (|x| < 2^14) split into f16 hi + lo (about 22
    // significant bits); the score of a token is then
    //   acc * 2^(-eq - kes) + sum_c q_c z_c,
    // acc the matrix-core sum of x against the Key codes.
    if constexpr (KIVI) {
      if (grp_open) {
        const float* ksr = &sm.kgrp[wave][0][fbase];
        const float* kzr = &sm.kgrp[wave][1][fbase];
        const float* qr = &sm.q[hh][fbase];
        uint32_t xh[NKW][4], xl[NKW][4];
        float qzs = 0.0f;
#pragma unroll
        for (int kw = 0; kw < NKW; ++kw)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int oa = cperm<BITS, KBYTE>(kw, 2 * e), ob = cperm<BITS, KBYTE>(kw, 2 * e + 1);
            const float x0 = qn[kw][e][0] * ksr[oa];
            const float x1 = qn[kw][e][1] * ksr[ob];
            xh[kw][e] = pack_f16(x0, x1);
            xl[kw][e] = f16_residual(xh[kw][e], x0, x1, m1);
            qzs = fmaf(qr[oa], kzr[oa], qzs);
            qzs = fmaf(qr[ob], kzr[ob], qzs);
          }
        // k-steps [0, NKW): hi lanes keep their own hi term, lo lanes take
        // the hi lane's lo term; [NKW, 2 NKW): the other way round
#pragma unroll
        for (int kw = 0; kw < NKW; ++kw)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bq[kw][e] = swap8_into<0xc>(xh[kw][e], xl[kw][e]);
            bq[NKW + kw][e] = swap8_into<0x3>(xl[kw][e], xh[kw][e]);
          }
        kbias = sum_rows(add_ror8(qzs)) * sm_log2;
        kscale = __builtin_amdgcn_ldexpf(sm_log2, -eq - kes);
      }
    }

    // ---- scores ----
    // group-wise INT4: one accumulator per channel group (its scale is per
    // token); the others: one per score tile
    constexpr int NACC = INT4G ? NVG : 1;
    f32x4 acc[2][NACC];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int gi = 0; gi < NACC; ++gi) acc[t][gi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int gi = INT4G ? kk / KPG : 0;
        if constexpr (KIVI) acc[t][gi] = mfma_f16(key_operand<FMT, BITS>(kc[t], kk), bq[kk], acc[t][gi]);
        else acc[t][gi] = mfma_bf16(key_operand<FMT, BITS>(kc[t], kk), bq[kk], acc[t][gi]);
      }
    }
    const int valid = KIVI ? kTile : min(kTile, t1 - T0);
    // this lane's tokens: tok(t, r, j) = base_t + j, 4 consecutive per t
    f32x4 ks[2], vs[2];
    if constexpr (!KIVI && SCALED && !INT4G) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ks[t] = *reinterpret_cast<const f32x4*>(meta0 + tok<BITS>(t, r, 0));
        vs[t] = *reinterpret_cast<const f32x4*>(meta1 + tok<BITS>(t, r, 0));
      }
    }
    // HALF: the hi and lo lanes of a head hold the same scores after the
    // column sum; each lane keeps the half its Value operand pairs need
    // (elements ja, ja + 1 of each score tile) and takes the softmax of
    // those only
    const int ja = lo_col ? 2 : 0;
    const uint32_t lo_mask = lo_col ? 0xffffffffu : 0u;
    constexpr int NSC = HALF ? 2 : 4;  // scores per score tile the lane keeps
    float sc[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float xs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x;
        if constexpr (INT4G) {
          // sum over channel groups of (dot - bias) * the token's group scale
          const float* ksr = meta0 + tok<BITS>(t, r, j) * NVG;
          x = 0.0f;
#pragma unroll
          for (int gi = 0; gi < NVG; ++gi) x = fmaf(add_ror8(acc[t][gi][j]) - kb4[gi], ksr[gi], x);
          x *= sm_log2;
        } else {
          x = add_ror8(acc[t][0][j]);
        }
        if constexpr (KIVI || INT4G) (void)0;
        else if constexpr (SCALED) x = x * ks[t][j] * sm_log2;
        else x = x * sm_log2;
        if (!KIVI && tok<BITS>(t, r, j) >= valid) x = -INFINITY;  // KIVI tiles are whole
        xs[j] = x;
      }
#pragma unroll
      for (int u = 0; u < NSC; ++u) {
        float x = HALF ? select_bits(lo_mask, xs[2 + u], xs[u]) : xs[u];
        if constexpr (KIVI) x = fmaf(x, kscale, kbias);
        sc[t][u] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    // Lazy rescale: the running maximum moves only when a score exceeds it
    // by more than kLazyLog2, so the accumulators are rescaled on few tiles
    // and every probability stays below 2^kLazyLog2. The four lanes of a
    // column share m_run, so a lane's own maximum decides whether any column
    // needs it; the column maximum across the lanes (two lane exchanges) is
    // taken only on the tiles that rescale.
    if (__any(tmax > m_run + kLazyLog2)) {
      tmax = max_rows(HALF ? max_ror8(tmax) : tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NMT; ++i) o[i] *= alpha;
      if constexpr (KIVI) {
#pragma unroll
        for (int j = 0; j < NVG; ++j) zb[j] *= alpha;
      }
    }
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int j = 0; j < NSC; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[t][j] - m_run);
        sc[t][j] = p;
        psum += p;
      }
    l_run += psum;

    // ---- values ----
    if constexpr (!KIVI && !INT4G) {
      float pv[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pv[t][j] = tok<BITS>(t, r, j) < valid ? (SCALED ? sc[t][j] * vs[t][j] : sc[t][j]) : 0.0f;
      const u32x4 bp = prob_operand<BITS>(pv, lo_col);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        u32x4 a = value_operand<FMT, BITS>(vc, mt, r);
        if (valid < kTile) a = mask_tokens8(a, r, valid);
        o[mt] = mfma_bf16(a, bp, o[mt]);
      }
    } else {
      // The hi and lo lanes of a column pair hold the same probabilities.
      // Each takes two of the four operand pairs (pair k = tokens (0, k) and
      // (1, k) of the score tiles: the hi lane k = 0, 1, the lo lane k = 2,
      // 3), splits them into both terms, and the two lanes swap halves.
      const float(&ps)[2][4] = sc;  // the lane's probabilities of pairs ja, ja + 1
      // per-token Value scale and zero of each channel group, for the lane's
      // two tokens of each score tile
      // KIVI: meta0 Value scales, meta1 Value zero-points; group-wise INT4:
      // meta1 Value scales (meta0 holds the Key scales), no zero-points
      const float* vsm = INT4G ? meta1 : meta0;
      float vsf[2][2 * NVG], vzf[2][2 * NVG];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int off = (tok<BITS>(t, r, 0) + ja) * NVG;
        if constexpr (NVG == 1) {
          const f32x2 a = *reinterpret_cast<const f32x2*>(vsm + off);
          const f32x2 z = *reinterpret_cast<const f32x2*>(meta1 + off);
          vsf[t][0] = a[0]; vsf[t][1] = a[1];
          vzf[t][0] = z[0]; vzf[t][1] = z[1];
        } else {
#pragma unroll
          for (int v = 0; v < NVG / 2; ++v) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(vsm + off + 4 * v);
            const f32x4 z = *reinterpret_cast<const f32x4*>(meta1 + off + 4 * v);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              vsf[t][4 * v + i] = a[i];
              vzf[t][4 * v + i] = z[i];
            }
          }
        }
      }
#pragma unroll
      for (int jg = 0; jg < NVG; ++jg) {
        float pv[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float vsc = vsf[t][u * NVG + jg];
            // group-wise INT4: a token past the end of the last, partial
            // tile contributes exactly 0, whatever its stored scale holds
            // (KIVI tiles are always whole)
            if constexpr (INT4G) pv[t][u] = tok<BITS>(t, r, ja + u) < valid ? ps[t][u] * vsc : 0.0f;
            else pv[t][u] = ps[t][u] * vsc;
            if constexpr (KIVI) zb[jg] = fmaf(ps[t][u], vzf[t][u * NVG + jg], zb[jg]);
          }
        const Split2 s0 = split_pair_dot(pv[0][0], pv[1][0], bu);  // pair ja
        const Split2 s1 = split_pair_dot(pv[0][1], pv[1][1], bu);  // pair ja + 1
        u32x4 bp;
        bp[0] = swap8_into<0xc>(s0.hi, s0.lo);
        bp[1] = swap8_into<0xc>(s1.hi, s1.lo);
        bp[2] = swap8_into<0x3>(s0.lo, s0.hi);
        bp[3] = swap8_into<0x3>(s1.lo, s1.hi);
#pragma unroll
        for (int mt = jg * MPG; mt < (jg + 1) * MPG; ++mt) {
          o[mt] = mfma_bf16(value_operand<FMT, BITS>(vc, mt, r), bp, o[mt]);
          // the codes entered as 128 + code: take (128 + kCenter) * p' off
          // in the same accumulator every tile
          o[mt] = mfma_bf16(kCenterA, bp, o[mt]);
        }
      }
    }
    wave_lds_sync();  // metadata reads done before the next tile overwrites it
  };

  if (nk > 0) {
    for (int base = 0; base < nk; base += NPF) {
      static_for<NPF>([&](auto uc) {
        constexpr int U = decltype(uc)::value;
        const int ti = base + U;
        if (ti < nk) process(ring[U], ti);
        load_tile(ring[U], ti + NPF, uc);
      });
    }
  }

  // ---- the fused step's new token: a fifth piece ----
  bool has_new = false;
  if constexpr (FUSED && !KIVI) {
    has_new = t_new >= 0;  // uniform
    if (has_new) new_token_piece<FMT, D, G, BF16>(cv, b, h, t_new, ap, q, sm_log2, sm);
  }

  // ---- merge the 4 waves (and the new token) through LDS ----
  const float l_tot = sum_rows(HALF ? add_ror8(l_run) : l_run);
  float zt[NVG];
#pragma unroll
  for (int j = 0; j < NVG; ++j) zt[j] = sum_rows(add_ror8(zb[j]));  // hi and lo lanes hold disjoint tokens
  if (lane < 8) {
    sm.m[wave][lane] = m_run;
    sm.l[wave][lane] = l_tot;
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = add_ror8(o[mt][j]);
      if constexpr (KIVI) x += zt[mt / MPG];
      if (!lo_col) sm.o[wave][hh][16 * mt + 4 * r + j] = x;
    }
  }
  __syncthreads();
  // thread (j, c4): head j, channels [4 c4, 4 c4 + 4); one 16-byte store
  constexpr int C4 = D / 4;
  const int tm = fresh(tid);
  const int j = tm / C4, c4 = tm % C4;
  if (j < g) {
    const int npiece = kWaves + (has_new ? 1 : 0);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves + 1; ++w)
      if (w < npiece) M = fmaxf(M, sm.m[w][j]);
    f32x4 ov = {0.0f, 0.0f, 0.0f, 0.0f};
    float L = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves + 1; ++w) {
        if (w >= npiece) break;
        const float f = __builtin_amdgcn_exp2f(sm.m[w][j] - M);
        ov += *reinterpret_cast<const f32x4*>(&sm.o[w][j][4 * c4]) * f;
        L += sm.l[w][j] * f;
      }
    }
    const size_t row = partial_row(cv, wk, b, h, j, s);
    const size_t row0 = partial_row(cv, wk, b, h, 0, 0);
    put_partial4(buffer_rsrc(wk.o + row0 * D, uint32_t(g * wk.S * D * 4)), uint32_t(((row - row0) * D + 4 * c4) * 4),
                 ov);
    if (c4 == 0) {
      put_partial(&wk.m[row], M);
      put_partial(&wk.l[row], L);
    }
  }
}

// ---------------------------------------------------------------------------
// KIVI residual ring (tokens [nq, n), full precision), in chunks of 64
// tokens on the vector ALU. Every load of a chunk is issued before any is
// used, so a chunk costs one memory round trip: the scores take four lanes
// per token (a quarter of the row each, 16-byte loads, summed by
// shuffles); the values take lane (channel pair, token part), the parts
// summed by shuffles at the end. Writes partial slot s.
//
// Fused append + decode (FUSED, app): token n - 1 is the new input token.
// It is written to its ring slot when it stays in the residual window, and
// read from the input row. When it completes a group (the flush rule now
// admits tokens [nq, nq + G)), that group is quantized here by the append's
// own steps, and attention reads it as the dequantized codes, code * s + z,
// exactly as an attention call after the append would.
// ---------------------------------------------------------------------------
template <int D, bool BF16, int BITS, int G, bool FUSED, bool M16>
__device__ __forceinline__ void split_residual(const CacheView& cv, int b, int h, int s, int nq, int n,
                                               const void* __restrict__ q, float sm_log2, const DecodeWork& wk,
                                               SmemResidT<D, G, FUSED>& sm, const AppendIn& ap, bool app) {
  constexpr int NH = 8;
  constexpr int T = kResidChunk;
  constexpr int QPT = kThreads / T;       // lanes per token in the score phase
  constexpr int CPT = D / QPT;            // their channels: 32 (d = 128) or 16 (d = 64)
  constexpr int NP = kThreads / (D / 2);  // token parts in the value phase: 4 (d = 128) or 8 (d = 64)
  constexpr int TPP = T / NP;             // tokens per part and chunk
  static_assert(T == kWave && QPT * T == kThreads && NP * (D / 2) == kThreads, "residual layout");
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = cv.g, C = cv.C;
  const size_t pair = pair_index(cv, b, h);
  const size_t ring = pair * size_t(C);
  for (int e = tid; e < NH * D; e += kThreads) {
    const int j = e / D, c = e % D;
    sm.q[j][c] = j < g ? load_elem<BF16>(q, (size_t(b) * cv.Hq + size_t(h) * g + j) * D + c) : 0.0f;
  }
  for (int e = tid; e < NH * T; e += kThreads) sm.sc[e / T][e % T] = 0.0f;  // heads >= g stay 0
  if (tid < NH) {
    sm.st_m[tid] = -INFINITY;
    sm.st_l[tid] = 0.0f;
    sm.st_a[tid] = 1.0f;
  }
  const int ti = tid / QPT, cq = (tid % QPT) * CPT;  // scores: token ti, channels [cq, cq + CPT)
  const int part = tid % NP, cp = tid / NP;          // values: channels 2 cp, 2 cp + 1
  float acc[NH][2];
#pragma unroll
  for (int j = 0; j < NH; ++j) acc[j][0] = acc[j][1] = 0.0f;

  // Steps of one chunk of nt tokens: the lane's partial dot products (token
  // ti) to scores, the online softmax update of every head, and the
  // weighted Value sum (the lane's tokens part + NP u, channels 2 cp, 2 cp+1).
  auto put_scores = [&](float (&sco)[NH], int nt) {
#pragma unroll
    for (int o = 1; o < QPT; o <<= 1)
#pragma unroll
      for (int j = 0; j < NH; ++j) sco[j] += __shfl_xor(sco[j], o, kWave);
    if (tid % QPT == 0 && ti < nt) {
#pragma unroll
      for (int j = 0; j < g && j < NH; ++j) sm.sc[j][ti] = sco[j] * sm_log2;
    }
    __syncthreads();
  };
  auto softmax_step = [&](int nt) {
    for (int j = wave; j < g; j += kWaves) {
      const float sc = lane < nt ? sm.sc[j][lane] : -INFINITY;
      const float mx = wave_max(sc);
      const float m_old = sm.st_m[j];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
      const float p = lane < nt ? __builtin_amdgcn_exp2f(sc - m_new) : 0.0f;
      sm.sc[j][lane] = p;
      const float sum = wave_sum(p);
      if (lane == 0) {
        sm.st_m[j] = m_new;
        sm.st_l[j] = sm.st_l[j] * alpha + sum;
        sm.st_a[j] = alpha;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float a = sm.st_a[j];
      acc[j][0] *= a;
      acc[j][1] *= a;
    }
  };
  auto value_step = [&](const float (&vx)[TPP][2], int nt) {
#pragma unroll
    for (int u = 0; u < TPP; ++u) {
      const int i = part + NP * u;
      const bool in = i < nt;
      const float v0 = in ? vx[u][0] : 0.0f, v1 = in ? vx[u][1] : 0.0f;
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const float p = sm.sc[j][i];
        acc[j][0] = fmaf(p, v0, acc[j][0]);
        acc[j][1] = fmaf(p, v1, acc[j][1]);
      }
    }
    __syncthreads();  // probability reads done before the next chunk's scores
  };

  int cs0 = nq;  // first token read from the ring
  if constexpr (FUSED) {
    if (app) {
      const int t_new = n - 1;
      const int nq1 = kivi_quantized(n, G, cv.R);
      if (t_new >= nq1) {
        // the new token stays in the residual window: its ring slot held a
        // token older than nq, no longer read
        constexpr int VPR = D * (BF16 ? 2 : 4) / 16;  // 16-byte vectors per row
        if (tid < 2 * VPR) {
          const int v = tid % VPR;
          const uint8_t* src = static_cast<const uint8_t*>(tid < VPR ? ap.k : ap.v) + (pair * VPR + v) * 16;
          uint8_t* dst = (tid < VPR ? cv.k_resid : cv.v_resid) + ((ring + size_t(t_new % C)) * VPR + v) * 16;
          *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        }
      }
      if (nq1 > nq) {
        // the group [nq, nq + G) completes: flush it, then attend over it
        constexpr float QMAX = float((1 << BITS) - 1);
        static_assert(G <= T, "a group fits one chunk");
        const int grp = nq / G;
        FlushSmem<G, D>& f = sm.f;
        flush_stage<BF16, G, D>(f, cv, pair, grp, t_new, ap.k, 1, cv.k_resid);
        flush_key<BITS, G, D, M16>(f, cv, pair, grp);
        // the staged tile becomes the dequantized Key rows, code * s + z
        for (int e = tid; e < G * D; e += kThreads) {
          const int i = e / D, c = e % D;
          f.xs[i][c] = float(asym_code(f.xs[i][c], f.sk[c], f.zk[c], QMAX)) * f.sk[c] + f.zk[c];
        }
        __syncthreads();
        float sco[NH];
#pragma unroll
        for (int j = 0; j < NH; ++j) sco[j] = 0.0f;
        if (ti < G) {
#pragma unroll
          for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int j = 0; j < NH; ++j) sco[j] = fmaf(sm.q[j][cq + k], f.xs[ti][cq + k], sco[j]);
        }
        put_scores(sco, G);
        softmax_step(G);
        flush_stage<BF16, G, D>(f, cv, pair, grp, t_new, ap.v, 1, cv.v_resid);
        flush_value<BITS, G, D, M16>(f, cv, pair, grp);
        for (int e = tid; e < G * D; e += kThreads) {
          const int i = e / D, c = e % D;
          const float sv = f.sv[i][c / G], zv = f.zv[i][c / G];
          f.xs[i][c] = float(asym_code(f.xs[i][c], sv, zv, QMAX)) * sv + zv;
        }
        __syncthreads();
        float vx[TPP][2];
#pragma unroll
        for (int u = 0; u < TPP; ++u) {
          const int i = min(part + NP * u, G - 1);
          vx[u][0] = f.xs[i][2 * cp];
          vx[u][1] = f.xs[i][2 * cp + 1];
        }
        value_step(vx, G);
        cs0 = nq1;
      }
    }
  }
  __syncthreads();
  // token t's row: its ring slot, or for the new token of a fused step the
  // input row
  auto row = [&](const uint8_t* ringp, const void* inp, int t) -> const void* {
    if constexpr (FUSED) {
      if (app && t == n - 1) return static_cast<const uint8_t*>(inp) + pair * D * (BF16 ? 2 : 4);
    }
    return ringp + (ring + size_t(t % C)) * D * (BF16 ? 2 : 4);
  };
  for (int cs = cs0; cs < n; cs += T) {
    const int nt = min(T, n - cs);
    // the chunk's loads (ring slots are in bounds for any token index; the
    // values of tokens past the chunk are zeroed below)
    float kx[CPT];
    load_elems<BF16, CPT>(row(cv.k_resid, ap.k, cs + ti), cq, kx);
    float vx[TPP][2];
#pragma unroll
    for (int u = 0; u < TPP; ++u) load_elems<BF16, 2>(row(cv.v_resid, ap.v, cs + part + NP * u), 2 * cp, vx[u]);
    float sco[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) sco[j] = 0.0f;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
      for (int j = 0; j < NH; ++j) sco[j] = fmaf(sm.q[j][cq + k], kx[k], sco[j]);
    put_scores(sco, nt);
    softmax_step(nt);
    value_step(vx, nt);
  }
#pragma unroll
  for (int o = 1; o < NP; o <<= 1)
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      acc[j][0] += __shfl_xor(acc[j][0], o, kWave);
      acc[j][1] += __shfl_xor(acc[j][1], o, kWave);
    }
  if (part == 0) {
    for (int j = 0; j < g; ++j) {
      const size_t prow = partial_row(cv, wk, b, h, j, s) * D + 2 * cp;
      put_partial(&wk.o[prow], acc[j][0]);
      put_partial(&wk.o[prow + 1], acc[j][1]);
    }
  }
  if (tid < g) {
    const size_t prow = partial_row(cv, wk, b, h, tid, s);
    put_partial(&wk.m[prow], sm.st_m[tid]);
    put_partial(&wk.l[prow], sm.st_l[tid]);
  }
}

// Work items. Each (sequence, kv head) pair's quantized tokens are cut into
// NC chunks (whole 32-token tiles, whole groups for KIVI) at fixed fractions
// of its length: n1 chunks of weight w1, then n2 of weight w2, then n3 of
// weight w3, so that (with decreasing weights) the later chunks are smaller.
// A KIVI pair has one more item, its residual window (slot NC). The items
// are numbered residual items first, then the first-phase chunks of every
// pair, the second, the third (pair by pair within a phase); one workgroup
// runs each (see decode_split for the order they go out in). Every item
// writes its partial state (an empty range writes an empty state) and takes
// a ticket from its pair's counter; the item that finishes last merges the
// pair's NC (+1) partial states of the g query heads by the log-sum-exp
// rule, writes the normalized output and resets the counter to zero.
template <int FMT, int BITS, int D, int G, bool FUSED, bool BF16>
constexpr int min_wg_per_cu() {
  if constexpr (KVQ_DECODE_MIN_WG_PER_CU > 0) return KVQ_DECODE_MIN_WG_PER_CU;
  // the fused INT2 KIVI step with fp32 inputs at d = 128 (its flush path
  // quantizes the completed group from fp32 rows) needs a few registers more
  if constexpr ((FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16) && BITS == 2 && D == 128 && FUSED && !BF16) return 2;
  // INT2 KIVI with binary16 metadata at G = 32, d = 128 (a Key fold every
  // tile plus the half widening; the fused step also the flush path) needs
  // a few registers more than three workgroups per unit leave
  if constexpr (FMT == KVQ_FMT_KIVI_F16 && BITS == 2 && D == 128 && G == 32) return 2;
  // bf16 rows hold twice the 8-bit codes' registers in the prefetch ring
  return ((FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16) && BITS == 4 && D == 128 && G == 32) || BITS == 16 ? 2
                                                                                                        : 3;
}

// Chunk j's first unit of nu units (j = NC gives nu): nu times the weight of
// the chunks before j, over the total weight.
__device__ __forceinline__ int chunk_start(const DecodeWork& wk, int j, int nu) {
  int c;
  if (j <= wk.n1) c = j * wk.w1;
  else if (j <= wk.n1 + wk.n2) c = wk.n1 * wk.w1 + (j - wk.n1) * wk.w2;
  else c = wk.n1 * wk.w1 + wk.n2 * wk.w2 + (j - wk.n1 - wk.n2) * wk.w3;
  const int wt = wk.n1 * wk.w1 + wk.n2 * wk.w2 + wk.n3 * wk.w3;
  return int(int64_t(nu) * c / wt);
}

// Partial state of an empty piece: output 0, maximum -inf, sum 0.
template <int D>
__device__ __forceinline__ void put_empty_partial(const CacheView& cv, const DecodeWork& wk, int b, int h, int s) {
  const int tid = threadIdx.x;
  for (int e = tid; e < cv.g * D; e += kThreads) {
    const int j = e / D, c = e % D;
    put_partial(&wk.o[partial_row(cv, wk, b, h, j, s) * D + c], 0.0f);
  }
  if (tid < cv.g) {
    const size_t row = partial_row(cv, wk, b, h, tid, s);
    put_partial(&wk.m[row], -INFINITY);
    put_partial(&wk.l[row], 0.0f);
  }
}

// What an item needs after its token loop, parked in LDS so that it does
// not hold scalar registers through the loop.
struct ItemTail {
  int b, h, n;
  int app;
};

// One work item: item i (numbered as above) of the P = B * Hkv pairs.
template <int FMT, int BITS, int D, int G, bool BF16, bool FUSED>
__device__ __forceinline__ void decode_item(const CacheView& cv, const int32_t* seq_lens, const void* __restrict__ q,
                                            int lens, float sm_log2, float* __restrict__ out,
                                            const DecodeWork& wk, const AppendIn& ap, int i, float* smem,
                                            uint32_t& ticket, ItemTail& tail) {
  constexpr bool KIVI = FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16;
  const int tid = threadIdx.x;
  const int g = cv.g;
  const int P = cv.B * cv.Hkv;
  const int NC = wk.n1 + wk.n2 + wk.n3;  // = S - 1
  int pair, s;
  if (KIVI && i < P) {
    pair = i;
    s = NC;
  } else {
    if (KIVI) i -= P;
    if (i < P * wk.n1) {
      pair = i / wk.n1;
      s = i % wk.n1;
    } else if ((i -= P * wk.n1) < P * wk.n2) {
      pair = i / wk.n2;
      s = wk.n1 + i % wk.n2;
    } else {
      i -= P * wk.n2;
      pair = i / wk.n3;
      s = wk.n1 + wk.n2 + i % wk.n3;
    }
  }
  const int b = pair / cv.Hkv, h = pair % cv.Hkv;
  // Tokens in the cache, and for a fused step whether this sequence takes
  // the new token (the append's rule: a valid length with room for one more;
  // otherwise the sequence is left unchanged and attention reads it as is).
  // lens: lane l holds seq_lens[l] for l < min(B, 64)
  const int raw = b < kWave ? __builtin_amdgcn_readlane(lens, b) : seq_lens[b];
  bool app = false;
  if constexpr (FUSED) app = raw >= 0 && raw < cv.max_tokens;
  if constexpr (FUSED) {
    if (ap.skipped != nullptr && s == 0 && h == 0 && tid == 0) ap.skipped[b] = app ? 0 : 1;
  }
  const int n_cache = min(max(raw, 0), cv.max_tokens);
  const int n = n_cache + (app ? 1 : 0);  // tokens attended
  // quantized tokens the chunks read (KIVI: the new token, and a group it
  // completes, are handled by the residual item)
  const int nq = KIVI ? kivi_quantized(n_cache, G, cv.R) : n_cache;
  if (tid == 0) tail = {b, h, n, app ? 1 : 0};
  if (s == NC) {
    // the KIVI residual window
    if constexpr (KIVI) {
      if (n > nq)
        split_residual<D, BF16, BITS, G, FUSED, FMT == KVQ_FMT_KIVI_F16>(
            cv, b, h, s, nq, n, q, sm_log2, wk, *reinterpret_cast<SmemResidT<D, G, FUSED>*>(smem), ap, app);
      else
        put_empty_partial<D>(cv, wk, b, h, s);
    }
  } else {
    // chunk s in whole tiles (whole groups for KIVI, so that a Key group
    // never straddles two chunks); a fused step of a per-token format also
    // takes the new token in chunk 0
    constexpr int kUnit = KIVI ? G : kTile;
    const int nu = (nq + kUnit - 1) / kUnit;
    const int t0 = min(chunk_start(wk, s, nu) * kUnit, nq);
    const int t1 = min(chunk_start(wk, s + 1, nu) * kUnit, nq);
    const int t_new = (FUSED && !KIVI && app && s == 0) ? n_cache : -1;
    split_quantized<FMT, BITS, D, G, BF16, FUSED>(cv, b, h, s, t0, t1, q, sm_log2, wk,
                                                  *reinterpret_cast<SmemQuant<D>*>(smem), t_new, ap);
  }

  // ---- arrival: the last item of this (sequence, kv head) merges ----
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed ...
  __syncthreads();                 // ... for every thread, before the ticket is taken
  const ItemTail it = tail;
  const size_t pr = pair_index(cv, it.b, it.h);
  if (tid == 0) ticket = __hip_atomic_fetch_add(&wk.count[pr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int nact = NC + (KIVI ? 1 : 0);  // pieces per pair, every one with a partial state
  if (ticket != uint32_t(nact - 1)) return;

  // Merge by the log-sum-exp rule. Thread (j, c4) owns channels [4 c4,
  // 4 c4 + 4) of head j. For up to kMergeBatch pieces at a time it loads,
  // in one batch of coherent loads, its 16 bytes of every piece's partial
  // output and the piece's (max, sum) of head j, and folds them into a
  // running (max, sum, output); at most kMergeBatch pieces merge in one
  // round trip, with no barrier. Piece k is partial slot k.
  constexpr int kMergeBatch = 16;
  constexpr int C4 = D / 4;
  const int tm = fresh(tid);
  const int j = tm / C4, c4 = tm % C4;
  const int jc = min(j, g - 1);
  const size_t row0 = partial_row(cv, wk, it.b, it.h, 0, 0);
  const size_t mrow = row0 + size_t(jc) * wk.S;
  const __amdgpu_buffer_rsrc_t orsrc = buffer_rsrc(wk.o + row0 * D, uint32_t(g * wk.S * D * 4));
  const uint32_t obase = uint32_t((size_t(jc) * wk.S * D + 4 * c4) * 4);
  float M = -INFINITY, L = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k0 = 0; k0 < nact; k0 += kMergeBatch) {
    f32x4 ov[kMergeBatch];
    float mv[kMergeBatch], lv[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      if (k0 + u < nact) {
        const int sl = k0 + u;
        ov[u] = get_partial4(orsrc, obase + uint32_t(sl * D * 4));
        mv[u] = get_partial(&wk.m[mrow + sl]);
        lv[u] = get_partial(&wk.l[mrow + sl]);
      } else {
        ov[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        mv[u] = -INFINITY;
        lv[u] = 0.0f;
      }
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) mn = fmaxf(mn, mv[u]);
    if (mn != -INFINITY) {
      const float a = __builtin_amdgcn_exp2f(M - mn);  // 0 while nothing is merged yet
      acc *= a;
      L *= a;
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = __builtin_amdgcn_exp2f(mv[u] - mn);  // 0 for empty pieces
        acc += ov[u] * w;
        L = fmaf(lv[u], w, L);
      }
      M = mn;
    }
  }
  if (j < g)
    *reinterpret_cast<f32x4*>(&out[(size_t(it.b) * cv.Hq + size_t(it.h) * g + j) * D + 4 * c4]) =
        acc * (L > 0.0f ? 1.0f / L : 0.0f);
  if (tid == 0) {
    __hip_atomic_store(&wk.count[pr], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if constexpr (FUSED) {
      if (it.app) {
        // the last (sequence, kv head) merge of sequence b: every item of
        // the sequence has read seq_lens[b]
        const uint32_t done = __hip_atomic_fetch_add(&wk.bcount[it.b], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        if (done == uint32_t(cv.Hkv - 1)) {
          __hip_atomic_store(&wk.bcount[it.b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ap.seq_lens[it.b] = it.n;
        }
      }
    }
  }
}

// One workgroup per work item. Workgroup x < wk.nstatic (with a dynamic
// plan, the first round: the workgroups the device holds at once) takes
// item x. Every later workgroup draws a number from wk.queue and takes item
// nstatic + number, so the items after the first round go out in the order
// slots free up (not by launch index): a unit that finishes early gets the
// next item of the list, whichever XCD it is on (each XCD launches its own
// share of the grid). Drawing only after the first round spreads the draws
// over the call; all of them at its start contend on the one counter. The
// workgroup that draws the last number resets the counter for the next
// call. The sequence lengths (up to 64 of them) are loaded in the same
// round trip as the number.
template <int FMT, int BITS, int D, int G, bool BF16, bool FUSED>
__global__ __launch_bounds__(kThreads, (min_wg_per_cu<FMT, BITS, D, G, FUSED, BF16>())) void decode_split(
    CacheView cv, const int32_t* seq_lens, const void* __restrict__ q, float sm_log2, float* __restrict__ out,
    DecodeWork wk, AppendIn ap) {
  constexpr bool KIVI = FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16;
  __shared__ float smem[smem_floats<D, (KIVI ? G : 0), FUSED>()];
  __shared__ uint32_t ticket, item_sh;
  __shared__ ItemTail tail;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int lens = lane < cv.B ? seq_lens[lane] : 0;
  int item = blockIdx.x;
  if (item >= wk.nstatic) {
    if (tid == 0) {
      const uint32_t nd = uint32_t(wk.nitems - wk.nstatic);
      const uint32_t it = __hip_atomic_fetch_add(wk.queue, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (it == nd - 1) __hip_atomic_store(wk.queue, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // a counter that was not zero on entry (a broken workspace contract)
      // still yields item numbers in range
      item_sh = uint32_t(wk.nstatic) + it % nd;
    }
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(int(item_sh));
  }
  decode_item<FMT, BITS, D, G, BF16, FUSED>(cv, seq_lens, q, lens, sm_log2, out, wk, ap, item, smem, ticket, tail);
}

// One kernel instantiation per (format, bits, head_dim, group, input type).
template <int FMT_, int BITS_, int D_, int G_, bool BF16_>
struct Variant {
  static constexpr int FMT = FMT_, BITS = BITS_, D = D_, G = G_;
  static constexpr bool BF16 = BF16_;
};

template <int FMT, int BITS, int D, bool BF16, class F>
void visit_g(const CacheView& cv, F&& f) {
  if constexpr (FMT == KVQ_FMT_INT4 || FMT == KVQ_FMT_INT4_HADAMARD) {
    // groups divide head_dim: 128-channel groups exist only at d = 128
    if (cv.G == 32) f(Variant<FMT, BITS, D, 32, BF16>{});
    else if constexpr (D == 64) f(Variant<FMT, BITS, D, 64, BF16>{});
    else if (cv.G == 64) f(Variant<FMT, BITS, D, 64, BF16>{});
    else f(Variant<FMT, BITS, D, 128, BF16>{});
  } else if constexpr (FMT == KVQ_FMT_KIVI || FMT == KVQ_FMT_KIVI_F16) {
    if (cv.G == 32) f(Variant<FMT, BITS, D, 32, BF16>{});
    else f(Variant<FMT, BITS, D, 64, BF16>{});
  } else {
    f(Variant<FMT, BITS, D, 0, BF16>{});
  }
}

template <int FMT, int BITS, bool BF16, class F>
void visit_d(const CacheView& cv, F&& f) {
  if (cv.D == 128) visit_g<FMT, BITS, 128, BF16>(cv, f);
  else visit_g<FMT, BITS, 64, BF16>(cv, f);
}

template <bool BF16, class F>
void visit_fmt(const CacheView& cv, F&& f) {
  switch (cv.fmt) {
    case KVQ_FMT_FP8_E4M3: visit_d<KVQ_FMT_FP8_E4M3, 8, BF16>(cv, f); break;
    case KVQ_FMT_INT8: visit_d<KVQ_FMT_INT8, 8, BF16>(cv, f); break;
    case KVQ_FMT_BF16: visit_d<KVQ_FMT_BF16, 16, BF16>(cv, f); break;
    case KVQ_FMT_INT4: visit_d<KVQ_FMT_INT4, 4, BF16>(cv, f); break;
    case KVQ_FMT_FP8_STATIC: visit_d<KVQ_FMT_FP8_STATIC, 8, BF16>(cv, f); break;
    case KVQ_FMT_INT4_HADAMARD: visit_d<KVQ_FMT_INT4_HADAMARD, 4, BF16>(cv, f); break;
    case KVQ_FMT_KIVI_F16:
      if (cv.bits == 4) visit_d<KVQ_FMT_KIVI_F16, 4, BF16>(cv, f);
      else visit_d<KVQ_FMT_KIVI_F16, 2, BF16>(cv, f);
      break;
    default:
      if (cv.bits == 4) visit_d<KVQ_FMT_KIVI, 4, BF16>(cv, f);
      else visit_d<KVQ_FMT_KIVI, 2, BF16>(cv, f);
  }
}

// Calls f(Variant<...>{}) for the kernel instantiation that serves cv.
template <class F>
void visit_variant(const CacheView& cv, F&& f) {
  if (cv.bf16) visit_fmt<true>(cv, f);
  else visit_fmt<false>(cv, f);
}

}  // namespace

hipError_t launch_decode(const CacheView& cv, const int32_t* seq_lens, const void* q, float sm_scale, float* out,
                         const DecodeWork& work, const AppendIn* app, hipStream_t stream) {
  const float sm_log2 = sm_scale * kLog2e;
  const AppendIn ap = app ? *app : AppendIn{nullptr, nullptr, nullptr};
  visit_variant(cv, [&](auto v) {
    using V = decltype(v);
    const dim3 grid(unsigned(work.nitems));  // one workgroup per item
    if (app)
      decode_split<V::FMT, V::BITS, V::D, V::G, V::BF16, true><<<grid, kThreads, 0, stream>>>(
          cv, ap.seq_lens, q, sm_log2, out, work, ap);
    else
      decode_split<V::FMT, V::BITS, V::D, V::G, V::BF16, false><<<grid, kThreads, 0, stream>>>(
          cv, seq_lens, q, sm_log2, out, work, ap);
  });
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// The fixed workspace of kvq_append_decode_noalloc: a file-scope device
// array, so that callers that cannot allocate (graph capture, serving loops)
// still have the arrival counters and partial states the split-K decode
// needs. Each device the library runs on holds its own copy for the life of
// the process. In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is passed on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

__global__ __launch_bounds__(256) void clear_words(uint32_t* __restrict__ p, int n) {
  for (int i = int(blockIdx.x) * 256 + int(threadIdx.x); i < n; i += int(gridDim.x) * 256) p[i] = 0u;
}
}  // namespace

hipError_t static_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_clear_words(uint32_t* p, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int blocks = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  clear_words<<<blocks, 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

int decode_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

int decode_resident_workgroups(const CacheView& cv) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  hipError_t e = hipSuccess;
  visit_variant(cv, [&](auto v) {
    using V = decltype(v);
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, decode_split<V::FMT, V::BITS, V::D, V::G, V::BF16, false>, kThreads, 0);
  });
  if (e != hipSuccess) return 0;
  return cus * per_cu;
}

}  // namespace kvq
