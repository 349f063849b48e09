// Wave-level building blocks of the decode kernels (gfx950, wave64): the
// cross-lane exchanges of the score and probability operands and the exact
// conversions of FP8-pattern bytes. They sit in a header of their own so
// that a GPU unit test can check each lane map and conversion against its
// definition.
//
// DPP controls used here (lanes within a 16-lane row, rows of a wave64):
//  0xb1 quad_perm [1, 0, 3, 2], 0x4e quad_perm [2, 3, 0, 1], 0x128 row_ror
//  by 8 (lane k of a row reads lane (k + 8) mod 16), 0x141 row_half_mirror
//  (k <-> 7 - k within each half-row), 0x140 row_mirror (k <-> 15 - k).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.h"

namespace kvq {

// Within each 16-lane row: the lanes of the banks in `banks` (bit b = lanes
// 4b..4b+3) take src from the lane 8 places along; the others keep old.
template <int BANKS>
__device__ __forceinline__ uint32_t swap8_into(uint32_t old, uint32_t src) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(src), 0x128, 0xf, BANKS, false));
}

// x + (x of the lane 8 places along the same 16-lane row): adds the hi and
// lo columns of one head.
__device__ __forceinline__ float add_ror8(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false);
  return x + __builtin_bit_cast(float, y);
}
__device__ __forceinline__ float max_ror8(float x) {  // max with the lane 8 places along the row
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false);
  return fmaxf(x, __builtin_bit_cast(float, y));
}
__device__ __forceinline__ float max_rows(float x) {  // max over lanes l, l^16, l^32, l^48
  x = fmaxf(x, __shfl_xor(x, 16, kWave));
  return fmaxf(x, __shfl_xor(x, 32, kWave));
}
__device__ __forceinline__ float sum_rows(float x) {
  x += __shfl_xor(x, 16, kWave);
  return x + __shfl_xor(x, 32, kWave);
}
// Maximum over lanes 0-31, wave-uniform, without LDS traffic, of the bit
// patterns of non-negative floats (+0 included), whose unsigned order is
// the order of the values: quad swaps, the half-row and row mirrors leave
// each 16-lane row holding its maximum (every step one integer maximum,
// with no NaN quieting of the exchanged values); lanes 0 and 16 then give
// the two rows' maxima.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
  const uint32_t y = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xf, 0xf, false));
  return v > y ? v : y;
}
__device__ __forceinline__ uint32_t max_lanes32_bits(uint32_t x) {
  x = umax_dpp<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x = umax_dpp<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x = umax_dpp<0x141>(x);  // row_half_mirror
  x = umax_dpp<0x140>(x);  // row_mirror
  const uint32_t r0 = uint32_t(__builtin_amdgcn_readlane(int(x), 0));
  const uint32_t r1 = uint32_t(__builtin_amdgcn_readlane(int(x), 16));
  return r0 > r1 ? r0 : r1;
}

// FP8 E4M3 byte pair (bytes 2*sel, 2*sel+1 of w) to a bf16 pair, exact.
template <int SEL>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, SEL != 0));
}
// Bytes 2 SEL, 2 SEL + 1 of w as an f16 pair, exact, for bytes holding an
// integer c in 0..15: such a byte is the E4M3 pattern of c * 2^-9 (the
// subnormals 1..7 continue evenly into the first normal binade 8..15), and
// the conversion's scale 2^9 restores c.
template <int SEL>
__device__ __forceinline__ uint32_t e4m3_pair_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 512.0f, SEL != 0));
}
// Byte SEL of w as an f16 pair, exact, for a byte whose two nibbles hold
// integers c in 0..3 (upper two bits of each nibble zero): such a nibble is
// the FP4 E2M1 pattern of c / 2 (the subnormal 0.5 continues evenly into
// 1.0 and 1.5), and the conversion's scale 2 restores c. The low half holds
// the low nibble.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, SEL));
}

// x minus one half of a bf16 pair, exactly, in one instruction: the bf16 dot
// product pair . unit + x, with unit the bf16 pair (-1, 0) (low half) or
// (0, -1) (high half) held in a register. The units come from bf16_units()
// as register values the compiler cannot see through: given as constants,
// the compiler encodes (-1, 0) as the inline constant -1.0, which the
// instruction reads as the 32-bit pattern of -1.0f, i.e. the pair (0, -1)
// (every lane of a GPU probe came out wrong; with register units every lane
// is exact).
struct Bf16Units {
  uint32_t lo, hi;  // (-1, 0) and (0, -1)
};
__device__ __forceinline__ Bf16Units bf16_units() {
  Bf16Units u;
  asm volatile("v_mov_b32 %0, 0x0000bf80" : "=v"(u.lo));
  asm volatile("v_mov_b32 %0, 0xbf800000" : "=v"(u.hi));
  return u;
}
__device__ __forceinline__ float sub_bf16_half(uint32_t pair, uint32_t unit, float x) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, pair), __builtin_bit_cast(b2, unit), x, false);
}

}  // namespace kvq
