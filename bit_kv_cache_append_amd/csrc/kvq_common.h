// Device helpers shared by the kvq kernels: input widening, DPP lane exchange,
// fp16 / E4M3 conversions.  gfx950, wave64.
#pragma once

#include "kvq_internal.h"

namespace kvq {

// fl32(1/sqrt(128)), the normalisation of the Walsh-Hadamard rotation
#define KVQ_INV_SQRT_D_BITS 0x3DB504F3u

__device__ __forceinline__ float bits_to_f32(uint32_t b) { return __uint_as_float(b); }

// fp16 / bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float widen(uint16_t h, bool bf16) {
  if (bf16) return __uint_as_float(((uint32_t)h) << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> fp16 round-to-nearest-even, saturating to +-65504 (never inf)
__device__ __forceinline__ uint16_t f16_sat_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round-to-nearest-even
  uint16_t b = __builtin_bit_cast(uint16_t, h);
  if ((b & 0x7FFF) == 0x7C00) b = (b & 0x8000) | 0x7BFF;
  return b;
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// DPP quad permutations (within groups of 4 lanes)
#define KVQ_DPP_XOR1 0xB1
#define KVQ_DPP_XOR2 0x4E
// v of another lane of the same row.  Only controls under which every lane reads a lane of
// its own row are used (quad permutations, row mirrors, row rotations), so the fill value
// (0) is never taken; in this form the compiler can read the value through the DPP operand
// of the instruction that uses it (a max or an add) instead of a separate move.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, true);
}

// Non-negative finite fp32 -> OCP E4M3FN code, round-to-nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
  if (v >= 448.0f) return 0x7Eu;
  uint32_t b = __float_as_uint(v);
  int e = (int)(b >> 23) - 127;
  if (e < -6) {  // E4M3 subnormal range: quantum 2^-9, codes 0..8 (8 == smallest normal)
    return (uint32_t)rintf(v * 512.0f);
  }
  uint32_t mant = b & 0x7FFFFFu;
  uint32_t keep = mant >> 20;
  uint32_t rest = mant & 0xFFFFFu;
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 code (non-negative) -> fp32 value (exact)
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  uint32_t e = (c >> 3) & 0xF, m = c & 7;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
}

}  // namespace kvq
