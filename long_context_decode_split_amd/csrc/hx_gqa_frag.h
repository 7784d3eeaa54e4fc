// Operand-fragment helpers shared by the GQA attention kernels (gfx950):
// bf16 packing, fp8 / FP4 conversion to bf16 pairs and e8m0 scales.
#pragma once

#include "hx_common.h"

namespace hx {
namespace frag {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ s16x4 as_s16x4(uint32_t lo, uint32_t hi) {
  uint2 t = make_uint2(lo, hi);
  return __builtin_bit_cast(s16x4, t);
}

__device__ __forceinline__ float bf16lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// fp8 e4m3 byte pairs -> packed bf16 (exact: e4m3 values are bf16 values).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two e2m1 codes of byte `sel` -> packed bf16, multiplied by `scale`.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}

// e8m0 byte -> fp32 2^(E-127) by placing E in the fp32 exponent field: one
// shift, no branch.  Exact for E = 1..254; E = 0 (2^-127, elements below
// 3.6e-38 in magnitude) reads as 0 and E = 255 (NaN) as +inf, so such blocks
// give zero resp. non-finite contributions.
// Byte J of w is taken through a sub-dword operand select of the shift, so
// the conversion is one instruction.
template <int J>
__device__ __forceinline__ float e8m0_byte(uint32_t w) {
  uint32_t r;
  if constexpr (J == 0)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(23u), "v"(w));
  else if constexpr (J == 1)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(23u), "v"(w));
  else if constexpr (J == 2)
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(23u), "v"(w));
  else
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(23u), "v"(w));
  return __uint_as_float(r);
}

// Byte j (a constant after unrolling) of w as 2^(byte - 127).
__device__ __forceinline__ float e8m0_sel(uint32_t w, int j) {
  switch (j) {
    case 0: return e8m0_byte<0>(w);
    case 1: return e8m0_byte<1>(w);
    case 2: return e8m0_byte<2>(w);
    default: return e8m0_byte<3>(w);
  }
}

typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;

// Bytes J of two e8m0 words a (low half) and b (high half) as the two 16-bit
// halves of one word: one byte permute.
template <int J>
__device__ __forceinline__ uint32_t e8m0_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, (uint32_t)J | 0x0C00u | ((uint32_t)(4 + J) << 16) | 0x0C000000u);
}

// A bf16 pair p (both halves in [2^-126, 2^9)) times 2^(E_lo - 127) and
// 2^(E_hi - 127) for the e8m0 pair e (e8m0_pair): E is added into each
// half's exponent field (bits 7-14; the sum stays below 2^16, so nothing
// carries into the other half), then 127 is taken off with unsigned
// saturation.  Exactly the product, a product by a power of two, while it is
// a normal bf16; below that range it becomes 0 (or, at exponent 0, P's
// mantissa bits: within 2^-126 of the product).  Products of 2^128 and more
// (scales above 2^119) are not finite, as in the fp32 product.  Three
// instructions for two weights, against two shifts, two multiplies and a
// pack.
__device__ __forceinline__ uint32_t scale_bf16x2_e8m0(uint32_t p, uint32_t e) {
  const u16x2 s = __builtin_bit_cast(u16x2, (e << 7) + p);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(s, (u16x2){0x3F80, 0x3F80}));
}

constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// c + (sum of a packed bf16 pair), in fp32.
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), kOnes2, c, false);
}

}  // namespace frag
}  // namespace hx
