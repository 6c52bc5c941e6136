// Block-scaled matrix-core helpers shared by the decode scan over token-sliced values and the
// few-query search scan (gfx950: v_mfma_scale_f32_16x16x128_f8f6f4, an fp6 e2m3 A operand
// of 16 x 128 and an fp4 e2m1 B operand of 128 x 16, one E8M0 scale per row and 32-element
// block, fp32 accumulation).
//
// B operands come straight from bit-plane words: a 32-bit plane word w becomes the fp4 B
// operand of 32 contraction indices with one AND per dword, dword D keeping bit D of every
// nibble, so nibble i of dword D is bit 4i + D of w, an e2m1 value 0.5 b, b or 2 b
// (D = 0, 1, 2); for D = 3 the bit lands on the nibble's sign and OR-ing 0001 gives -0.5 s
// (s = 2b - 1).  Scaling the matching A entries by 4, 2, 1, -2 turns every product into
// a (s + 1) or a s; the constant over the first three nibble positions is removed after
// the product.  K index 32 g + p of a block g therefore stands for coordinate
// 32 g + 4 (p % 8) + p / 8.
//
// A operands are integers written as base-16 digits: for each row of weights and
// 32-element block an exponent e from the block's largest magnitude, x = |v| 2^-e in [0, 1),
// digit l of x one row of A stored as d / 2 (exact in e2m3) with the E8M0 block scale
// 2^(e - 4(l + 1) + 1); every block sum is then exact and each row comes out of the product
// in absolute units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_device.h"

namespace tqx {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A (fp6 e2m3 digit rows, E8M0 scale byte `sa` of this lane's row and block) x B (fp4) + C
__device__ __forceinline__ f32x4 mma(const i32x8& a, const i32x4& b, f32x4 c, int sa) {
  const i32x8 bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 2, 4, 0, sa, 0, 127);
}

// fp4 B operand of one plane word (see the header comment); the nibble-sign dword gives -0.5 s:
// (w & 0x88888888) | 0x11111111 as one bitfield insert, `ones` holding 0x11111111
__device__ __forceinline__ i32x4 fp4_of(uint32_t w, uint32_t ones) {
  i32x4 b;
  b[0] = (int)(w & 0x11111111u);
  b[1] = (int)(w & 0x22222222u);
  b[2] = (int)(w & 0x44444444u);
  uint32_t d3;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d3) : "s"(0x88888888u), "v"(w), "v"(ones));
  b[3] = (int)d3;
  return b;
}

// fp4 operand of the XOR of three plane words from theirs: every dword is the XOR of the
// three (the sign dword's 0001 nibbles XOR to 0001 again), one three-input bit operation each
// (truth table 0x96).  Written as instructions: the compiler builds a three-input XOR from two
// two-input ones, and rebuilds this one from the plane words (two instructions per dword).
__device__ __forceinline__ i32x4 fp4_xor3(const i32x4& a, const i32x4& b, const i32x4& c) {
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r[i]) : "v"(a[i]), "v"(b[i]), "v"(c[i]));
  return r;
}

// A row of 32 digits (element p = K index 32 g + p of this lane) as fp6 e2m3 values d / 2,
// from the digits given as f16 bit patterns: half i of dword j is element 2 j + i, its low 4
// bits the digit d (an f16 subnormal, d 2^-24) and bit 15 its sign, so a digit takes a shift
// and mask of the word it sits in and no conversion to float.  The packed conversion divides
// by its scale operand, 2^-23, which gives d / 2 exactly (checked against the f32 form of the
// conversion on every digit and sign).  It writes its first result dwords before it has read
// the last source registers, so the result must not share registers with the sources:
// written as an instruction with an early-clobber result (the compiler's builtin may overlap
// them).
__device__ __forceinline__ i32x8 fp6_row_f16(const u32x16& h) {
  u32x6 r;
  asm volatile("v_cvt_scalef32_pk32_fp6_f16 %0, %1, %2" : "=&v"(r) : "v"(h), "v"(1.1920928955078125e-07f));
  return (i32x8){(int)r[0], (int)r[1], (int)r[2], (int)r[3], (int)r[4], (int)r[5], 0, 0};
}

// Block exponent: e with |x| 2^-e in [0.5, 1); blocks below 2^-80 count as zero (e = -100)
constexpr int kZeroExp = -100;
__device__ __forceinline__ int block_exp(float amax) {
  return amax >= 8.271806125530277e-25f ? __builtin_amdgcn_frexp_expf(amax) : kZeroExp;
}

// E8M0 scale byte of digit row l (digits stored as d / 2) of a block with exponent e:
// 2^(e - 4(l + 1) + 1); zero blocks (all digits 0) get any valid byte
__device__ __forceinline__ int digit_scale(int e, int l) {
  return e == kZeroExp ? 127 : e - 4 * (l + 1) + 128;
}

}  // namespace tqx
