// Device-side building blocks shared by the W4A16 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;  // rows of K per quantization group (one chunk of the layout)

// Per-lane offsets (1024 + z, 64 + z) subtracted from the magic-number halves.
struct ZeroOffsets {
  f16x2 o1024;
  f16x2 o64;
};

__device__ __forceinline__ ZeroOffsets zero_offsets(int z) {
  const f16 a = (f16)(1024 + z);
  const f16 b = (f16)(64 + z);
  return ZeroOffsets{f16x2{a, a}, f16x2{b, b}};
}

// The two exponent patterns of the dequant, held in VGPRs.  gfx9 VOP3 encodings take at
// most one literal or SGPR operand, so with the mask as literal the OR pattern must come
// from a VGPR for (w & mask) | pattern to fold into a single v_and_or_b32.  The inline asm
// keeps the compiler from turning the values back into literals.
struct MagicRegs {
  uint32_t m1024;
  uint32_t m64;
};

__device__ __forceinline__ MagicRegs magic_regs() {
  MagicRegs r;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(r.m1024));
  asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(r.m64));
  return r;
}

// One layout word -> the eight values (q - z) of its rows, in row order, as fp16.
// Slots hold row offsets {0,2,4,6} in nibbles 0..3 and {1,3,5,7} in nibbles 4..7, so a
// 0x000F000F mask picks a pair of rows into the two mantissas; OR-ing the exponent of
// 1024.0 (0x6400, unit ulp) turns nibble q into 1024 + q, and for the nibbles one place
// higher the exponent of 64.0 (0x5400, ulp 1/16) turns (q << 4) into 64 + q.  Subtracting
// 1024 + z (resp. 64 + z) leaves the exact integer q - z in [-15, 15].
__device__ __forceinline__ f16x8 dequant8(uint32_t w, ZeroOffsets zo, MagicRegs mr) {
  const uint32_t w8 = w >> 8;
  const f16x2 p0 = __builtin_bit_cast(f16x2, (w & 0x000F000Fu) | mr.m1024) - zo.o1024;
  const f16x2 p1 = __builtin_bit_cast(f16x2, (w & 0x00F000F0u) | mr.m64) - zo.o64;
  const f16x2 p2 = __builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) | mr.m1024) - zo.o1024;
  const f16x2 p3 = __builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) | mr.m64) - zo.o64;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Zero-point code of column c (0..15) of a 16-column block: two words, 8 codes each.
__device__ __forceinline__ int zero_code(u32x2 zw, int c) {
  const uint32_t w = (c < 8) ? zw[0] : zw[1];
  return (int)((w >> (4 * (c & 7))) & 0xFu);
}

// silu(g) * u = g / (1 + exp(-g)) * u in fp32 (hardware exp and reciprocal), the SwiGLU
// activation of a gate sum g and an up sum u.
__device__ __forceinline__ float silu_times(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u;
}

__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

}  // namespace wq
