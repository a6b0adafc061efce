// Device-side building blocks shared by the W4A16 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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

// Wait until at most N of this wave's vector-memory operations are outstanding; they
// complete in issue order, so this is the wait for everything issued before the last N.
// Direct-to-LDS loads count here too, and the compiler does not wait for them by itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7 = none), lgkmcnt 11:8.
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

// ---- bf16 activations -------------------------------------------------------------------
// gfx950 has bf16 MFMAs but no packed bf16 add, so the dequant forms (q - z) in fp32 and
// packs pairs with v_cvt_pk_bf16_f32 (exact: |q - z| <= 15 needs 4 significant bits).  A
// nibble at bits 4j..4j+3 OR-ed into the mantissa of 2^(23 - 4j) gives 2^(23 - 4j) + q
// (the nibble's unit is then the ulp), and subtracting 2^(23 - 4j) + z leaves q - z.
struct ZeroOffsetsBf {
  float o[4];  // 2^(23 - 4j) + z, j = 0..3
};

__device__ __forceinline__ ZeroOffsetsBf zero_offsets_bf(int z) {
  const float fz = (float)z;
  return ZeroOffsetsBf{{0x1p23f + fz, 0x1p19f + fz, 0x1p15f + fz, 0x1p11f + fz}};
}

// The four exponent patterns in VGPRs (so that mask-and-pattern folds into v_and_or_b32).
struct MagicRegsBf {
  uint32_t m[4];
};

__device__ __forceinline__ MagicRegsBf magic_regs_bf() {
  MagicRegsBf r;
  asm volatile("v_mov_b32 %0, 0x4b000000" : "=v"(r.m[0]));
  asm volatile("v_mov_b32 %0, 0x49000000" : "=v"(r.m[1]));
  asm volatile("v_mov_b32 %0, 0x47000000" : "=v"(r.m[2]));
  asm volatile("v_mov_b32 %0, 0x45000000" : "=v"(r.m[3]));
  return r;
}

// One layout word -> the eight values (q - z) of its rows, in row order, as bf16 (rows 2j
// and 2j + 1 are nibbles j and j + 4, at bits 4j of the word and of its upper half).
__device__ __forceinline__ bf16x8 dequant8_bf(uint32_t w, ZeroOffsetsBf zo, MagicRegsBf mr) {
  const uint32_t w16 = w >> 16;
  bf16x8 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t mask = 0xFu << (4 * j);
    const float lo = __builtin_bit_cast(float, (w & mask) | mr.m[j]) - zo.o[j];
    const float hi = __builtin_bit_cast(float, (w16 & mask) | mr.m[j]) - zo.o[j];
    out[2 * j] = (bf16)lo;
    out[2 * j + 1] = (bf16)hi;
  }
  return out;
}

// ---- FP8 (E4M3) weights ------------------------------------------------------------------
// Two layout words (rows 0-3 and 4-7 of a lane's 8-row slice, one byte per row) -> the
// eight weights as fp16, in row order.  gfx950 converts two E4M3 bytes to two fp16 values
// per instruction (scale 1.0); every E4M3 value is exact in fp16.
__device__ __forceinline__ f16x8 dequant8_fp8(uint32_t lo, uint32_t hi) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The same for bf16 activations: two E4M3 bytes to two bf16 values per instruction (exact:
// E4M3 magnitudes need 4 significant bits and lie inside bf16's range).
__device__ __forceinline__ bf16x8 dequant8_fp8_bf(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Biased bf16 dequant for kernels with MFMA to spare: one layout word -> the eight values
// 128 + q of its rows (row order as above), each nibble OR-ed into the mantissa of 128.0
// (bf16 0x4300, whose ulp is 1).  A product with these operands is corrected afterwards
// by subtracting (128 + z) times the product with all-ones operands, the activation sums.
__device__ __forceinline__ bf16x8 dequant8_bf_biased(uint32_t w, uint32_t m128) {
  u32x4 d;
  d[0] = (w & 0x000F000Fu) | m128;
  d[1] = ((w >> 4) & 0x000F000Fu) | m128;
  d[2] = ((w >> 8) & 0x000F000Fu) | m128;
  d[3] = ((w >> 12) & 0x000F000Fu) | m128;
  return __builtin_bit_cast(bf16x8, d);
}

__device__ __forceinline__ uint32_t magic_reg_bf128() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(r));
  return r;
}

// The two activation types behind one interface.  A, scales and outputs are 16-bit values
// of type T; activations travel as raw 16-byte granules (f16x8) until the MFMA.
template <bool BF16>
struct Act;

template <>
struct Act<false> {
  using Zo = ZeroOffsets;
  using Mr = MagicRegs;
  using W8 = f16x8;
  __device__ static Zo zero(int z) { return zero_offsets(z); }
  __device__ static Mr magic() { return magic_regs(); }
  __device__ static W8 dequant(uint32_t w, Zo zo, Mr mr) { return dequant8(w, zo, mr); }
  __device__ static W8 fp8(uint32_t lo, uint32_t hi) { return dequant8_fp8(lo, hi); }
  __device__ static f32x4 mfma16(f16x8 a, W8 b, f32x4 c) { return mfma16x16x32(a, b, c); }
  __device__ static f32x16 mfma32(f16x8 a, W8 b, f32x16 c) { return mfma32x32x16(a, b, c); }
  __device__ static float value(uint16_t bits) {
    return (float)__builtin_bit_cast(f16, bits);
  }
  __device__ static uint16_t round(float v) { return __builtin_bit_cast(uint16_t, (f16)v); }
};

template <>
struct Act<true> {
  using Zo = ZeroOffsetsBf;
  using Mr = MagicRegsBf;
  using W8 = bf16x8;
  __device__ static Zo zero(int z) { return zero_offsets_bf(z); }
  __device__ static Mr magic() { return magic_regs_bf(); }
  __device__ static W8 dequant(uint32_t w, Zo zo, Mr mr) { return dequant8_bf(w, zo, mr); }
  __device__ static W8 fp8(uint32_t lo, uint32_t hi) { return dequant8_fp8_bf(lo, hi); }
  __device__ static f32x4 mfma16(f16x8 a, W8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0,
                                                   0);
  }
  __device__ static f32x16 mfma32(f16x8 a, W8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0,
                                                   0);
  }
  __device__ static float value(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
  }
  __device__ static uint16_t round(float v) { return __builtin_bit_cast(uint16_t, (bf16)v); }
};

}  // namespace wq
