// Register-level helpers shared by the MFMA kernels (gfx950).
#pragma once

#include "bf_common.h"

namespace bifocal {

// R(-n) with the table entry (cos, sin) of n: (x1, x2) -> (x1 c + x2 s, x2 c - x1 s).
// Written with explicit roundings so that every caller gets identical bits.  The empty
// asm pins the float32 results: without it the compiler may fold "fma, then convert to
// fp16" into one mixed-precision FMA that rounds once, straight to fp16, at some call
// sites and not at others, and the hi/lo split must see the very hi value the main
// operand carries.
__device__ __forceinline__ void rot_neg(float x1, float x2, float c, float s, float& y1,
                                        float& y2) {
  y1 = __fmaf_rn(x1, c, __fmul_rn(x2, s));
  y2 = __fmaf_rn(x2, c, -__fmul_rn(x1, s));
  asm volatile("" : "+v"(y1), "+v"(y2));
}

// fp16 hi part and the fp16 remainder, from the same conversion as the main remote
// operands (pack_f16), so the correction completes exactly the hi value they carry.
__device__ __forceinline__ void split_f16(float y, uint32_t& hi, uint32_t& lo) {
  hi = f16_bits_of(y);
  const float hf = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
  lo = f16_bits_of(y - hf);
}

// max(x[l], x[l ^ 32]) in every lane l: the two 32-lane halves of a wave exchanged with
// v_permlane32_swap (no LDS round trip, no wait on the wave's outstanding LDS reads).
__device__ __forceinline__ float max_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_at(const uint4& w, int e) {
  const uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}

// One 16-byte LDS-DMA transfer per lane: lane l's 16 bytes land at dst + 16 l (dst
// wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0,
                                   0);
}
// The same from a wave-uniform base plus a 32-bit lane offset.  The empty asm keeps the
// offset's zero extension next to the add, so the transfer takes the scalar-base form
// instead of a 64-bit vector address computed per transfer.
__device__ __forceinline__ void dma16_at(const uint8_t* base, uint32_t off, void* lds_dst) {
  asm volatile("" : "+v"(off));
  dma16(base + off, lds_dst);
}

}  // namespace bifocal
