// Device-side helpers shared by the gfx950 kernels: vector types for the bf16 MFMA
// operands, the 32x32x16 MFMA, LDS/global tile movers and small math helpers.
//
// MFMA register layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//  * operand A (32 x 16): lane l holds row l % 32 and eight k-slots selected by l / 32;
//  * operand B (16 x 32): lane l holds column l % 32 and the same eight k-slots;
//  * result (32 x 32 fp32, 16 registers): lane l holds column l % 32; register r holds
//    row 8 * (r / 4) + 4 * (l / 32) + r % 4.
// Because A and B share the lane-half -> k-slot assignment, a contraction is correct for
// any consistent mapping of the contracted index onto (lane half, slot); the kernels
// choose that mapping to match the result layout of the previous MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fcp {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint16_t u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8_t, z);
}

// Eight fp32 values -> eight bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8_t to_bf16x8(const float* x) {
  bf16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
  return r;
}

__device__ __forceinline__ float bf16_to_f32(u16 x) {
  return __uint_as_float((uint32_t)x << 16);
}

__device__ __forceinline__ u16 f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(u16, b);
}

// Low halves (element 2w) or high halves (element 2w + 1) of two dwords, packed
// lo | hi << 16 (v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Position of key k inside a transposed tile row, such that the eight keys one lane
// half feeds to a 32x32x16 MFMA (result-layout rows 8*(s/4) + 4*half + s%4 of a 16-key
// chunk, slot s = 0..7) are contiguous: within each 16-key chunk the 4-key groups 1 and
// 2 trade places.
__device__ __forceinline__ int tpos(int k) {
  const int g = (k >> 2) & 3;
  const int pg = (g == 1) ? 2 : (g == 2 ? 1 : g);
  return (k & ~15) | (pg << 2) | (k & 3);
}

}  // namespace fcp
