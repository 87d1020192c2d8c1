// Device-side helpers shared by the SFI kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfi {

constexpr int kWave = 64;
constexpr int kPage = 16;   // positions per cache page == rows per attention tile
constexpr int kMaxG = 16;   // query heads per KV head handled by one MFMA tile

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// Upper 16 bits of two floats packed as two bf16 lanes: lo in bits [0,16), hi in [16,32).
// For floats that hold bf16 values this is exact; otherwise it truncates.
__device__ __forceinline__ uint32_t pack_hi16(float lo, float hi) {
  return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
}

__device__ __forceinline__ float trunc_bf16(float x) { return u2f(f2u(x) & 0xffff0000u); }

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.
// Lane l: A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16], D[4*(l/16)+i][l%16].
__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D = A(16x16) * B(16x16) + C.  Lane l: A[l%16][4*(l/16)+j], B[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4_t mfma16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, a),
                                                   __builtin_bit_cast(bf16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max_xor(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_xor(float v, int width) {
  for (int o = 1; o < width; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace sfi
