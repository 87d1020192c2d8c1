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

// Sum of squares of the 16 bytes of a cache row one lane holds (8 bf16 or 4 f32 values),
// in a fixed order.  A row's squared norm is this summed over its D * sizeof(T) / 16
// lanes with wave_sum_xor; every kernel that stores key norms uses the same two steps.
template <typename T>
__device__ __forceinline__ float sumsq16(u32x4_t v) {
  float ss = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = u2f(v[w] << 16), c = u2f(v[w] & 0xffff0000u);
      ss = fmaf(a, a, ss);
      ss = fmaf(c, c, ss);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float a = u2f(v[w]);
      ss = fmaf(a, a, ss);
    }
  }
  return ss;
}

// Exclusive prefix of v over a block of BLOCK threads; the block total goes to *tot.
// wsum holds BLOCK / 64 + 1 words.
template <int BLOCK>
__device__ __forceinline__ uint32_t block_exscan(uint32_t v, uint32_t* wsum, uint32_t* tot) {
  constexpr int NWV = BLOCK / 64;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (tid < 64) {
    const uint32_t w = tid < NWV ? wsum[tid] : 0u;
    uint32_t s = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(s, o);
      if (tid >= o) s += y;
    }
    if (tid < NWV) wsum[tid] = s - w;  // exclusive
    if (tid == NWV - 1) wsum[NWV] = s;
  }
  __syncthreads();
  const uint32_t res = wsum[wv] + x - v;
  *tot = wsum[NWV];
  __syncthreads();
  return res;
}

}  // namespace sfi
