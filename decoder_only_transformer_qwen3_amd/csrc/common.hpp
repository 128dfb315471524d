// Shared device helpers for the gfx950 kernels: fixed model dimensions,
// bfloat16 bit conversions, MFMA operand vector types and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q3 {

constexpr int C = 1024;        // hidden size
constexpr int HQ = 16;         // query heads
constexpr int HKV = 8;         // key/value heads
constexpr int D = 128;         // head dim
constexpr int I = 3072;        // MLP intermediate size
constexpr int V = 151936;      // vocabulary
constexpr int NL = 28;         // layers
constexpr int MAXPOS = 40960;  // max position
constexpr int QKV_N = (HQ + 2 * HKV) * D;  // 4096
constexpr int QDIM = HQ * D;               // 2048
constexpr int ROPE_HALF = D / 2;           // 64 table columns
constexpr float EPS = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace q3
