// Shared device helpers for libmuon (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon.h"

namespace muon {

typedef unsigned short bf16_t;  // bfloat16 bit pattern in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Wave-wide sum of a double with a fixed butterfly order (deterministic).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dtype(int d) { return d == MUON_F32 || d == MUON_BF16; }
inline size_t dtype_size(int d) { return d == MUON_F32 ? 4 : 2; }
inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MUON_OK : MUON_ELAUNCH;
}

}  // namespace muon
