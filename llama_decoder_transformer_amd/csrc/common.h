// Device helpers shared by the HIP kernels of the decoder pass (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llm {

typedef uint16_t bf16_t;  // raw bfloat16 bits (weights as supplied by the caller)
typedef _Float16 f16_t;   // compute / storage type of the bf16-weight path
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even narrowing (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Generic element access for the two storage types.
template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }
template <> __device__ __forceinline__ float to_f32<f16_t>(f16_t v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) { return (f16_t)v; }

// Value of lane ^ 1 (the neighbouring column of an MFMA result), via a DPP quad
// permutation [1, 0, 3, 2]: a plain VALU move, no LDS traffic.
__device__ __forceinline__ float lane_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Load 8 consecutive elements as fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16_t* p, float* out) {
  u32x4_t raw = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(raw[i] << 16);
    out[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
  }
}
// 8 fp16 values packed in a 16-byte word, widened to fp32 (exact).  Each 32-bit
// element is copied to a scalar before the bit cast: applying __builtin_bit_cast
// to a vector element directly makes this compiler read element 0 every time.
__device__ __forceinline__ void f16x8_to_f32(const u32x4_t raw, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = raw[i];
    out[2 * i] = (float)__builtin_bit_cast(f16_t, (uint16_t)(w & 0xFFFFu));
    out[2 * i + 1] = (float)__builtin_bit_cast(f16_t, (uint16_t)(w >> 16));
  }
}
__device__ __forceinline__ void load8(const f16_t* p, float* out) {
  f16x8_to_f32(*reinterpret_cast<const u32x4_t*>(p), out);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
}

}  // namespace llm
