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

// Device error bit (LLM_DEVERR_RANGE in llm.h): a value stored as fp16 was outside fp16's
// finite range (it became +-inf) or was not a number.
constexpr int LLM_DEVERR_RANGE_BIT = 8;
// Device error bit (LLM_DEVERR_SYNC in llm.h): a bounded wait inside a kernel gave up.
constexpr int LLM_DEVERR_SYNC_BIT = 16;

// True when fp16(v) is not finite: |v| rounds past the largest fp16 value (65504) or v is NaN.
__device__ __forceinline__ bool f16_out_of_range(float v) { return !(__builtin_fabsf(v) < 65520.0f); }

// Greedy-argmax key of logit v at index i: the unsigned order of keys is the order "higher logit,
// then lower index", the one the argmax kernels use, so the row's argmax is the maximum key (an
// atomicMax).  The high word maps the float to an order-preserving integer (-0 taken as +0, so
// that a tie of the two zeros goes to the lower index as a float compare has it), the low word
// is ~i.  A NaN logit gets key 0 and is never chosen; 0 also means "no key yet".
__device__ __forceinline__ unsigned long long argmax_key(float v, int i) {
  if (v != v) return 0ull;
  const uint32_t b = __float_as_uint(v + 0.0f);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)~(uint32_t)i;
}

// Range check of a value about to be stored in the activation dtype (only fp16 can overflow).
template <typename T> __device__ __forceinline__ bool store_out_of_range(float v) {
  if constexpr (__is_same(T, f16_t)) return f16_out_of_range(v);
  else return false;
}

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

// One DPP data move of a float across the lanes of a wave (rows of 16 lanes); lanes of rows
// outside ROWS, and lanes whose source is outside the row, receive 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf, false));
}

// Sum over the 64 lanes of a wave, returned to every lane.  The adds run on DPP moves (within
// quads, rotations within each 16-lane row, then the row broadcasts that carry lane 15 into the
// next row and lane 31 into rows 2 and 3), which leave the total in lane 63; one readlane hands it
// to the wave.  A butterfly of ds_bpermute shuffles took six LDS round trips in series instead.
// Call with every lane of the wave active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_move<0xB1>(v);        // quad_perm [1, 0, 3, 2]: pairs
  v += dpp_move<0x4E>(v);        // quad_perm [2, 3, 0, 1]: quads
  v += dpp_move<0x124>(v);       // row_ror:4: two quads
  v += dpp_move<0x128>(v);       // row_ror:8: the whole row of 16
  v += dpp_move<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3: rows 0 + 1, rows 2 + 3
  v += dpp_move<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: row 3 holds the total
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
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

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding).
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte-per-lane global -> LDS DMA from base + byte_off (uniform base, per-lane 32-bit
// offset; lane l's bytes land at lds + 16 l), in asm so that the
// compiler does not count it among the LDS operations: with the builtin, every later fragment
// wait becomes a wait for all LDS reads.  Completion is tracked by the callers' explicit
// vector-memory waits, and one wait state follows the M0 write.  The compiler reserves M0 and
// need not honour it on a clobber list, so this is for kernels in which nothing else uses M0:
// the kernels that use it (the 64-wide-stage GEMM, the prefill attention) have no other M0 access.
// tests/test_isa_m0.py compiles the sources and fails if the compiler ever emits an M0 access of
// its own in a function that holds this asm.
__device__ __forceinline__ void dma16_asm(const f16_t* base, unsigned byte_off, const f16_t* lds) {
  const unsigned lds_addr =
      __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(const void __attribute__((address_space(3)))*)lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(byte_off), "s"(base),
               "s"(lds_addr)
               : "memory", "m0");
}

}  // namespace llm
