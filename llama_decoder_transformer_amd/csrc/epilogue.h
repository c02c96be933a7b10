// Projection epilogues shared by the MFMA GEMM and the GEMV kernels.
#pragma once
#include "common.h"
#include "launch.h"

namespace llm {

// Position and slot of output row m; false (and an error flag) when out of range.
__device__ __forceinline__ bool epi_row(const EpiParams& p, int m, int& pos, int& slot) {
  pos = p.row_pos ? p.row_pos[m] : p.pos0 + m;
  slot = p.row_slot ? p.row_slot[m] : p.slot0;
  bool ok = true;
  if (pos < 0 || pos >= p.max_seq) { atomicOr(p.err, 2); ok = false; }
  if (slot < 0 || slot >= p.n_slots) { atomicOr(p.err, 4); ok = false; }
  return ok;
}

// One element of the fused q|k|v projection, given its value v and the value vp
// of its RoPE partner column n^1.  Columns [0, H*d) are q, then G*d of k, then
// G*d of v.  RoPE rotates the pair (2j, 2j+1) of a head by pos * theta^(-2j/d):
// (x0, x1) -> (x0 cos - x1 sin, x0 sin + x1 cos).
//
// The inputs that do not depend on v (row position and slot, the rotation's cos
// and sin) are gathered by qkv_prepare, so a kernel can fetch them while its dot
// products are still in flight; qkv_store then writes the element.
//
// The storing helpers below return true when a value written in fp16 left fp16's
// finite range; the kernel ORs these and raises LLM_DEVERR_RANGE once
// (raise_range_error).
struct QkvPrep {
  int pos, slot;
  float c, s;
  bool ok;
};

__device__ __forceinline__ QkvPrep qkv_prepare(const EpiParams& p, int m, int n) {
  QkvPrep q;
  q.c = 1.f;
  q.s = 0.f;
  q.ok = epi_row(p, m, q.pos, q.slot);
  const int d = p.head_dim;
  const int qd = p.n_heads * d, kd = p.n_kv_heads * d;
  if (q.ok && n < qd + kd) {
    const int col = n < qd ? n : n - qd;
    const int j = (col % d) >> 1;
    q.c = p.rope_cos[(size_t)q.pos * (d >> 1) + j];
    q.s = p.rope_sin[(size_t)q.pos * (d >> 1) + j];
  }
  return q;
}

template <typename TA>
__device__ __forceinline__ bool qkv_store(const EpiParams& p, const QkvPrep& q, int m, int n, float v, float vp) {
  if (!q.ok) return false;
  const int d = p.head_dim;
  const int qd = p.n_heads * d, kd = p.n_kv_heads * d;
  if (n < qd + kd) {
    const int col = n < qd ? n : n - qd;
    const int e = col % d;
    const float r = (n & 1) ? (vp * q.s + v * q.c) : (v * q.c - vp * q.s);
    if (n < qd) {
      reinterpret_cast<TA*>(p.out_act)[(size_t)m * p.ld + n] = from_f32<TA>(r);
    } else {
      const int g = col / d;
      size_t off = (((size_t)q.slot * p.n_kv_heads + g) * p.max_seq + q.pos) * d + e;
      reinterpret_cast<TA*>(p.k_cache)[off] = from_f32<TA>(r);
    }
    return store_out_of_range<TA>(r);
  }
  const int col = n - qd - kd;
  const int g = col / d, e = col % d;
  size_t off = (((size_t)q.slot * p.n_kv_heads + g) * p.max_seq + q.pos) * d + e;
  reinterpret_cast<TA*>(p.v_cache)[off] = from_f32<TA>(v);
  return store_out_of_range<TA>(v);
}

template <typename TA>
__device__ __forceinline__ bool epi_qkv(const EpiParams& p, int m, int n, float v, float vp) {
  return qkv_store<TA>(p, qkv_prepare(p, m, n), m, n, v, vp);
}

// One flag write per thread that stored an out-of-range value.
__device__ __forceinline__ void raise_range_error(const EpiParams& p, bool bad) {
  if (bad) atomicOr(p.err, LLM_DEVERR_RANGE_BIT);
}

// Four consecutive columns n .. n + 3 of one row (n % 4 == 0, head_dim % 4 == 0): they share
// the role (q, k or v), head and row, hold RoPE pairs (n, n + 1) and (n + 2, n + 3), and land
// in 4 consecutive fp16 elements of the destination, written as one 8-byte store.
__device__ __forceinline__ bool qkv_store4(const EpiParams& p, int m, int n, const float (&a)[4]) {
  int pos, slot;
  if (!epi_row(p, m, pos, slot)) return false;
  const int d = p.head_dim;
  const int qd = p.n_heads * d, kd = p.n_kv_heads * d;
  const int kind = n < qd ? 0 : (n < qd + kd ? 1 : 2);
  const int col = kind == 0 ? n : (kind == 1 ? n - qd : n - qd - kd);
  const int g = col / d, e = col - g * d;
  float r[4] = {a[0], a[1], a[2], a[3]};
  if (kind < 2) {
    const size_t t = (size_t)pos * (d >> 1) + (e >> 1);
    const float2 c = *reinterpret_cast<const float2*>(p.rope_cos + t);
    const float2 s = *reinterpret_cast<const float2*>(p.rope_sin + t);
    r[0] = a[0] * c.x - a[1] * s.x;
    r[1] = a[1] * c.x + a[0] * s.x;
    r[2] = a[2] * c.y - a[3] * s.y;
    r[3] = a[3] * c.y + a[2] * s.y;
  }
  f16_t* dst = kind == 0 ? reinterpret_cast<f16_t*>(p.out_act) + (size_t)m * p.ld + n
                         : reinterpret_cast<f16_t*>(kind == 1 ? p.k_cache : p.v_cache) +
                               (((size_t)slot * p.n_kv_heads + g) * p.max_seq + pos) * d + e;
  f16x2_t lo, hi;
  lo.x = (f16_t)r[0];
  lo.y = (f16_t)r[1];
  hi.x = (f16_t)r[2];
  hi.y = (f16_t)r[3];
  *reinterpret_cast<uint2*>(dst) = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
  return f16_out_of_range(r[0]) | f16_out_of_range(r[1]) | f16_out_of_range(r[2]) | f16_out_of_range(r[3]);
}

// q|k|v epilogue of an MFMA tile held as acc[FM][FN] (16 x 16 blocks; this lane holds rows
// m_base + 16 i + 4 lg + r of column n_base + 16 jn + l16).  The column's role (q, k or v),
// head, RoPE pair, destination base and row stride depend only on the column, so they are
// decoded once per block column; the rotation is written without branches (sign of the
// partner term from the column parity; cos 1 and sin 0 for v columns).  All lanes must
// call it (the RoPE partner comes from lane ^ 1).  Returns whether a stored value left fp16's range.
//
// STAGED: the rows are a prefill run (positions pos0 + m, slot slot0, ranges checked by the
// caller) and the tile's rows of the RoPE table are staged in s_cos / s_sin (row m at
// (m - m_tile) * d/2).  Otherwise each element validates its row (decode rows carry their
// own position and slot) and reads the global table.
template <int FM, int FN, bool STAGED>
__device__ __forceinline__ bool qkv_tile_epilogue(const EpiParams& p, const f32x4_t (&acc)[FM][FN], int M, int N,
                                                  int m_base, int n_base, int lg, int l16,
                                                  const float* s_cos = nullptr, const float* s_sin = nullptr,
                                                  int m_tile = 0) {
  const int d = p.head_dim, half = d >> 1;
  const int qd = p.n_heads * d, kd = p.n_kv_heads * d;
  bool bad = false;
#pragma unroll
  for (int jn = 0; jn < FN; ++jn) {
    const int n = n_base + jn * 16 + l16;
    const int kind = n < qd ? 0 : (n < qd + kd ? 1 : 2);
    const int col = kind == 0 ? n : (kind == 1 ? n - qd : n - qd - kd);
    const int g = col / d, e = col - g * d;
    const int j = e >> 1;
    const bool rot = kind < 2;
    const float sgn = (n & 1) ? 1.f : -1.f;
    f16_t* const cache = reinterpret_cast<f16_t*>(kind == 1 ? p.k_cache : p.v_cache);
    if constexpr (STAGED) {
      f16_t* const dst = kind == 0
          ? reinterpret_cast<f16_t*>(p.out_act) + n
          : cache + (((size_t)p.slot0 * p.n_kv_heads + g) * p.max_seq + p.pos0) * d + e;
      const size_t rstride = kind == 0 ? (size_t)p.ld : (size_t)d;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[i][jn][r];
          const float vp = lane_xor1(v);
          const int m = m_base + i * 16 + lg * 4 + r;
          if (m < M && n < N) {
            const int t = (m - m_tile) * half + j;
            const float c = rot ? s_cos[t] : 1.f;
            const float sn = rot ? s_sin[t] : 0.f;
            const float o = fmaf(sgn * vp, sn, v * c);
            bad |= f16_out_of_range(o);
            dst[(size_t)m * rstride] = (f16_t)o;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[i][jn][r];
          const float vp = lane_xor1(v);
          const int m = m_base + i * 16 + lg * 4 + r;
          int pos, slot;
          if (m < M && n < N && epi_row(p, m, pos, slot)) {
            const float c = rot ? p.rope_cos[(size_t)pos * half + j] : 1.f;
            const float sn = rot ? p.rope_sin[(size_t)pos * half + j] : 0.f;
            const float o = fmaf(sgn * vp, sn, v * c);
            bad |= f16_out_of_range(o);
            const f16_t out = (f16_t)o;
            if (kind == 0) reinterpret_cast<f16_t*>(p.out_act)[(size_t)m * p.ld + n] = out;
            else cache[(((size_t)slot * p.n_kv_heads + g) * p.max_seq + pos) * d + e] = out;
          }
        }
      }
    }
  }
  return bad;
}

// Residual add of an MFMA tile (layout as in qkv_tile_epilogue): all residual values are
// loaded first, then all sums stored.  Every load is unconditional, from row and column indices
// clamped into the matrix (the sums of clamped elements are never stored): with each load under
// its element's bounds check the compiler waited for every load before issuing the next, one
// memory round trip per element (128 per lane on a 256 x 256 tile).  A wave whose whole block
// lies inside the matrix stores without per-element checks.
template <int FM, int FN>
__device__ __forceinline__ void resid_tile_epilogue(float* out, int ld, f32x4_t (&acc)[FM][FN], int M, int N,
                                                    int m_base, int n_base, int lg, int l16) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float* row = out + (size_t)min(m_base + i * 16 + lg * 4 + r, M - 1) * ld;
#pragma unroll
      for (int jn = 0; jn < FN; ++jn) acc[i][jn][r] += row[min(n_base + jn * 16 + l16, N - 1)];
    }
  if (m_base + FM * 16 <= M && n_base + FN * 16 <= N) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* row = out + (size_t)(m_base + i * 16 + lg * 4 + r) * ld + n_base + l16;
#pragma unroll
        for (int jn = 0; jn < FN; ++jn) row[jn * 16] = acc[i][jn][r];
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m_base + i * 16 + lg * 4 + r, n = n_base + jn * 16 + l16;
        if (m < M && n < N) out[(size_t)m * ld + n] = acc[i][jn][r];
      }
}

// SwiGLU of one output column c from its gate (w1) and up (w3) values.
template <typename TA>
__device__ __forceinline__ bool epi_swiglu(const EpiParams& p, int m, int c, float gate, float up) {
  const float LOG2E = 1.4426950408889634f;
  const float sg = gate * __builtin_amdgcn_rcpf(1.0f + exp2f(-gate * LOG2E));
  const float u = sg * up;
  reinterpret_cast<TA*>(p.out_act)[(size_t)m * p.ld + c] = from_f32<TA>(u);
  return store_out_of_range<TA>(u);
}

}  // namespace llm
