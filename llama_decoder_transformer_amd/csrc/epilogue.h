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
__device__ __forceinline__ void qkv_store(const EpiParams& p, const QkvPrep& q, int m, int n, float v, float vp) {
  if (!q.ok) return;
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
  } else {
    const int col = n - qd - kd;
    const int g = col / d, e = col % d;
    size_t off = (((size_t)q.slot * p.n_kv_heads + g) * p.max_seq + q.pos) * d + e;
    reinterpret_cast<TA*>(p.v_cache)[off] = from_f32<TA>(v);
  }
}

template <typename TA>
__device__ __forceinline__ void epi_qkv(const EpiParams& p, int m, int n, float v, float vp) {
  qkv_store<TA>(p, qkv_prepare(p, m, n), m, n, v, vp);
}

// SwiGLU of one output column c from its gate (w1) and up (w3) values.
template <typename TA>
__device__ __forceinline__ void epi_swiglu(const EpiParams& p, int m, int c, float gate, float up) {
  const float LOG2E = 1.4426950408889634f;
  const float sg = gate / (1.0f + exp2f(-gate * LOG2E));
  reinterpret_cast<TA*>(p.out_act)[(size_t)m * p.ld + c] = from_f32<TA>(sg * up);
}

}  // namespace llm
