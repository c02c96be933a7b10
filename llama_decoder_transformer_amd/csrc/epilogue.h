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
template <typename TA>
__device__ __forceinline__ void epi_qkv(const EpiParams& p, int m, int n, float v, float vp) {
  int pos, slot;
  if (!epi_row(p, m, pos, slot)) return;
  const int d = p.head_dim;
  const int qd = p.n_heads * d, kd = p.n_kv_heads * d;
  if (n < qd + kd) {
    const int col = n < qd ? n : n - qd;
    const int e = col % d;
    const int j = e >> 1;
    const float c = p.rope_cos[(size_t)pos * (d >> 1) + j];
    const float sn = p.rope_sin[(size_t)pos * (d >> 1) + j];
    const float r = (n & 1) ? (vp * sn + v * c) : (v * c - vp * sn);
    if (n < qd) {
      reinterpret_cast<TA*>(p.out_act)[(size_t)m * p.ld + n] = from_f32<TA>(r);
    } else {
      const int g = col / d;
      size_t off = (((size_t)slot * p.n_kv_heads + g) * p.max_seq + pos) * d + e;
      reinterpret_cast<TA*>(p.k_cache)[off] = from_f32<TA>(r);
    }
  } else {
    const int col = n - qd - kd;
    const int g = col / d, e = col % d;
    size_t off = (((size_t)slot * p.n_kv_heads + g) * p.max_seq + pos) * d + e;
    reinterpret_cast<TA*>(p.v_cache)[off] = from_f32<TA>(v);
  }
}

// SwiGLU of one output column c from its gate (w1) and up (w3) values.
template <typename TA>
__device__ __forceinline__ void epi_swiglu(const EpiParams& p, int m, int c, float gate, float up) {
  const float LOG2E = 1.4426950408889634f;
  const float sg = gate / (1.0f + exp2f(-gate * LOG2E));
  reinterpret_cast<TA*>(p.out_act)[(size_t)m * p.ld + c] = from_f32<TA>(sg * up);
}

}  // namespace llm
