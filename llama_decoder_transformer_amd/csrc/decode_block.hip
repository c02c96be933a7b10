// Batch-1 decode: the attention half of a layer in one launch.
//
// For one new token the q|k|v projection, the attention over the KV cache and the wo
// projection are each far too small to fill the GPU on their own: launched separately,
// each pays a launch gap, a ramp while its first loads are in flight and a tail, and the
// attention (about 2.6 MB of cache at 640 positions) is nothing but latency.  Here they are
// three roles of one grid, in this order of workgroup index:
//
//   [0, nq)            q|k|v GEMV with the RMSNorm fused (QR weight rows per workgroup, as
//                      the stand-alone fp16 GEMV), RoPE and the cache write of the new K/V;
//   [nq, nq + na)      attention: one workgroup per (chunk of DB_CH keys, KV head); it loads
//                      its cached keys and values before the new q exists, then waits for the
//                      q|k|v rows of its KV-head group, computes its chunk on the matrix cores
//                      and leaves a partial; the last chunk of a group to finish merges them;
//   [nq + na, grid)    wo GEMV with the residual add (OR rows per workgroup); it loads its
//                      weight rows and residual values first, then waits for the attention
//                      output of every KV-head group.
//
// Scaled dot-product attention with the causal mask, softmax and the GQA head map are those
// of the "Scaled Dot-Product Attention" and "GQA" sections of the NumPy page; the projections
// and RoPE as in the stand-alone kernels.
//
// Synchronisation.  A workgroup waits only for workgroups of lower index, which the
// dispatcher starts first, so a waiting workgroup never holds a slot that one it waits for
// still needs.  Data that crosses workgroups inside the launch (q, the new K/V row, the chunk
// partials, the attention output) is written and read with device-scope accesses, which are
// coherent across the per-XCD L2 caches; a producer waits for its stores to complete, then one
// thread increments a device-scope counter; a consumer polls the counter
// (thread 0, with sleeps) and then reads.  Every wait is bounded: past DB_SPIN_LIMIT polls it
// gives up, raises LLM_DEVERR_SYNC and carries on, so the grid always drains.  The counters
// (one per 128-byte line) are cleared by the embedding kernel at the start of each decode step.
#include <algorithm>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace llm {

namespace {

constexpr int DB_D = 128;               // head_dim
constexpr int DB_MAXH = 16;             // query heads per KV head (MFMA columns)
constexpr int DB_STEP = 32;             // keys per wave
constexpr int DB_CH = 4 * DB_STEP;      // keys per attention workgroup
constexpr int DB_VLD = DB_D + 16;       // wave V tile row stride (elements)
constexpr int DB_VT = DB_STEP * DB_VLD; // one wave's V tile (elements)
constexpr unsigned DB_SPIN_LIMIT = 1u << 22;
constexpr int DB_MERGE = 8;             // chunk partials per batch of loads in the merge
constexpr int DB_SMEM = 4 * DB_VT * 2 + 2 * 4 * DB_MAXH * 4 + 64;
constexpr float DB_LOG2E = 1.4426950408889634f;

typedef short db_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) db_v4i16 db_lds_v4i16;

// Device-scope (agent) 32-bit accesses: coherent between workgroups on different XCDs within
// one launch (the per-XCD L2 caches are not coherent for ordinary accesses).
__device__ __forceinline__ void st_dev(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 64-bit device-scope loads (8-byte aligned addresses): measured on MI355X, a GEMV-shaped launch
// in which every workgroup also reads a shared 28 KB vector this way took 24.4 us against 22.7
// with plain loads, and 30.6 with 32-bit device-scope loads.
__device__ __forceinline__ uint64_t ld_dev64(const void* p) {
  return __hip_atomic_load((const uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(void* p, float lo, float hi) {
  const uint64_t v = (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
  __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ld_dev2f(const float* p, float& lo, float& hi) {
  const uint64_t v = ld_dev64(p);
  lo = __uint_as_float((uint32_t)v);
  hi = __uint_as_float((uint32_t)(v >> 32));
}
__device__ __forceinline__ u32x4_t ld_dev4(const void* p) {
  const uint64_t a = ld_dev64(p), b = ld_dev64((const char*)p + 8);
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f16x2_t h;
  h.x = (f16_t)a;
  h.y = (f16_t)b;
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ void wait_stores() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's stores have completed
}

// Every thread's device-scope stores complete, then the counter moves by one.
__device__ __forceinline__ void signal(int* cnt) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The attention-done counter, which every wo workgroup waits on, is kept in DB_REP copies on
// consecutive lines, each moved by every signal; a waiter polls copy (its index % DB_REP), so the
// polls spread over that many lines instead of queueing on one (measured at the Llama-3-8B shape,
// positions 512..767: with the 64-bit accesses above, 21.9 us per block against 23.4).
constexpr int DB_REP = 16;
__device__ __forceinline__ void signal_rep(int* cnt) {
  wait_stores();
  __syncthreads();
  if (threadIdx.x < DB_REP)
    __hip_atomic_fetch_add(cnt + threadIdx.x * DB_SYNC_LINE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ const int* rep_copy(const int* cnt) { return cnt + (blockIdx.x % DB_REP) * DB_SYNC_LINE; }

// Until *cnt reaches target (thread 0 polls, the workgroup waits at the barrier), bounded.
__device__ __forceinline__ void wait_count(const int* cnt, int target, int* err) {
  if (threadIdx.x == 0) {
    unsigned n = 0;
    while ((int)ld_dev(cnt) < target) {
      if (++n > DB_SPIN_LIMIT) {
        atomicOr(err, LLM_DEVERR_SYNC_BIT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint2 read_tr(const f16_t* lds_elem) {
  const db_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((db_lds_v4i16*)(lds_elem));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace

// ------------------------------------------------------------------ role 1: q|k|v GEMV
// The fp16 GEMV with the norm fused (one row, QR weight rows per workgroup, 4 waves over
// 512-element chunks of K): residual loads first, then the weights, the norm statistics, the
// dot products; the epilogue rotates each (even, odd) pair and writes it as one device-scope
// 32-bit store.
template <int QR>
__device__ __forceinline__ void qkv_role(const DecodeBlockParams& p, int b, char* smem) {
  constexpr int KW = WAVE * 8;
  float* s_acc = reinterpret_cast<float*>(smem);  // [4][QR]
  float* s_ss = s_acc + 4 * QR;                     // [4]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int K = p.dim, D = DB_D;
  const int n0 = b * QR;
  const int qd = p.H * D, kd = p.G * D, N = qd + 2 * kd;
  const int hpg = p.H / p.G;
  const int grp = n0 < qd ? (n0 / D) / hpg : (n0 < qd + kd ? (n0 - qd) / D : (n0 - qd - kd) / D);

  const int pos = p.row_pos[0], slot = p.row_slot[0];
  const bool ok_row = pos >= 0 && pos < p.max_seq && slot >= 0 && slot < p.n_slots;

  const f16_t* wr[QR];
#pragma unroll
  for (int r = 0; r < QR; ++r) wr[r] = p.wqkv + (size_t)min(n0 + r, N - 1) * K;
  const int nchunks = (K + KW - 1) / KW;
  int kk[2];
  bool ok[2];
  u32x4_t wraw[2][QR];
  auto load_w = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kk[u] = (c0 + 4 * u) * KW + lane * 8;
      ok[u] = kk[u] < K;
      const int kc = min(kk[u], K - 8);
#pragma unroll
      for (int r = 0; r < QR; ++r) wraw[u][r] = *reinterpret_cast<const u32x4_t*>(wr[r] + kc);
    }
  };
  // The epilogue's RoPE factors, fetched ahead of the weights (unconditionally, from clamped
  // indices: no load sits under a branch, so the waits below count only the loads they need).
  const int t = threadIdx.x;
  const int n_pair = n0 + 2 * t;
  const int pos_c = ok_row ? pos : 0;
  const int col_r = n_pair < qd ? n_pair : n_pair - qd;
  const int j_r = (col_r % D) >> 1;
  const float rc_t = p.rope_cos[(size_t)pos_c * (D >> 1) + j_r];
  const float rs_t = p.rope_sin[(size_t)pos_c * (D >> 1) + j_r];
  float xa[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u) load8(p.x + min((wid + 4 * u) * KW + lane * 8, K - 8), xa[u]);
  load_w(min(wid, nchunks - 1));

  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if ((wid + 4 * u) * KW + lane * 8 >= K) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(xa[u][e], xa[u][e], ss);
  }
  for (int c = wid + 8; c < nchunks; c += 4) {
    const int k = c * KW + lane * 8;
    if (k < K) {
      float a[8];
      load8(p.x + k, a);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(a[e], a[e], ss);
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) s_ss[wid] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf((s_ss[0] + s_ss[1] + s_ss[2] + s_ss[3]) / (float)K + p.eps);

  float acc[QR];
#pragma unroll
  for (int r = 0; r < QR; ++r) acc[r] = 0.f;
  bool range_bad = false;
  for (int c0 = wid; c0 < nchunks; c0 += 8) {
    const bool first = c0 == wid;
    if (!first) load_w(c0);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
      float g[8], a[8];
      load8(p.attn_norm + kk[u], g);
      if (first) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = xa[u][e];
      } else {
        load8(p.x + kk[u], a);
      }
      uint32_t ah[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = a[e] * inv * g[e];
        range_bad |= f16_out_of_range(a[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ah[e] = pack2(a[2 * e], a[2 * e + 1]);
#pragma unroll
      for (int r = 0; r < QR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the vector element goes through a scalar first: a bit cast applied to the element
          // itself reads element 0 on this compiler
          const uint32_t wv = wraw[u][r][e];
          acc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ah[e]), __builtin_bit_cast(f16x2_t, wv),
                                          acc[r], false);
        }
    }
  }
#pragma unroll
  for (int r = 0; r < QR; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < QR; ++r) s_acc[wid * QR + r] = acc[r];
  }
  __syncthreads();

  if (t < QR / 2 && n_pair < N) {
    const int r = 2 * t;
    const float v0 = s_acc[r] + s_acc[QR + r] + s_acc[2 * QR + r] + s_acc[3 * QR + r];
    const float v1 = s_acc[r + 1] + s_acc[QR + r + 1] + s_acc[2 * QR + r + 1] + s_acc[3 * QR + r + 1];
    if (ok_row) {
      // RoPE on the pair (2j, 2j + 1) of a q or k head; v rows go through unrotated
      const bool rot = n_pair < qd + kd;
      const float rc = rot ? rc_t : 1.f, rs = rot ? rs_t : 0.f;
      const float o0 = v0 * rc - v1 * rs, o1 = v1 * rc + v0 * rs;
      range_bad |= f16_out_of_range(o0) | f16_out_of_range(o1);
      const uint32_t w = pack2(o0, o1);
      if (n_pair < qd) {
        st_dev(p.q + n_pair, w);
      } else {
        const int kind = n_pair < qd + kd ? 1 : 2;
        const int col = n_pair - qd - (kind == 2 ? kd : 0);
        const int g = col / D, e = col % D;
        f16_t* cache = kind == 1 ? p.kc : p.vc;
        st_dev(cache + (((size_t)slot * p.G + g) * p.max_seq + pos) * D + e, w);
      }
    } else if (t == 0) {
      atomicOr(p.err, (pos < 0 || pos >= p.max_seq) ? 2 : 4);
    }
  }
  if (range_bad) atomicOr(p.err, LLM_DEVERR_RANGE_BIT);
  signal(p.sync + grp * DB_SYNC_LINE);
}

// ------------------------------------------------------------------ role 2: attention
// Workgroup (chunk, KV head g): keys [chunk * 128, ...) of the row's cache, wave w taking 32 of
// them.  Scores S^T = K Q^T take K straight from memory (lane = key row l16, 16 bytes of d) with
// the group's query heads as the MFMA columns; the softmax runs per column; O^T += V^T P^T
// reads V^T through the transposing LDS read from the wave's row-major V tile.
__device__ __forceinline__ void attn_role(const DecodeBlockParams& p, int a, char* smem) {
  constexpr int D = DB_D;
  f16_t* s_v = reinterpret_cast<f16_t*>(smem);                              // [4][DB_VT]
  float* s_m = reinterpret_cast<float*>(smem + 4 * DB_VT * 2);              // [4][16]
  float* s_l = s_m + 4 * DB_MAXH;                                           // [4][16]
  int* s_last = reinterpret_cast<int*>(s_l + 4 * DB_MAXH);
  const int G = p.G, H = p.H, hpg = H / G;
  const int g = a % G, chunk = a / G;
  const int h0 = g * hpg;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int pos = p.row_pos[0], slot = p.row_slot[0];
  int* const ocnt = p.sync + 2 * G * DB_SYNC_LINE;

  if (pos < 0 || pos >= p.max_seq || slot < 0 || slot >= p.n_slots) {
    // no attention for an invalid row: the first chunk of each group writes zeros
    if (chunk == 0) {
      for (int i = tid; i < hpg * D / 2; i += 256) st_dev(p.o + (size_t)h0 * D + 2 * i, 0u);
      signal_rep(ocnt);
    }
    return;
  }
  const int start = chunk * DB_CH;
  if (start > pos) return;
  const int nvalid = pos / DB_CH + 1;
  const int wbeg = start + wid * DB_STEP;
  const int wend = min(pos + 1, wbeg + DB_STEP);  // keys [wbeg, wend) of this wave (maybe none)
  const size_t base = ((size_t)slot * G + g) * (size_t)p.max_seq * D;
  const f16_t* kb = p.kc + base;
  const f16_t* vb = p.vc + base;

  // Cached rows (positions before pos, written by earlier steps) load now; the new row at pos
  // is written by the q|k|v role of this launch and loads after the wait.
  u32x4_t kr[2][4], vr[8];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    const int key = wbeg + kb2 * 16 + l16;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      kr[kb2][s4] = u32x4_t{0u, 0u, 0u, 0u};
      if (key < pos) kr[kb2][s4] = *reinterpret_cast<const u32x4_t*>(kb + (size_t)key * D + s4 * 32 + lg * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = lane + 64 * i, key = wbeg + (idx >> 4), c = idx & 15;
    vr[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (key < pos) vr[i] = *reinterpret_cast<const u32x4_t*>(vb + (size_t)key * D + c * 8);
  }

  wait_count(p.sync + g * DB_SYNC_LINE, p.qkv_per_group, p.err);

  // the new K/V row and the group's q (device-scope loads)
  if (pos >= wbeg && pos < wend) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
      if (wbeg + kb2 * 16 + l16 == pos) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) kr[kb2][s4] = ld_dev4(kb + (size_t)pos * D + s4 * 32 + lg * 8);
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      if (wbeg + (idx >> 4) == pos) vr[i] = ld_dev4(vb + (size_t)pos * D + (idx & 15) * 8);
    }
  }
  f16x8_t qf[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (l16 < hpg) raw = ld_dev4(p.q + (size_t)(h0 + l16) * D + s4 * 32 + lg * 8);
    qf[s4] = __builtin_bit_cast(f16x8_t, raw);
  }

  // one 32-key step per wave
  f16_t* const Vw = s_v + wid * DB_VT;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = lane + 64 * i;
    *reinterpret_cast<u32x4_t*>(&Vw[(idx >> 4) * DB_VLD + (idx & 15) * 8]) = vr[i];
  }
  f32x4_t st[2];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2) {
    st[kb2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
      st[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kr[kb2][s4]), qf[s4], st[kb2], 0,
                                                       0, 0);
  }
  // st[kb][r] = score(key wbeg + 16 kb + 4 lg + r, head l16); keys past wend are masked
  const float scale = DB_LOG2E / sqrtf((float)D);
  float tmax = -INFINITY;
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (wbeg + kb2 * 16 + lg * 4 + r >= wend) st[kb2][r] = -INFINITY;
      tmax = fmaxf(tmax, st[kb2][r]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const float mrow = wend > wbeg ? tmax * scale : -1e30f;  // log2-domain running max of this wave
  float lrow = 0.f;
  float pv[2][4];
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[kb2][r] = __builtin_amdgcn_exp2f(fmaf(st[kb2][r], scale, -mrow));
      lrow += pv[kb2][r];
    }
  const u32x4_t pu = {pack2(pv[0][0], pv[0][1]), pack2(pv[0][2], pv[0][3]), pack2(pv[1][0], pv[1][1]),
                      pack2(pv[1][2], pv[1][3])};
  const f16x8_t pf = __builtin_bit_cast(f16x8_t, pu);
  f32x4_t o[8];
  const f16_t* vlane = Vw + (4 * lg + (l16 >> 2)) * DB_VLD + 4 * (l16 & 3);
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    const uint2 lo = read_tr(vlane + 16 * mb);
    const uint2 hi = read_tr(vlane + 16 * DB_VLD + 16 * mb);
    const u32x4_t u = {lo.x, lo.y, hi.x, hi.y};
    o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, u), pf, f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                   0, 0, 0);
  }
  lrow += __shfl_xor(lrow, 16);
  lrow += __shfl_xor(lrow, 32);

  // merge the 4 waves through LDS: lane (l16, lg) holds head l16, d = 16 mb + 4 lg + r
  __syncthreads();  // every wave is done with its V tile
  float* s_o = reinterpret_cast<float*>(s_v);  // [4][DB_MAXH][D]
  if (l16 < hpg) {
    if (lg == 0) {
      s_m[wid * DB_MAXH + l16] = mrow;
      s_l[wid * DB_MAXH + l16] = lrow;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[((size_t)wid * DB_MAXH + l16) * D + mb * 16 + lg * 4 + r] = o[mb][r];
  }
  __syncthreads();
  // thread: head hh, elements 2 e2, 2 e2 + 1
  const int npairs = hpg * D / 2;
  for (int i = tid; i < npairs; i += 256) {
    const int hh = i / (D / 2), e = 2 * (i % (D / 2));
    float M = s_m[hh];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w * DB_MAXH + hh]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = exp2f(s_m[w * DB_MAXH + hh] - M);
      L += s_l[w * DB_MAXH + hh] * wt;
      a0 += s_o[((size_t)w * DB_MAXH + hh) * D + e] * wt;
      a1 += s_o[((size_t)w * DB_MAXH + hh) * D + e + 1] * wt;
    }
    if (nvalid == 1) {
      st_dev(p.o + (size_t)(h0 + hh) * D + e, pack2(a0 / L, a1 / L));
    } else {
      float* pr = p.partial + ((size_t)(h0 + hh) * p.nch + chunk) * (D + 2);
      // a partial is 130 floats (520 bytes), so every pair below is 8-byte aligned
      st_dev64(pr + e, a0, a1);
      if (e == 0) st_dev64(pr + D, M, L);
    }
  }
  if (nvalid == 1) {
    signal_rep(ocnt);
    return;
  }
  // the last chunk of the group to arrive merges the partials
  wait_stores();
  __syncthreads();
  if (tid == 0)
    *s_last = __hip_atomic_fetch_add(p.sync + (G + g) * DB_SYNC_LINE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              nvalid - 1;
  __syncthreads();
  if (!*s_last) return;
  // The partials are read DB_MERGE chunks at a time, all loads of a batch issued before any is
  // used (device-scope loads go past the L2, so a load-use chain per chunk would cost one
  // memory round trip per chunk).  Indices past the last chunk are clamped and skipped.
  for (int i = tid; i < npairs; i += 256) {
    const int hh = i / (D / 2), e = 2 * (i % (D / 2));
    const float* pr = p.partial + (size_t)(h0 + hh) * p.nch * (D + 2);
    float m = -1e30f, l = 0.f, a0 = 0.f, a1 = 0.f;
    for (int c0 = 0; c0 < nvalid; c0 += DB_MERGE) {
      float mc[DB_MERGE], lc[DB_MERGE], ac0[DB_MERGE], ac1[DB_MERGE];
#pragma unroll
      for (int j = 0; j < DB_MERGE; ++j) {
        const float* pc = pr + (size_t)min(c0 + j, nvalid - 1) * (D + 2);
        ld_dev2f(pc + D, mc[j], lc[j]);
        ld_dev2f(pc + e, ac0[j], ac1[j]);
      }
#pragma unroll
      for (int j = 0; j < DB_MERGE; ++j) {
        if (c0 + j >= nvalid) break;
        const float mn = fmaxf(m, mc[j]);
        const float s0 = exp2f(m - mn), s1 = exp2f(mc[j] - mn);
        l = l * s0 + lc[j] * s1;
        a0 = a0 * s0 + ac0[j] * s1;
        a1 = a1 * s0 + ac1[j] * s1;
        m = mn;
      }
    }
    st_dev(p.o + (size_t)(h0 + hh) * D + e, pack2(a0 / l, a1 / l));
  }
  signal_rep(ocnt);
}

// ------------------------------------------------------------------ role 3: wo GEMV
// x[n0 .. n0 + OR) += o W_o^T: the weight rows and residual values load first; the attention
// output (device-scope loads) once every KV-head group has finished.
template <int OR>
__device__ __forceinline__ void wo_role(const DecodeBlockParams& p, int w, char* smem) {
  constexpr int KW = WAVE * 8;
  float* s_acc = reinterpret_cast<float*>(smem);  // [4][OR]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int K = p.H * DB_D, N = p.dim;
  const int n0 = w * OR;
  const f16_t* wr[OR];
#pragma unroll
  for (int r = 0; r < OR; ++r) wr[r] = p.wo + (size_t)min(n0 + r, N - 1) * K;
  const int nchunks = (K + KW - 1) / KW;
  int kk[2];
  bool ok[2];
  u32x4_t wraw[2][OR];
  auto load_w = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kk[u] = (c0 + 4 * u) * KW + lane * 8;
      ok[u] = kk[u] < K;
      const int kc = min(kk[u], K - 8);
#pragma unroll
      for (int r = 0; r < OR; ++r) wraw[u][r] = *reinterpret_cast<const u32x4_t*>(wr[r] + kc);
    }
  };
  const int t = threadIdx.x;
  float resid = 0.f;
  if (t < OR && n0 + t < N) resid = p.x[n0 + t];
  // Hold the weight stream back a little (wo_delay x 2048 cycles): these workgroups start as q|k|v
  // workgroups retire, and weight loads issued at once would compete with the last q|k|v loads the
  // attention waits for; a few microseconds later they fall into the attention's wait instead.
  for (int i = 0; i < p.wo_delay; ++i) __builtin_amdgcn_s_sleep(32);
  load_w(min(wid, nchunks - 1));

  wait_count(rep_copy(p.sync + 2 * p.G * DB_SYNC_LINE), p.G, p.err);

  float acc[OR];
#pragma unroll
  for (int r = 0; r < OR; ++r) acc[r] = 0.f;
  for (int c0 = wid; c0 < nchunks; c0 += 8) {
    if (c0 != wid) load_w(c0);
    // Both chunks' attention outputs are loaded before either is used, from clamped addresses:
    // with each load under its chunk's bound the compiler waited for the first before issuing
    // the second, two device-scope round trips after the wait instead of one.
    u32x4_t oa[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) oa[u] = ld_dev4(p.o + min(kk[u], K - 8));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
      uint32_t os[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) os[e] = oa[u][e];  // scalars before the bit casts (see qkv_role)
#pragma unroll
      for (int r = 0; r < OR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = wraw[u][r][e];
          acc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, os[e]), __builtin_bit_cast(f16x2_t, wv),
                                          acc[r], false);
        }
    }
  }
#pragma unroll
  for (int r = 0; r < OR; ++r) acc[r] = wave_sum(acc[r]);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < OR; ++r) s_acc[wid * OR + r] = acc[r];
  }
  __syncthreads();
  if (t < OR && n0 + t < N)
    p.x[n0 + t] = resid + s_acc[t] + s_acc[OR + t] + s_acc[2 * OR + t] + s_acc[3 * OR + t];
}

// At most 128 VGPRs (4 waves per SIMD): with the attention role's 37 KB of LDS, 4 workgroups
// per CU, so the q|k|v role's workgroups and the attention's all fit the GPU at once.
template <int QR, int OR>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
decode_block_kernel(DecodeBlockParams p) {
  __shared__ __attribute__((aligned(16))) char smem[DB_SMEM];
  const int b = blockIdx.x;
  if (b < p.nq) qkv_role<QR>(p, b, smem);
  else if (b < p.nq + p.na) attn_role(p, b - p.nq, smem);
  else wo_role<OR>(p, b - p.nq - p.na, smem);
}

constexpr int DB_QR = 8;
constexpr int DB_OR = 8;

bool decode_block_supported(int dtype, int dim, int n_heads, int n_kv_heads) {
  if (dtype != 1 || n_heads % n_kv_heads) return false;
  const int hd = dim / n_heads, hpg = n_heads / n_kv_heads;
  return hd == DB_D && hpg <= DB_MAXH && dim % 8 == 0 && (hd % DB_QR) == 0;
}

// per layer: G group counters (q|k|v rows done), G chunk counters and DB_REP copies of the
// attention-done counter, one 128-byte line each
int decode_block_sync_ints(int n_kv_heads) { return (2 * n_kv_heads + DB_REP) * DB_SYNC_LINE; }

// Workgroups per CU.  The q|k|v workgroups should all run at once and alone at first: the wo
// workgroups (later in dispatch order) then start, and stream their weights, only as q|k|v
// workgroups retire, instead of sharing the bandwidth the attention is waiting on.  So the
// launch asks for as much LDS per workgroup as makes ceil(nq / CUs) workgroups fit a CU (2 to
// 4; 4 is the register limit).  Measured on MI355X at the Llama-3-8B shape (768 q|k|v
// workgroups): 4 per CU let 208 wo workgroups start at once and the block took 26.4 us.
struct DbGeometry {
  int cus = 0, lds_per_cu = 0;
};

static const DbGeometry& db_geometry() {
  static const DbGeometry g = [] {
    DbGeometry r;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
      (void)hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev);
      (void)hipDeviceGetAttribute(&r.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    }
    (void)hipGetLastError();
    if (r.cus <= 0) r.cus = 256;
    if (r.lds_per_cu <= 0) r.lds_per_cu = 160 * 1024;
    return r;
  }();
  return g;
}

void launch_decode_block(DecodeBlockParams p, hipStream_t s) {
  const int D = DB_D;
  const int N = (p.H + 2 * p.G) * D;
  p.nq = N / DB_QR;
  p.nch = (p.max_seq + DB_CH - 1) / DB_CH;
  p.na = p.nch * p.G;
  p.qkv_per_group = (p.H / p.G + 2) * D / DB_QR;
  const int nw = (p.dim + DB_OR - 1) / DB_OR;
  const DbGeometry& geo = db_geometry();
  // wo's weight-stream delay, measured at the Llama-3-8B shape (768 q|k|v workgroups, 256 CUs):
  // 25.1 us per block without, 23.5 / 23.7 / 24.0 us with 3 / 4 / 5 units.  Only q|k|v streams of
  // at least two workgroups per CU run long enough for it to pay.
  p.wo_delay = p.nq >= 2 * geo.cus ? 3 : 0;
  // (at least 2: one workgroup per CU would need more LDS than a launch may take by default)
  const int per_cu = std::max(2, std::min(4, (p.nq + geo.cus - 1) / geo.cus));
  // the smallest LDS size at which per_cu + 1 workgroups no longer fit, in 256-byte units
  size_t lds = ((size_t)geo.lds_per_cu / (per_cu + 1) + 256) & ~(size_t)255;
  lds = std::max(lds, (size_t)DB_SMEM);
  if (lds * per_cu > (size_t)geo.lds_per_cu) lds = DB_SMEM;  // cannot shape it: no padding
  launch_k(decode_block_kernel<DB_QR, DB_OR>, dim3(p.nq + p.na + nw), 256, lds - DB_SMEM, s, p);
}

size_t decode_block_partial_floats(int n_heads, int max_seq) {
  return (size_t)n_heads * ((max_seq + DB_CH - 1) / DB_CH) * (DB_D + 2);
}

}  // namespace llm
