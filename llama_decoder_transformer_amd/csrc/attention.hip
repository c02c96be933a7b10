// Causal grouped-query attention over the KV cache.
//
// Scores are q.k / sqrt(d) over the keys at positions <= the query's position,
// softmax, then the weighted sum of the values; query head h reads KV head
// h / (n_heads / n_kv_heads) ("Scaled Dot-Product Attention" and "GQA" sections
// of the NumPy page; attention / mask / softmax bullets of the Spanish summary).
// Both kernels use the online (running-max) softmax, which reaches the same
// result as the plain softmax; scores are kept in the log2 domain so the
// exponentials are exp2.
//
// Cache layout (per layer, per K/V): [slot][kv_head][max_seq][head_dim].
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace llm {

constexpr float LOG2E_F = 1.4426950408889634f;

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2_t h;
  h.x = (f16_t)a;
  h.y = (f16_t)b;
  return __builtin_bit_cast(uint32_t, h);
}

// ============================================================== split-KV decode
//
// Grid (chunk, kv-head x head-block, row).  A workgroup handles one row (decode
// sequence or prefill token), one KV head, up to 4 of its query heads, and the
// CH keys of one chunk.  Groups of 16 lanes each take 4 keys per round
// (the loads of the next round are issued before the current one is consumed),
// a lane holding d/16 elements (16 bytes for fp16 d = 128).  Each group keeps its own running
// max / sum / accumulator; the groups are merged through LDS.  A row whose keys
// fit one chunk is written out directly; otherwise each chunk writes a partial
// (max, sum, acc[d]) that attn_combine_kernel merges.  (Merging in the last
// workgroup to arrive needs agent-scope fences, which cost more than the extra
// launch on this GPU.)  Short caches with few rows use one 1024-thread
// workgroup per (row, query head) and no merge pass at all.

constexpr int DEC_MAXH = 4;

template <typename T, int EPL>
__device__ __forceinline__ void load_epl(const T* p, float* out) {
  if constexpr (EPL == 8) {
    load8(p, out);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = to_f32<T>(p[e]);
  }
}

// One key row slice of a lane: d/16 elements, kept raw (one 16-byte word for
// fp16 d = 128) from the load until the math so that a round's loads can be in
// flight while the previous round is consumed.
template <typename T, int EPL>
struct KeySlice {
  float v[EPL];
  __device__ __forceinline__ void load(const T* p) { load_epl<T, EPL>(p, v); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = 0.f;
  }
  __device__ __forceinline__ void get(float* o) const {
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = v[e];
  }
};
template <>
struct KeySlice<f16_t, 8> {
  u32x4_t raw;
  __device__ __forceinline__ void load(const f16_t* p) { raw = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ void zero() { raw = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void get(float* o) const { f16x8_to_f32(raw, o); }
};

template <typename T, int D, int NT, int MAXH>
__global__ void __launch_bounds__(NT) attn_decode_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                         const T* __restrict__ vc, const int* __restrict__ row_pos,
                                                         const int* __restrict__ row_slot, int pos0, int slot0,
                                                         int H, int G, int max_seq, int n_slots, int CH, int nchunks,
                                                         int hpb, float* partial, T* __restrict__ out, int* err) {
  constexpr int EPL = D / 16;
  constexpr int NG = NT / 16;                 // groups of 16 lanes
  constexpr int GPP = NG >= 64 ? 8 : NG;      // groups merged per part in the first merge level
  constexpr int PARTS = NG / GPP;
  __shared__ float s_m[NG][MAXH];
  __shared__ float s_l[NG][MAXH];
  __shared__ float s_acc[NG][MAXH][D];
  __shared__ float s_M[MAXH];
  __shared__ float s_pa[PARTS][MAXH][D];
  __shared__ float s_pl[PARTS][MAXH];

  const int chunk = blockIdx.x, gy = blockIdx.y, row = blockIdx.z;
  const int hpg = H / G;
  const int nhb = hpg / hpb;
  const int g = gy / nhb;
  const int h0 = g * hpg + (gy % nhb) * hpb;
  const int tid = threadIdx.x, grp = tid >> 4, gl = tid & 15;
  const int pos = row_pos ? row_pos[row] : pos0 + row;
  const int slot = row_slot ? row_slot[row] : slot0;
  T* orow = out + (size_t)row * H * D;
  if (pos < 0 || pos >= max_seq || slot < 0 || slot >= n_slots) {
    if (chunk == 0) {
      for (int t = tid; t < hpb * D; t += NT) orow[(size_t)h0 * D + t] = from_f32<T>(0.f);
      if (tid == 0) atomicOr(err, (pos < 0 || pos >= max_seq) ? 2 : 4);
    }
    return;
  }
  const int start = chunk * CH;
  if (start > pos) return;
  const int end = min(pos + 1, start + CH);
  const int nvalid = pos / CH + 1;
  const float scale = LOG2E_F / sqrtf((float)D);

  const size_t base = ((size_t)slot * G + g) * (size_t)max_seq * D;
  const T* kb = kc + base;
  const T* vb = vc + base;

  KeySlice<T, EPL> kf[2][4], vf[2][4];
  bool ok[2][4];
  auto fetch = [&](int buf, int r0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = r0 + grp + NG * t;
      ok[buf][t] = j < end;
      if (ok[buf][t]) {
        kf[buf][t].load(kb + (size_t)j * D + gl * EPL);
        vf[buf][t].load(vb + (size_t)j * D + gl * EPL);
      } else {
        kf[buf][t].zero();
        vf[buf][t].zero();
      }
    }
  };
  fetch(0, start);

  float qv[MAXH][EPL];
#pragma unroll
  for (int hh = 0; hh < MAXH; ++hh) {
    if (hh < hpb) {
      load_epl<T, EPL>(q + (size_t)row * H * D + (size_t)(h0 + hh) * D + gl * EPL, qv[hh]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[hh][e] *= scale;
    }
  }
  float mx[MAXH], sm[MAXH], acc[MAXH][EPL];
#pragma unroll
  for (int hh = 0; hh < MAXH; ++hh) {
    mx[hh] = -1e30f;
    sm[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  auto consume = [&](int buf) {
    float kv[4][EPL], vv[4][EPL];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kf[buf][t].get(kv[t]);
      vf[buf][t].get(vv[t]);
    }
#pragma unroll
    for (int hh = 0; hh < MAXH; ++hh) {
      if (hh < hpb) {
        float sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float d = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d = fmaf(qv[hh][e], kv[t][e], d);
          d += __shfl_xor(d, 8);
          d += __shfl_xor(d, 4);
          d += __shfl_xor(d, 2);
          d += __shfl_xor(d, 1);
          sc[t] = ok[buf][t] ? d : -INFINITY;
        }
        const float mloc = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        const float mn = fmaxf(mx[hh], mloc);
        const float alpha = exp2f(mx[hh] - mn);
        float p[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) p[t] = exp2f(sc[t] - mn);
        sm[hh] = sm[hh] * alpha + (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          float a = acc[hh][e] * alpha;
#pragma unroll
          for (int t = 0; t < 4; ++t) a = fmaf(p[t], vv[t][e], a);
          acc[hh][e] = a;
        }
        mx[hh] = mn;
      }
    }
  };

  // Rounds of 4 * NG keys, two register sets: the next round's loads are issued
  // before the current round is consumed.
  for (int r0 = start; r0 < end; r0 += 8 * NG) {
    const bool more1 = r0 + 4 * NG < end;
    if (more1) fetch(1, r0 + 4 * NG);
    consume(0);
    if (!more1) break;
    const bool more2 = r0 + 8 * NG < end;
    if (more2) fetch(0, r0 + 8 * NG);
    consume(1);
    if (!more2) break;
  }

  // Merge the groups: per-head maximum, then PARTS partial sums of GPP groups each,
  // then the parts.
#pragma unroll
  for (int hh = 0; hh < MAXH; ++hh) {
    if (hh < hpb) {
      if (gl == 0) { s_m[grp][hh] = mx[hh]; s_l[grp][hh] = sm[hh]; }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[grp][hh][gl * EPL + e] = acc[hh][e];
    }
  }
  __syncthreads();
  if (tid < 64) {
#pragma unroll
    for (int hh = 0; hh < MAXH; ++hh) {
      if (hh < hpb) {
        const float v = tid < NG ? s_m[tid][hh] : -1e30f;
        const float M = wave_max(v);
        if (tid == 0) s_M[hh] = M;
      }
    }
  }
  __syncthreads();
  for (int t = tid; t < PARTS * hpb * D; t += NT) {
    const int part = t / (hpb * D), rem = t % (hpb * D);
    const int hh = rem / D, e = rem % D;
    const float M = s_M[hh];
    float L = 0.f, a = 0.f;
#pragma unroll 8
    for (int i = part * GPP; i < part * GPP + GPP; ++i) {
      const float w = exp2f(s_m[i][hh] - M);
      L += s_l[i][hh] * w;
      a += s_acc[i][hh][e] * w;
    }
    s_pa[part][hh][e] = a;
    if (e == 0) s_pl[part][hh] = L;
  }
  __syncthreads();
  for (int t = tid; t < hpb * D; t += NT) {
    const int hh = t / D, e = t % D;
    float L = 0.f, a = 0.f;
#pragma unroll
    for (int part = 0; part < PARTS; ++part) {
      L += s_pl[part][hh];
      a += s_pa[part][hh][e];
    }
    if (nvalid == 1) {
      orow[(size_t)(h0 + hh) * D + e] = from_f32<T>(a / L);
    } else {
      float* pr = partial + (((size_t)row * H + h0 + hh) * nchunks + chunk) * (D + 2);
      pr[e] = a;
      if (e == 0) { pr[D] = s_M[hh]; pr[D + 1] = L; }
    }
  }
}

// Merge the chunk partials of one (row, head) when the row spans several chunks:
// o = sum_c acc_c 2^(m_c - M) / sum_c l_c 2^(m_c - M), M = max_c m_c, as a running merge over
// rounds of CB chunks.  Thread e owns output element e.  The first round's loads do not
// depend on the row's position (a chunk past the row's last is loaded and then ignored), so
// they are in flight together with the position load: one memory round trip for short rows.
template <typename T, int D>
__global__ void __launch_bounds__(128) attn_combine_kernel(const float* __restrict__ partial,
                                                           const int* __restrict__ row_pos,
                                                           const int* __restrict__ row_slot, int pos0, int slot0,
                                                           int H, int max_seq, int n_slots, int CH, int nchunks,
                                                           T* __restrict__ out) {
  constexpr int CB = 8;
  const int h = blockIdx.x, row = blockIdx.y, e = threadIdx.x;
  const float* pr = partial + ((size_t)row * H + h) * nchunks * (D + 2);
  float mc[CB], lc[CB], ac[CB];
  auto load_round = [&](int c0) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = c0 + j;
      mc[j] = -1e30f;
      lc[j] = 0.f;
      ac[j] = 0.f;
      if (c < nchunks) {
        mc[j] = pr[(size_t)c * (D + 2) + D];
        lc[j] = pr[(size_t)c * (D + 2) + D + 1];
        if (e < D) ac[j] = pr[(size_t)c * (D + 2) + e];
      }
    }
  };
  load_round(0);
  const int pos = row_pos ? row_pos[row] : pos0 + row;
  const int slot = row_slot ? row_slot[row] : slot0;
  if (pos < 0 || pos >= max_seq || slot < 0 || slot >= n_slots) return;
  const int nv = pos / CH + 1;
  if (nv == 1) return;
  float m = -1e30f, l = 0.f, a = 0.f;
  for (int c0 = 0;; c0 += CB) {
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      if (c0 + j < nv) {
        const float mn = fmaxf(m, mc[j]);
        const float s0 = exp2f(m - mn), s1 = exp2f(mc[j] - mn);
        l = l * s0 + lc[j] * s1;
        a = a * s0 + ac[j] * s1;
        m = mn;
      }
    }
    if (c0 + CB >= nv) break;
    load_round(c0 + CB);
  }
  if (e < D) out[(size_t)row * H * D + (size_t)h * D + e] = from_f32<T>(a / l);
}

int attn_decode_chunk(int rows, int n_kv_heads, int max_seq) {
  int ch = 512;
  while (ch > 64 && (long)rows * n_kv_heads * ((max_seq + ch - 1) / ch) < 2048) ch >>= 1;
  return ch;
}

size_t attn_decode_partial_floats(int rows, int n_heads, int head_dim, int max_seq) {
  const int nch = (max_seq + 63) / 64;
  return (size_t)rows * n_heads * nch * (head_dim + 2);
}

static int dec_hpb(int n_heads, int n_kv_heads) {
  const int hpg = n_heads / n_kv_heads;
  return hpg <= DEC_MAXH ? hpg : DEC_MAXH;
}

// One chunk per row (no merge pass) when the cache is short and there are few rows:
// 1024-thread workgroups, one query head each.
static bool dec_single_pass(int rows, int n_heads, int max_seq) {
  return max_seq <= 1024 && rows * n_heads <= 512;
}

static bool attn_decode_mfma(const f16_t* q, const f16_t* kc, const f16_t* vc, const int* row_pos,
                             const int* row_slot, int pos0, int slot0, int rows, int H, int G, int max_seq,
                             int n_slots, float* partial, f16_t* out, int* err, hipStream_t s);

template <typename T, int D>
static void attn_decode_dispatch(const T* q, const T* kc, const T* vc, const int* row_pos, const int* row_slot,
                                 int pos0, int slot0, int rows, int H, int G, int max_seq, int n_slots,
                                 float* partial, T* out, int* err, hipStream_t s) {
  const int hpg = H / G;
  if constexpr (std::is_same<T, f16_t>::value && D == 128) {
    if (attn_decode_mfma(q, kc, vc, row_pos, row_slot, pos0, slot0, rows, H, G, max_seq, n_slots, partial, out, err,
                         s))
      return;
  }
  if (dec_single_pass(rows, H, max_seq)) {
    dim3 grid(1, H, rows);
    launch_k(attn_decode_kernel<T, D, 1024, 1>, grid, 1024, 0, s, q, kc, vc, row_pos, row_slot, pos0, slot0, H, G, max_seq,
                                                           n_slots, max_seq, 1, 1, partial, out, err);
    return;
  }
  const int CH = attn_decode_chunk(rows, G, max_seq);
  const int nch = (max_seq + CH - 1) / CH;
  const int hpb = dec_hpb(H, G);
  dim3 grid(nch, G * (hpg / hpb), rows);
  launch_k(attn_decode_kernel<T, D, 256, DEC_MAXH>, grid, 256, 0, s, q, kc, vc, row_pos, row_slot, pos0, slot0, H, G,
                                                              max_seq, n_slots, CH, nch, hpb, partial, out, err);
  if (nch > 1)
    launch_k(attn_combine_kernel<T, D>, dim3(H, rows), 128, 0, s, partial, row_pos, row_slot, pos0, slot0,
                                                                            H, max_seq, n_slots, CH, nch, out);
}

void launch_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache, const int* row_pos,
                        const int* row_slot, int pos0, int slot0, int rows, int n_heads, int n_kv_heads,
                        int head_dim, int max_seq, int n_slots, float* partial, void* out, int* err,
                        hipStream_t s) {
  if (rows <= 0) return;
#define LLM_DEC(T, D)                                                                                        \
  attn_decode_dispatch<T, D>((const T*)q, (const T*)k_cache, (const T*)v_cache, row_pos, row_slot, pos0, slot0, \
                             rows, n_heads, n_kv_heads, max_seq, n_slots, partial, (T*)out, err, s)
  if (dtype == 1) {
    if (head_dim == 128) LLM_DEC(f16_t, 128);
    else if (head_dim == 64) LLM_DEC(f16_t, 64);
    else LLM_DEC(f16_t, 48);
  } else {
    if (head_dim == 128) LLM_DEC(float, 128);
    else if (head_dim == 64) LLM_DEC(float, 64);
    else LLM_DEC(float, 48);
  }
#undef LLM_DEC
}

// ============================================================== MFMA prefill
//
// fp16 operands, fp32 accumulation and softmax, head_dim 128.  Grid (query block, kv-head x head-block).  A workgroup
// holds 4 waves; each wave owns 32 queries of one query head, and the waves of a workgroup
// share one KV head so a K/V tile of 64 keys is staged in LDS once for all of them (GQA
// packing: 4 query heads x 32 queries when the group has 4 or more heads).  For one sequence
// the work order is folded (heaviest blocks first in the first half of the grid, lightest
// first in the second), so the two workgroups a CU holds carry an even causal load.
//
// Per 64-key tile a wave computes S^T = K Q^T (keys as MFMA rows, queries as
// columns), so each lane's accumulators all belong to one query column and the
// scaled probabilities, packed to fp16, are already the B operand of
// O^T += V^T P^T (details at the kernel).
//
// A batched prefill runs all its sequences in one launch: the grid's x index is a
// flat list of (sequence, query block) work items, taken from the last (the
// heaviest blocks of the last sequence) to the first, and each workgroup finds its
// sequence by a binary search over the descriptors' first-block indices.
//
// K/V tiles are double-buffered in LDS and arrive by LDS DMA (no registers stage them), K one
// tile ahead of V: while tile t is processed, K(t + 2) and V(t + 1) are in flight, so the scores
// of tile t + 1 can be computed on the matrix cores between tile t's exponentials (a software
// pipeline inside each wave); each wave waits for its own DMA at the end of the tile, and a
// single barrier per tile separates the buffers' uses.  The causal mask is applied
// only on tiles that cross a wave's diagonal, and the running max is raised only
// when a score exceeds it by more than 2^8 (the accumulators are rescaled then,
// for the whole wave at once); between raises the probabilities stay below 256,
// well inside fp16, and the normalised result is the same softmax.

constexpr int PF_D = 128;
constexpr int PF_KT = 64;
constexpr int PF_VLD = PF_D + 16;   // decode V tile row stride: 288 bytes (transposing reads of 8 rows x 32 bytes hit distinct banks)
// Prefill K and V tiles: 64 unpadded rows of 256 bytes (16 chunks of 16 bytes), filled by LDS DMA
// (one instruction fills 4 whole rows, lane l taking physical chunk l % 16 of row l / 16), with
// the chunks permuted per row so that the fragment reads hit distinct banks:
//  - K, chunk c of row r at c ^ pf_kswz(r).  A 16-byte read is served a pair of lane octets at a
//    time, (0-7, 16-23), ...; the S^T fragments put rows r and r + 16 of one chunk in such a pair,
//    so the permutation takes row bits 0-2 and bit 4: 16 distinct chunks, all 64 banks.
//  - V, chunk c of row r at c ^ pf_vswz(r).  A 32-lane half of a transposing read covers 4
//    consecutive rows x 4 chunks; XOR-ing row bits 0-1 into chunk bits 2-3 puts the 4 rows on 4
//    distinct groups of 4 chunks.
constexpr int PF_KTILE = PF_KT * PF_D;  // elements
constexpr int PF_VTILE = PF_KT * PF_D;
constexpr size_t PF_LDS_BYTES = 2 * (size_t)(PF_KTILE + PF_VTILE) * sizeof(f16_t);
__device__ __forceinline__ int pf_kswz(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int pf_vswz(int r) { return (r & 3) << 2; }
constexpr float PF_RESCALE_LOG2 = 8.0f;

typedef short pf_v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) pf_v4i16 pf_lds_v4i16;

__device__ __forceinline__ uint2 pf_read_tr(const f16_t* lds_elem) {
  const pf_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((pf_lds_v4i16*)(lds_elem));
  return __builtin_bit_cast(uint2, v);
}

// The products run on v_mfma_f32_32x32x16_f16 (twice the issue rate of 16x16x32 on this GPU:
// 79 against 88 us at S = 2048, 788 against 876 us at S = 8192).  Per 64-key tile a wave (32
// queries of one head) computes S^T = K Q^T as 2 key blocks x 8 dimension slices of 16: lane l
// holds query l % 32 and keys (e % 4) + 8 (e / 4) + 4 (l / 32) of each 32-key block, so a
// query's 64 scores sit in lanes l and l ^ 32 and the softmax needs one cross-lane step.
// O^T += V^T P^T takes 16 keys per product: k-step t (block t / 2, half t % 2) uses this lane's
// own probabilities e = 8 (t % 2) .. +7 as its B operand, i.e. keys {0..3, 8..11} (lanes < 32)
// and {4..7, 12..15} (lanes >= 32) of the half, and the V^T operand is assembled in that key
// order from row-major V by two transposing LDS reads (ds_read_b64_tr_b16: lane i of a 16-lane
// group receives element i % 4 of the reads of lanes i / 4 + 4 j, so lane 4 j + c addresses key j
// of its 4-key run at columns 4 c .. 4 c + 3).
template <int HPW, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_prefill_kernel(const f16_t* __restrict__ q, const f16_t* __restrict__ kc, const f16_t* __restrict__ vc,
                      int slot_arg, int pos0_arg, int S_arg, int H, int G, int max_seq, f16_t* __restrict__ out,
                      const SeqDesc* __restrict__ seqs, int nseq) {
  typedef float f32x16_t __attribute__((ext_vector_type(16)));
  constexpr int QSUB = NW / HPW;  // 32-query sub-blocks per workgroup
  constexpr int QB = 32 * QSUB;
  constexpr int NI = 16 / NW;     // DMA instructions per wave per K (and V) tile: 4 rows each
  static_assert(16 % NW == 0, "the 16 four-row blocks of a tile do not split over the waves");
  extern __shared__ __attribute__((aligned(16))) f16_t pf_smem[];
  f16_t* const Ks0 = pf_smem;
  f16_t* const Vs0 = pf_smem + 2 * PF_KTILE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: its derived values live in scalar registers
  const int l32 = lane & 31, lh = lane >> 5;
  const int hpg = H / G;
  const int nhb = hpg / HPW;
  const int ld_q = H * PF_D;
  int qblk = gridDim.x - 1 - blockIdx.x;
  int ycol = blockIdx.y;
  int slot = slot_arg, pos0 = pos0_arg, S = S_arg;
  if (!seqs) {
    // One sequence: workgroup id (dispatch order) -> (query block, KV-head column) so that the
    // column is id % columns (with 8 KV heads each XCD then holds one head's K/V in its L2) and
    // the query blocks come heaviest first for the first half of the ids and lightest first for
    // the second: a CU that takes ids i and i + half gets blocks n - 1 - r and r, an even load.
    const int ny = gridDim.y, nb = gridDim.x;
    const int id = blockIdx.x + nb * blockIdx.y;
    ycol = id % ny;
    const int rank = id / ny, half = (nb + 1) >> 1;
    qblk = rank < half ? nb - 1 - rank : rank - half;
  }
  if (seqs) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seqs[mid].blk0 <= qblk) lo = mid;
      else hi = mid - 1;
    }
    const SeqDesc sd = seqs[lo];
    qblk -= sd.blk0;
    slot = sd.slot;
    pos0 = sd.start;
    S = sd.n;
    q += (size_t)sd.row0 * ld_q;
    out += (size_t)sd.row0 * ld_q;
  }
  const int g = ycol / nhb;
  const int head = g * hpg + (ycol % nhb) * HPW + (wid % HPW);
  const int qw0 = qblk * QB + 32 * (wid / HPW);
  const int wg_last = min(S, qblk * QB + QB) - 1;
  const int kv_end = pos0 + wg_last + 1;
  const float scale = LOG2E_F / sqrtf((float)PF_D);

  // Q^T fragments (B operand): column = query l32, k = dims 16 s + 8 lh .. +7.
  f16x8_t qf[8];
  {
    const int i = qw0 + l32;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      u32x4_t raw = {0u, 0u, 0u, 0u};
      if (i < S) raw = *reinterpret_cast<const u32x4_t*>(q + (size_t)i * ld_q + head * PF_D + s8 * 16 + lh * 8);
      qf[s8] = __builtin_bit_cast(f16x8_t, raw);
    }
  }

  f32x16_t o[4];  // O^T blocks of 32 dimensions
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[mb][e] = 0.f;
  float mrow = -1e30f, lrow = 0.f;  // this lane's query: running max (log2 domain), partial sum

  const size_t base = ((size_t)slot * G + g) * (size_t)max_seq * PF_D;
  const f16_t* kb = kc + base;
  const f16_t* vb = vc + base;
  const int ntiles = (kv_end + PF_KT - 1) / PF_KT;
  const int wave_first_pos = pos0 + qw0;
  const int wave_last_pos = wave_first_pos + 31;
  const int qpos = wave_first_pos + l32;

  // DMA of the tile at key k0 into buffer buf: this wave's 4-row blocks wid * NI .. + NI - 1 of K
  // and of V.  Rows past kv_end load row kv_end - 1 (finite values; their scores are masked).
  const int d_row = lane >> 4, d_pc = lane & 15;
  auto issue_k = [&](int buf, int k0) __attribute__((always_inline)) {
    f16_t* Ks = Ks0 + buf * PF_KTILE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wid * NI + i, r = blk * 4 + d_row;
      const size_t key = (size_t)min(k0 + r, kv_end - 1);
      dma16_asm(kb, (unsigned)((key * PF_D + ((d_pc ^ pf_kswz(r)) << 3)) * sizeof(f16_t)), Ks + blk * 4 * PF_D);
    }
  };
  auto issue_v = [&](int buf, int k0) __attribute__((always_inline)) {
    f16_t* Vs = Vs0 + buf * PF_VTILE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wid * NI + i, r = blk * 4 + d_row;
      const size_t key = (size_t)min(k0 + r, kv_end - 1);
      dma16_asm(vb, (unsigned)((key * PF_D + ((d_pc ^ pf_vswz(r)) << 3)) * sizeof(f16_t)), Vs + blk * 4 * PF_D);
    }
  };
  auto tile_barrier = [&]() __attribute__((always_inline)) {
    wait_vmcnt<0>();  // this wave's DMA has landed
    __syncthreads();  // every wave's has, and every wave is done with the buffers being refilled next
  };

  // V^T read address of this lane: key row 4 lh + (l % 16) / 4 of a 16-key half, columns
  // 16 ((l / 16) % 2) + 4 (l % 4) of a 32-dimension block, i.e. logical chunk
  // 2 ((l / 16) % 2) + (l % 4) / 2 + 4 mb of block mb, half (l % 2).  Every row a lane reads is
  // 4 lh + (l % 16) / 4 modulo 4, so its chunk permutation is the same for all of them.
  const int v_row = 4 * lh + ((lane & 15) >> 2);
  const int v_c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_sw = pf_vswz(v_row);
  const int v_half = 4 * (lane & 1);

  // S^T of the tile in K buffer kbuf into st (keys as rows, this lane's query as the column).
  auto scores = [&](int kbuf, f32x16_t (&st)[2]) __attribute__((always_inline)) {
    const f16_t* Ks = Ks0 + kbuf * PF_KTILE;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) st[kb2][e] = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int kr = kb2 * 32 + l32;
        const f16x8_t kf = *reinterpret_cast<const f16x8_t*>(&Ks[kr * PF_D + (((2 * s8 + lh) ^ pf_kswz(kr)) << 3)]);
        st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[s8], st[kb2], 0, 0, 0);
      }
    }
  };

  // One 64-key tile t, software-pipelined: on entry sc holds S^T of tile t, K(t + 1) and V(t)
  // have landed.  The DMA of K(t + 2) (into the K buffer tile t used) and V(t + 1) goes out first;
  // then, after the max of tile t, the products S^T of tile t + 1 are interleaved with tile t's
  // exponentials, and O^T += V^T P^T of tile t follows.  The barrier at the end makes K(t + 2)
  // and V(t + 1) visible and frees both buffers that tile t + 1 refills.
  auto body = [&](int t, f32x16_t (&sc)[2], f32x16_t (&sn)[2], auto next_c) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_c)::value;
    const int k0 = t * PF_KT;
    if (t + 2 < ntiles) issue_k(t & 1, k0 + 2 * PF_KT);
    if (NEXT) issue_v((t + 1) & 1, k0 + PF_KT);
    if (k0 <= wave_last_pos) {
      if (k0 + PF_KT - 1 > wave_first_pos) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (k0 + kb2 * 32 + (e & 3) + 8 * (e >> 2) + 4 * lh > qpos) sc[kb2][e] = -INFINITY;
      }
      float mx[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        mx[i] = fmaxf(fmaxf(sc[i >> 2][4 * (i & 3)], sc[i >> 2][4 * (i & 3) + 1]),
                      fmaxf(sc[i >> 2][4 * (i & 3) + 2], sc[i >> 2][4 * (i & 3) + 3]));
#pragma unroll
      for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) mx[i] = fmaxf(mx[i], mx[i + w]);
      float m = fmaxf(mx[0], __shfl_xor(mx[0], 32));
      const float tmax = m * scale;
      if (__any(tmax > mrow + PF_RESCALE_LOG2)) {
        const float mn = fmaxf(mrow, tmax);
        const float alpha = exp2f(mrow - mn);
        mrow = mn;
        lrow *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
      }
      const float mneg = -mrow;
      if (NEXT) scores((t + 1) & 1, sn);
      // P^T operands: k-step t4 = (block t4 / 2, half t4 % 2) holds scores e = 8 (t4 % 2) .. +7.
      f16x8_t pf[4];
      float ls[2] = {0.f, 0.f};
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t pk[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb2][8 * hh + 2 * i], scale, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb2][8 * hh + 2 * i + 1], scale, mneg));
            ls[i & 1] += p0 + p1;
            pk[i] = pack_f16x2(p0, p1);
          }
          const u32x4_t u = {pk[0], pk[1], pk[2], pk[3]};
          pf[2 * kb2 + hh] = __builtin_bit_cast(f16x8_t, u);
        }
      }
      if (NEXT) {
        // 16 fragment reads and 16 products of S^T(t + 1) spread through tile t's exponentials
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // three K fragment reads ahead
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i < 13) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one more read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six vector ALU operations
        }
      }
      lrow += ls[0] + ls[1];
      __builtin_amdgcn_sched_barrier(0);  // O^T += V^T P^T below is scheduled on its own
      // O^T += V^T P^T
      const f16_t* Vs = Vs0 + (t & 1) * PF_VTILE;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const f16_t* vrow = Vs + (16 * t4 + v_row) * PF_D + v_half;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int pc = ((v_c0 + 4 * mb) ^ v_sw) << 3;
          const uint2 lo = pf_read_tr(vrow + pc);
          const uint2 hi = pf_read_tr(vrow + 8 * PF_D + pc);
          const u32x4_t u = {lo.x, lo.y, hi.x, hi.y};
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, u), pf[t4], o[mb], 0, 0, 0);
        }
      }
      // the transposing reads run 4 products ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < 12) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    if (NEXT) tile_barrier();
  };

  // Prologue: K(0), V(0) and K(1) land, S^T(0) is computed, and a barrier frees K buffer 0
  // for K(2).
  f32x16_t sa[2], sb[2];
  issue_k(0, 0);
  issue_v(0, 0);
  if (ntiles > 1) issue_k(1, PF_KT);
  tile_barrier();
  scores(0, sa);
  __syncthreads();

  std::integral_constant<bool, true> yes;
  std::integral_constant<bool, false> no;
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    body(t, sa, sb, yes);
    body(t + 1, sb, sa, yes);
  }
  if (t + 1 < ntiles) {
    body(t, sa, sb, yes);
    body(t + 1, sb, sa, no);
  } else {
    body(t, sa, sb, no);
  }

  // Normalise and store: lane holds dims 32 mb + (e % 4) + 8 (e / 4) + 4 lh of query l32.
  float L = lrow + __shfl_xor(lrow, 32);
  const float inv = 1.0f / L;
  const int i = qw0 + l32;
  if (i < S) {
    f16_t* orow = out + (size_t)i * ld_q + head * PF_D;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        uint2 w;
        w.x = pack_f16x2(o[mb][4 * e4] * inv, o[mb][4 * e4 + 1] * inv);
        w.y = pack_f16x2(o[mb][4 * e4 + 2] * inv, o[mb][4 * e4 + 3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * mb + 8 * e4 + 4 * lh) = w;
      }
  }
}

// ============================================================== MFMA decode
//
// Decode rows (one query per row) with the group's query heads as the columns of
// the matrix-core products (up to 16 heads per KV head).  Grid (chunk, kv-head,
// row); each of the 4 waves takes a contiguous quarter of the chunk's keys in
// steps of 32.  Per step, S^T = K Q^T takes its K operand straight from global
// memory (lane = key row l16, 16 bytes of d), the online softmax runs per head
// column as in the prefill kernel, and O^T += V^T P^T reads V^T through the
// transposing LDS read from a wave-private row-major copy of the step's V rows.
// The next step's K and V rows are loaded while the current step is computed.
// The waves are merged through LDS; a chunk writes its (acc, max, sum) partial
// for attn_combine_kernel, or the output when the row has a single chunk.

constexpr int DM_STEP = 32;  // keys per wave step
constexpr int DM_MAXH = 16;  // query heads per KV head (MFMA columns)

template <int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_decode_mfma_kernel(const f16_t* __restrict__ q, const f16_t* __restrict__ kc, const f16_t* __restrict__ vc,
                        const int* __restrict__ row_pos, const int* __restrict__ row_slot, int pos0, int slot0, int H,
                        int G, int max_seq, int n_slots, int CH, int nchunks, float* __restrict__ partial,
                        f16_t* __restrict__ out, int* err) {
  constexpr int D = PF_D;
  constexpr int NT = 64 * NW;
  constexpr int VT = DM_STEP * PF_VLD;  // elements of one wave's V tile
  // V tiles during the key loop; the wave merge reuses the same bytes afterwards.
  __shared__ __attribute__((aligned(16))) f16_t s_v[NW * VT];
  __shared__ float s_m[NW][DM_MAXH], s_l[NW][DM_MAXH];
  static_assert(NW * DM_MAXH * D * sizeof(float) <= sizeof(s_v), "merge buffer does not fit");

  const int chunk = blockIdx.x, g = blockIdx.y, row = blockIdx.z;
  const int hpg = H / G, h0 = g * hpg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the step loop branches on scalars
  const int l16 = lane & 15, lg = lane >> 4;
  const int pos = row_pos ? row_pos[row] : pos0 + row;
  const int slot = row_slot ? row_slot[row] : slot0;
  f16_t* orow = out + (size_t)row * H * D;
  if (pos < 0 || pos >= max_seq || slot < 0 || slot >= n_slots) {
    if (chunk == 0) {
      for (int t = tid; t < hpg * D; t += NT) orow[(size_t)h0 * D + t] = (f16_t)0.f;
      if (tid == 0) atomicOr(err, (pos < 0 || pos >= max_seq) ? 2 : 4);
    }
    return;
  }
  const int start = chunk * CH;
  if (start > pos) return;
  const int end = min(pos + 1, start + CH);
  const int nvalid = pos / CH + 1;
  const int quarter = CH / NW;
  const int wbeg = start + wid * quarter;
  const int wend = min(end, wbeg + quarter);
  const int nsteps = wend > wbeg ? (wend - wbeg + DM_STEP - 1) / DM_STEP : 0;
  const float scale = LOG2E_F / sqrtf((float)D);

  // Q^T fragments (B operand): column = head l16 of the group, k = 32 s + 8 lg .. +7.
  f16x8_t qf[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
    u32x4_t raw = {0u, 0u, 0u, 0u};
    if (l16 < hpg)
      raw = *reinterpret_cast<const u32x4_t*>(q + (size_t)row * H * D + (size_t)(h0 + l16) * D + s4 * 32 + lg * 8);
    qf[s4] = __builtin_bit_cast(f16x8_t, raw);
  }

  const size_t base = ((size_t)slot * G + g) * (size_t)max_seq * D;
  const f16_t* kb = kc + base;
  const f16_t* vb = vc + base;
  f16_t* const Vw = s_v + wid * VT;

  f32x4_t o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow = -1e30f, lrow = 0.f;

  // Raw rows of one step: K as MFMA A operands (key k0 + 16 kb + l16, d = 32 s + 8 lg), V in
  // copy order (key (lane + 64 i) / 16, 16-byte column (lane + 64 i) % 16).  Every load is
  // unconditional, from a key clamped to wend - 1 (its score is masked and its V row meets a zero
  // probability): with the loads under a branch the compiler could not count them and waited for
  // the next step's loads too (vmcnt(0)) before each step, which undid the prefetch.
  u32x4_t kr[2][2][4], vr[2][8];
  auto fetch = [&](int set, int k0) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = min(k0 + kb2 * 16 + l16, wend - 1);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        kr[set][kb2][s4] = *reinterpret_cast<const u32x4_t*>(kb + (size_t)key * D + s4 * 32 + lg * 8);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i, key = min(k0 + (idx >> 4), wend - 1), c = idx & 15;
      vr[set][i] = *reinterpret_cast<const u32x4_t*>(vb + (size_t)key * D + c * 8);
    }
  };

  auto step = [&](int set, int k0) {
    // V rows of this step into the wave's tile (LDS operations of one wave complete in order,
    // so the transposing reads below see these stores, and the next step's stores follow them).
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      *reinterpret_cast<u32x4_t*>(&Vw[(idx >> 4) * PF_VLD + (idx & 15) * 8]) = vr[set][i];
    }
    f32x4_t st[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      st[kb2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        st[kb2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, kr[set][kb2][s4]), qf[s4],
                                                         st[kb2], 0, 0, 0);
    }
    // st[kb][r] = score(key k0 + 16 kb + 4 lg + r, head l16); keys past wend are masked.
    float tmax = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + kb2 * 16 + lg * 4 + r >= wend) st[kb2][r] = -INFINITY;
        tmax = fmaxf(tmax, st[kb2][r]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    tmax *= scale;
    if (__any(tmax > mrow + PF_RESCALE_LOG2)) {
      const float mn = fmaxf(mrow, tmax);
      const float alpha = exp2f(mrow - mn);
      mrow = mn;
      lrow *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
    }
    const float mneg = -mrow;
    float p[2][4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb2][r] = __builtin_amdgcn_exp2f(fmaf(st[kb2][r], scale, mneg));
        lrow += p[kb2][r];
      }
    const u32x4_t pu = {pack_f16x2(p[0][0], p[0][1]), pack_f16x2(p[0][2], p[0][3]), pack_f16x2(p[1][0], p[1][1]),
                        pack_f16x2(p[1][2], p[1][3])};
    const f16x8_t pf = __builtin_bit_cast(f16x8_t, pu);
    const f16_t* vlane = Vw + (4 * lg + (l16 >> 2)) * PF_VLD + 4 * (l16 & 3);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const uint2 lo = pf_read_tr(vlane + 16 * mb);
      const uint2 hi = pf_read_tr(vlane + 16 * PF_VLD + 16 * mb);
      const u32x4_t u = {lo.x, lo.y, hi.x, hi.y};
      o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, u), pf, o[mb], 0, 0, 0);
    }
  };

  // The next step's rows are always fetched (past the last step they are clamped copies of row
  // wend - 1 and go unused), so no load sits under a branch.
  if (nsteps > 0) fetch(0, wbeg);
  for (int i = 0; i < nsteps; i += 2) {
    const int k0 = wbeg + i * DM_STEP;
    fetch(1, k0 + DM_STEP);
    step(0, k0);
    if (i + 1 >= nsteps) break;
    fetch(0, k0 + 2 * DM_STEP);
    step(1, k0 + DM_STEP);
  }

  // Merge the 4 waves: lane (l16, lg) holds head l16, d = 16 mb + 4 lg + r.
  lrow += __shfl_xor(lrow, 16);
  lrow += __shfl_xor(lrow, 32);
  __syncthreads();  // every wave is done with its V tile
  float* s_o = reinterpret_cast<float*>(s_v);  // [NW][DM_MAXH][D]
  if (l16 < hpg) {
    if (lg == 0) { s_m[wid][l16] = mrow; s_l[wid][l16] = lrow; }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) s_o[((size_t)wid * DM_MAXH + l16) * D + mb * 16 + lg * 4 + r] = o[mb][r];
  }
  __syncthreads();
  for (int t = tid; t < hpg * D; t += NT) {
    const int hh = t / D, e = t % D;
    float M = s_m[0][hh];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][hh]);
    float L = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = exp2f(s_m[w][hh] - M);
      L += s_l[w][hh] * wt;
      a += s_o[((size_t)w * DM_MAXH + hh) * D + e] * wt;
    }
    if (nvalid == 1) {
      orow[(size_t)(h0 + hh) * D + e] = (f16_t)(a / L);
    } else {
      float* pr = partial + (((size_t)row * H + h0 + hh) * nchunks + chunk) * (D + 2);
      pr[e] = a;
      if (e == 0) { pr[D] = M; pr[D + 1] = L; }
    }
  }
}

// Chunk of the MFMA decode kernel: a multiple of 128 keys (4 waves x 32), halved from 2048
// until rows x kv-heads x chunks reaches 4096 workgroups.  With cached lengths spread over
// U{1024..8192} at 64 rows, 4096 (1024-key chunks) balanced the uneven rows better than 2048
// (attention 240.5 against 245.3 us per layer on MI355X); one row keeps the 128-key floor.
static int dec_mfma_chunk(int rows, int n_kv_heads, int max_seq) {
  int ch = 2048;
  while (ch > 128 && (long)rows * n_kv_heads * ((max_seq + ch - 1) / ch) < 4096) ch >>= 1;
  return ch;
}

static bool attn_decode_mfma(const f16_t* q, const f16_t* kc, const f16_t* vc, const int* row_pos,
                             const int* row_slot, int pos0, int slot0, int rows, int H, int G, int max_seq,
                             int n_slots, float* partial, f16_t* out, int* err, hipStream_t s) {
  const int hpg = H / G;
  if (hpg > DM_MAXH) return false;
  const int CH = dec_mfma_chunk(rows, G, max_seq);
  const int nch = (max_seq + CH - 1) / CH;
  launch_k(attn_decode_mfma_kernel<4>, dim3(nch, G, rows), 256, 0, s, q, kc, vc, row_pos, row_slot, pos0, slot0, H, G, max_seq,
                                                             n_slots, CH, nch, partial, out, err);
  if (nch > 1)
    launch_k(attn_combine_kernel<f16_t, PF_D>, dim3(H, rows), 128, 0, s, 
        partial, row_pos, row_slot, pos0, slot0, H, max_seq, n_slots, CH, nch, out);
  return true;
}

size_t attn_decode_partial_floats_used(int dtype, int rows, int n_heads, int n_kv_heads, int head_dim, int max_seq) {
  if (rows <= 0) return 0;
  int nch = 1;
  if (dtype == 1 && head_dim == PF_D && n_heads / n_kv_heads <= DM_MAXH) {
    const int ch = dec_mfma_chunk(rows, n_kv_heads, max_seq);
    nch = (max_seq + ch - 1) / ch;
  } else if (!dec_single_pass(rows, n_heads, max_seq)) {
    const int ch = attn_decode_chunk(rows, n_kv_heads, max_seq);
    nch = (max_seq + ch - 1) / ch;
  }
  return nch > 1 ? (size_t)rows * n_heads * nch * (head_dim + 2) : 0;
}

bool attn_prefill_supported(int head_dim, int n_heads, int n_kv_heads) {
  if (head_dim != PF_D || n_kv_heads <= 0 || n_heads % n_kv_heads) return false;
  const int hpg = n_heads / n_kv_heads;
  return hpg == 1 || hpg == 2 || hpg % 4 == 0;
}

template <int HPW, int NW>
static void attn_prefill_launch(dim3 grid, hipStream_t s, const f16_t* q, const f16_t* k, const f16_t* v, int slot,
                                  int pos0, int n_tokens, int H, int G, int max_seq, f16_t* out,
                                  const SeqDesc* seqs, int nseq) {
  // The double-buffered tiles exceed the default 64 KiB dynamic LDS limit, raised once (a
  // function-local static is initialised exactly once even with concurrent callers).
  static const hipError_t attr = hipFuncSetAttribute((const void*)attn_prefill_kernel<HPW, NW>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)PF_LDS_BYTES);
  (void)attr;
  launch_k(attn_prefill_kernel<HPW, NW>, grid, 64 * NW, PF_LDS_BYTES, s, q, k, v, slot, pos0, n_tokens, H, G, max_seq,
           out, seqs, nseq);
}

// Waves per workgroup: 4 / hpw sub-blocks of 32 queries share each K/V tile.  With the folded
// work order of a single sequence (two workgroups per CU, a heavy and a light query block) 4 waves
// beat 8 (one workgroup per CU, each as heavy as its causal block): measured on MI355X at the
// Llama-3-8B shape, S = 2048 62-66 us against 74-75 with 8 waves, S = 8192 683 us against 763
// before the fold.
constexpr int PF_WAVES = 4;

int attn_prefill_block_rows(int max_n, int n_heads, int n_kv_heads) {
  (void)max_n;
  const int hpg = n_heads / n_kv_heads;
  const int hpw = hpg >= 4 ? 4 : hpg;
  return 32 * (PF_WAVES / hpw);
}

static void attn_prefill_any(const void* q, const void* k_cache, const void* v_cache, int slot, int pos0,
                             int n_tokens, int max_n, int n_blocks, const SeqDesc* seqs, int nseq, int n_heads,
                             int n_kv_heads, int max_seq, void* out, hipStream_t s) {
  (void)max_n;
  const int hpg = n_heads / n_kv_heads;
  const int hpw = hpg >= 4 ? 4 : hpg;
  dim3 grid(n_blocks, n_kv_heads * (hpg / hpw));
  const f16_t* qq = (const f16_t*)q;
  const f16_t* kk = (const f16_t*)k_cache;
  const f16_t* vv = (const f16_t*)v_cache;
  f16_t* oo = (f16_t*)out;
#define LLM_PF(HPW) \
  attn_prefill_launch<HPW, PF_WAVES>(grid, s, qq, kk, vv, slot, pos0, n_tokens, n_heads, n_kv_heads, max_seq, oo, \
                                     seqs, nseq)
  if (hpw == 4) LLM_PF(4);
  else if (hpw == 2) LLM_PF(2);
  else LLM_PF(1);
#undef LLM_PF
}

void launch_attn_prefill(const void* q, const void* k_cache, const void* v_cache, int slot, int pos0, int n_tokens,
                         int n_heads, int n_kv_heads, int head_dim, int max_seq, void* out, hipStream_t s) {
  if (n_tokens <= 0) return;
  (void)head_dim;
  const int qb = attn_prefill_block_rows(n_tokens, n_heads, n_kv_heads);
  attn_prefill_any(q, k_cache, v_cache, slot, pos0, n_tokens, n_tokens, (n_tokens + qb - 1) / qb, nullptr, 0, n_heads,
                   n_kv_heads, max_seq, out, s);
}

void launch_attn_prefill_varlen(const void* q, const void* k_cache, const void* v_cache, const SeqDesc* seqs,
                                int nseq, int n_blocks, int max_n, int n_heads, int n_kv_heads, int head_dim,
                                int max_seq, void* out, hipStream_t s) {
  if (nseq <= 0 || n_blocks <= 0) return;
  (void)head_dim;
  attn_prefill_any(q, k_cache, v_cache, 0, 0, 0, max_n, n_blocks, seqs, nseq, n_heads, n_kv_heads, max_seq, out, s);
}

}  // namespace llm
