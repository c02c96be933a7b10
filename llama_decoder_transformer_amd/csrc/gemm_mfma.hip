// Projections on the matrix cores: C[m][n] = sum_k A[m][k] * W[n][k] with fp16
// operands and fp32 accumulation, A = activations [M][K], W = weights [N][K]
// (both K-major, so both operands are staged into LDS with 16-byte row loads).
// The bf16 weights are held as fp16 (converted exactly at init) and activations
// are rounded to fp16 rather than bf16: same bytes and MFMA rate, 8x finer
// rounding, which keeps 32 layers within the bf16 parity bar.
//
// Three kernels share the tiling, fragment layout and epilogues: gemm_dma_kernel (the LDS-DMA
// pipeline further below, 32-wide stages) serves every K % 32 == 0 shape but a batch's LM head,
// gemm_dma64_kernel (64-wide stages) takes its 256-row tiles when K % 64 == 0, and the
// register-staged gemm_f16_kernel described here serves the rest.  A fourth, gemm_stream_kernel,
// takes batches of 9 to 64 rows, which stream the weights.  launch_gemm_f16 at the end of the
// file picks the kernel, tiles and K splits per shape.
//
// Tiling: BM x BN output tile per 256-thread workgroup (4 waves as 2 x 2, each
// owning a BM/2 x BN/2 sub-tile), BK = 64 per stage, v_mfma_f32_16x16x32_f16 on
// 16x16 blocks.  A lane feeds row (lane % 16) and the 8 k-values starting at
// 8 * (lane / 16) of a 16x32 block; it receives rows 4 * (lane / 16) + r,
// r = 0..3, of column lane % 16 of the 16x16 result.  The epilogue therefore
// sees RoPE partners (columns 2j, 2j+1) and SwiGLU gate/up pairs (packed columns
// 2c, 2c+1) in lanes l and l ^ 1.
//
// Pipeline: two LDS stages; while the waves run the MFMAs of stage k, the global
// loads of stage k+1 are in flight in registers and are written to the other
// stage afterwards, so each K step needs one barrier.  LDS tiles use an XOR
// swizzle of the 16-byte chunks (lds_off) instead of padding.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin, so the 1-D grid
// index is remapped so that each XCD receives a contiguous run of tiles, ordered
// N-tile-major: the M tiles that share a weight tile run on the same XCD (one L2)
// at about the same time and the weights are fetched from HBM once.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace llm {

constexpr int GEMM_BK = 64;
constexpr int GEMM_LDK = GEMM_BK;  // LDS row = 128 bytes = 8 chunks of 16 bytes

// LDS position of 16-byte chunk c (0..7) of tile row r: rows are not padded;
// the chunk index is XORed with (r / 2) % 8 so that the 16 lanes of a fragment
// read (16 consecutive rows, one chunk) and of a tile store (2 rows, 8 chunks
// each) hit distinct banks.
__device__ __forceinline__ int lds_off(int r, int c) { return r * GEMM_LDK + ((c ^ ((r >> 1) & 7)) << 3); }

template <int BM, int BN, int WGM, int WGN, int EPI, bool SB = false>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_f16_kernel(const f16_t* __restrict__ A,
                                                                  const f16_t* __restrict__ W, int M, int N, int K,
                                                                  int tiles_m, int tiles_n, EpiParams ep,
                                                                  int kb_per) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int BK = GEMM_BK, LDK = GEMM_LDK;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * BK / 8 / NT;  // 16-byte loads per thread per stage
  constexpr int B_LD = BN * BK / 8 / NT;
  static_assert(A_LD >= 1 && B_LD >= 1 && A_LD * NT * 8 == BM * BK && B_LD * NT * 8 == BN * BK,
                "tile does not split evenly over the threads");
  constexpr int STAGE = (BM + BN) * LDK;  // f16 elements per LDS stage

  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  // XCD-aware tile order (see the file header).
  const int T = tiles_m * tiles_n;
  const int id = blockIdx.x;
  const int per = T / 8, rem = T % 8;
  const int xcd = id % 8, j = id / 8;
  const int t = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + j;
  const int tn_idx = t / tiles_m, tm_idx = t % tiles_m;
  const int tm = tm_idx * BM, tn = tn_idx * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int l16 = lane & 15, lg = lane >> 4;

  // The next stage's global loads sit in registers while the current stage is multiplied.
  constexpr int PA = A_LD, PB = B_LD;
  u32x4_t ra[PA], rb[PB];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // Out-of-range rows / columns load from a clamped in-range address and are then
  // replaced by zero with a select, so the loads stay branch-free.
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int idx = tid + i * NT, r = idx >> 3, c = (idx & 7) * 8;
      const int gm = tm + r, gk = k0 + c;
      const bool ok = gm < M && gk < K;
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(A + (size_t)min(gm, M - 1) * K + min(gk, K - 8));
      ra[i] = ok ? v : zero;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int idx = tid + i * NT, r = idx >> 3, c = (idx & 7) * 8;
      const int gn = tn + r, gk = k0 + c;
      const bool ok = gn < N && gk < K;
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(W + (size_t)min(gn, N - 1) * K + min(gk, K - 8));
      rb[i] = ok ? v : zero;
    }
  };
  auto sstore = [&](int stage) {
    f16_t* As = smem + stage * STAGE;
    f16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int idx = tid + i * NT, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&As[lds_off(r, c >> 3)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int idx = tid + i * NT, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&Bs[lds_off(r, c >> 3)]) = rb[i];
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // K range of this workgroup: kb_per steps of BK starting at split blockIdx.y.
  const int kb0 = blockIdx.y * kb_per;
  const int nk = min(kb_per, (K + BK - 1) / BK - kb0);
  const int kbase = kb0 * BK;
  gload(kbase);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const f16_t* As = smem + cur * STAGE;
    const f16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      if (more && ks == 0) gload(kbase + (kt + 1) * BK);
      f16x8_t af[FM], bw[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const f16x8_t*>(&As[lds_off(wm * WM + i * 16 + l16, ks * 4 + lg)]);
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        bw[jn] = *reinterpret_cast<const f16x8_t*>(&Bs[lds_off(wn * WN + jn * 16 + l16, ks * 4 + lg)]);
      // Keep every fragment read of this k-step ahead of its MFMAs (the scheduler
      // otherwise reuses one register set and waits on each read in turn).
      if (SB) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jn = 0; jn < FN; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bw[jn], acc[i][jn], 0, 0, 0);
      if (more && ks == BK / 32 - 1) sstore(cur ^ 1);
    }
    __syncthreads();
  }

  // Epilogue.  A split-K workgroup stores its partial sums to slice blockIdx.y.
  if constexpr (EPI == EPI_QKV) {
    raise_range_error(ep, qkv_tile_epilogue<FM, FN, false>(ep, acc, M, N, tm + wm * WM, tn + wn * WN, lg, l16));
    return;
  }
  float* const out_f32 = ep.out_f32 + (size_t)blockIdx.y * M * ep.ld;
  if constexpr (EPI == EPI_RESID) {
    resid_tile_epilogue<FM, FN>(out_f32, ep.ld, acc, M, N, tm + wm * WM, tn + wn * WN, lg, l16);
    return;
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = tm + wm * WM + i * 16 + lg * 4 + r;
        const int n = tn + wn * WN + jn * 16 + l16;
        const float v = acc[i][jn][r];
        if (EPI == EPI_SWIGLU) {
          const float vp = lane_xor1(v);
          if (m < M && n < N && (n & 1) == 0) bad |= epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
        } else if (m < M && n < N) {
          if (EPI == EPI_STORE_F32) out_f32[(size_t)m * ep.ld + n] = v;
          else out_f32[(size_t)m * ep.ld + n] += v;
        }
      }
    }
  }
  raise_range_error(ep, bad);
}

// ------------------------------------------------------------------ LDS-DMA variant
//
// Same tiling and epilogue, but the global loads go straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at the instruction's LDS
// base + 16 * lane), so no registers stage the tiles and NS stages rotate through
// LDS: one holds the k-step being multiplied (its fragments already in registers),
// one the k-step whose fragments are being read, and NS - 2 are in flight, so a
// stage's loads have NS - 2 k-steps to land.  BK = 32 per stage
// (one MFMA k-step): a tile row is 64 bytes = 4 chunks of 16 bytes, stored at
// chunk c ^ ((r / 2) % 4) so that the 8 lanes of one LDS read cycle (8
// consecutive rows, one chunk) hit distinct banks.  One DMA instruction fills 16
// rows; lane l takes row l / 4 and physical chunk l % 4, i.e. the logical chunk
// (l % 4) ^ ((l / 8) % 4) of that row.  Rows past M or N load a clamped row (their
// results are discarded); K must be a multiple of 32.

constexpr int DS_BK = 32;

// Tile of workgroup `id` for the DMA kernel.  Workgroups are dealt to the 8 XCDs
// round-robin (XCD = id % 8, j = id / 8 is the order within one XCD).  When the N
// tiles split evenly, XCD x owns the band of N tiles [x * tn / 8, (x + 1) * tn / 8),
// walked in groups of GM M tiles: the about 32 workgroups an XCD runs at once then
// cover GM M tiles x a few N tiles, so each A and W k-slice they read is shared in
// that XCD's L2 by several tiles (a column-major walk shares W only, and streams
// all of A once per N tile).  Otherwise: contiguous N-major runs per XCD.
__device__ __forceinline__ void dma_tile_of(int id, int tiles_m, int tiles_n, int& tm_idx, int& tn_idx) {
  constexpr int GM = 8;
  const int xcd = id % 8, j = id / 8;
  if (tiles_n % 8 == 0) {
    const int band = tiles_n / 8;
    const int full = tiles_m / GM, rem = tiles_m % GM;
    const int g = j / (GM * band);
    if (g < full) {
      const int r = j % (GM * band);
      tm_idx = g * GM + r % GM;
      tn_idx = xcd * band + r / GM;
    } else {
      const int r = j - full * GM * band;
      tm_idx = full * GM + r % rem;
      tn_idx = xcd * band + r / rem;
    }
    return;
  }
  const int T = tiles_m * tiles_n;
  const int per = T / 8, rm = T % 8;
  const int t = (xcd < rm ? xcd * (per + 1) : rm * (per + 1) + (xcd - rm) * per) + j;
  tn_idx = t / tiles_m;
  tm_idx = t % tiles_m;
}

__device__ __forceinline__ int ds_off(int r, int c) { return r * DS_BK + ((c ^ ((r >> 1) & 3)) << 3); }


// Epilogue of the DMA kernels: the wave's FM x FN accumulator blocks cover rows m0.. and columns
// n0.. of the BM-row tile starting at row tm; smem holds at least BM x d floats for the RoPE rows.
template <int BM, int FM, int FN, int NW, int EPI>
__device__ __forceinline__ void dma_tile_epilogue(const EpiParams& ep, f32x4_t (&acc)[FM][FN], f16_t* smem, int M, int N,
                                                  int tm, int m0, int n0, int tid, int lg, int l16) {
  if constexpr (EPI == EPI_QKV) {
    // Prefill rows only (positions pos0 + m, slot slot0, ranges checked by the host, and the
    // table rows fit the stage buffers; the launcher sends other q|k|v projections to the
    // register-staged kernel).  The tile stages its rows of the RoPE table (cos and sin, d/2
    // each) in the idle LDS stage buffers with coalesced loads, so the epilogue reads hit LDS.
    const int half = ep.head_dim >> 1;
    __syncthreads();  // every wave is done with the stage buffers
    float* s_cos = reinterpret_cast<float*>(smem);
    float* s_sin = s_cos + BM * half;
    const int n_el = min(BM, M - tm) * half;
    const float* cs = ep.rope_cos + (size_t)(ep.pos0 + tm) * half;  // rows are consecutive positions
    const float* sn = ep.rope_sin + (size_t)(ep.pos0 + tm) * half;
    // UN elements of each table per thread per pass, every load unconditional (index clamped
    // into the tile's rows): with the load under the loop bound, the compiler waited for each
    // pair of loads before the next (32 memory round trips per thread for a 256-row tile).
    constexpr int NT = NW * 64, UN = 8;
    for (int i0 = tid; i0 < n_el; i0 += UN * NT) {
      float c[UN], sv[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int idx = min(i0 + u * NT, n_el - 1);
        c[u] = cs[idx];
        sv[u] = sn[idx];
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int idx = i0 + u * NT;
        if (idx < n_el) {
          s_cos[idx] = c[u];
          s_sin[idx] = sv[u];
        }
      }
    }
    __syncthreads();
    raise_range_error(ep, qkv_tile_epilogue<FM, FN, true>(ep, acc, M, N, m0, n0, lg, l16, s_cos, s_sin, tm));
    return;
  }
  if constexpr (EPI == EPI_RESID) {
    resid_tile_epilogue<FM, FN>(ep.out_f32, ep.ld, acc, M, N, m0, n0, lg, l16);
    return;
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + i * 16 + lg * 4 + r;
        const int n = n0 + jn * 16 + l16;
        const float v = acc[i][jn][r];
        if (EPI == EPI_SWIGLU) {
          const float vp = lane_xor1(v);
          if (m < M && n < N && (n & 1) == 0) bad |= epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
        } else if (m < M && n < N) {
          if (EPI == EPI_STORE_F32) ep.out_f32[(size_t)blockIdx.y * M * ep.ld + (size_t)m * ep.ld + n] = v;
          else ep.out_f32[(size_t)m * ep.ld + n] += v;
        }
      }
    }
  }
  raise_range_error(ep, bad);
}

template <int BM, int BN, int WGM, int WGN, int NS, int EPI, bool SCHED>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_dma_kernel(const f16_t* __restrict__ A,
                                                                  const f16_t* __restrict__ W, int M, int N, int K,
                                                                  int tiles_m, int tiles_n, EpiParams ep,
                                                                  int kb_per) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int STAGE = (BM + BN) * DS_BK;  // f16 elements per stage
  constexpr int NI = (BM + BN) / 16;        // DMA instructions per stage
  constexpr int PW = NI / NW;               // ... per wave
  static_assert(NI % NW == 0, "DMA instructions do not split evenly over the waves");
  static_assert(NS >= 3 && NS <= 8 && (NS - 2) * PW < 64, "stages");

  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  int tm_idx, tn_idx;
  dma_tile_of(blockIdx.x, tiles_m, tiles_n, tm_idx, tn_idx);
  const int tm = tm_idx * BM, tn = tn_idx * BN;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int l16 = lane & 15, lg = lane >> 4;

  // K range of this workgroup: kb_per k-steps starting at split blockIdx.y (all of K unsplit).
  const int kb0 = blockIdx.y * kb_per;
  const int kbase = kb0 * DS_BK;

  // This lane's source row offsets (elements) and logical chunk for each of the wave's DMA instructions.
  const int dr = lane >> 2;
  const int dc = ((lane & 3) ^ ((dr >> 1) & 3)) * 8;
  const f16_t* src[PW];
  int dst_off[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int blk = wid + NW * i;  // 16-row block of the stage: A blocks first, then W blocks
    if (blk < BM / 16) {
      src[i] = A + (size_t)min(tm + blk * 16 + dr, M - 1) * K + kbase + dc;
      dst_off[i] = blk * 16 * DS_BK;
    } else {
      const int b = blk - BM / 16;
      src[i] = W + (size_t)min(tn + b * 16 + dr, N - 1) * K + kbase + dc;
      dst_off[i] = BM * DS_BK + b * 16 * DS_BK;
    }
  }
  auto issue = [&](int stage_buf, int k0) {
    f16_t* base = smem + stage_buf * STAGE;
#pragma unroll
    for (int i = 0; i < PW; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src[i] + k0),
                                       (void __attribute__((address_space(3)))*)(base + dst_off[i]), 16, 0, 0);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragments are double-buffered in registers: the reads of k-step kt+1 are issued
  // before the MFMAs of k-step kt, so the matrix cores do not wait on LDS latency.
  f16x8_t af[2][FM], bw[2][FN];
  auto read_frags = [&](f16x8_t* a, f16x8_t* b, int stage_buf) {
    const f16_t* As = smem + stage_buf * STAGE;
    const f16_t* Bs = As + BM * DS_BK;
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = *reinterpret_cast<const f16x8_t*>(&As[ds_off(wm * WM + i * 16 + l16, lg)]);
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) b[jn] = *reinterpret_cast<const f16x8_t*>(&Bs[ds_off(wn * WN + jn * 16 + l16, lg)]);
  };
  auto mfmas = [&](const f16x8_t* a, const f16x8_t* b) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[jn], acc[i][jn], 0, 0, 0);
  };
  // Stage st's loads are complete once at most min(depth, nk - 1 - st) later stages are
  // outstanding, depth being the number of stages issued after st so far; after every wave has
  // waited for its own part and passed the barrier, the stage is in LDS.
  auto stage_ready = [&](int st, int nk, int depth) {
    const int later = min(depth, nk - 1 - st);
    switch (later) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<PW>(); break;
      case 2: wait_vmcnt<2 * PW>(); break;
      case 3: wait_vmcnt<3 * PW>(); break;
      case 4: wait_vmcnt<4 * PW>(); break;
      case 5: wait_vmcnt<5 * PW>(); break;
      default: wait_vmcnt<6 * PW>(); break;
    }
    // A bare barrier: __syncthreads() would add a release fence that waits for all loads in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int nk = min(kb_per, K / DS_BK - kb0);
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st * DS_BK);
  if constexpr (!SCHED) {
    // Iteration kt: make stage kt visible (NS-2 later stages may still be in flight), refill the
    // buffer of stage kt-1 (every wave finished reading it before this barrier), read and multiply.
    for (int kt = 0; kt < nk; ++kt) {
      stage_ready(kt, nk, NS - 2);
      if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, (kt + NS - 1) * DS_BK);
      read_frags(af[0], bw[0], kt % NS);
      mfmas(af[0], bw[0]);
    }
  } else {
    // Scheduled loop.  Fragments are double-buffered in registers: iteration kt makes stage
    // kt+1 visible, refills the buffer of stage kt-1 (every wave read it before the MFMAs of
    // iteration kt-1, which precede this barrier), reads stage kt+1's fragments and runs
    // stage kt's MFMAs.  In the steady state k-steps go in pairs that both issue a real stage
    // (kt + NS < nk), so the wait before stage kt+1 always allows NS-3 later stages in flight
    // and the body has no branch: the DMA issue, then the next k-step's fragment reads
    // interleaved with this k-step's MFMAs by scheduling groups, so the matrix pipe is fed
    // while the reads are in flight.  The last (at most 4) k-steps run a guarded iteration.
    // Unrolled by two so the fragment buffers have fixed registers.
    stage_ready(0, nk, NS - 2);
    read_frags(af[0], bw[0], 0);
    auto step = [&](int kt, f16x8_t* a_cur, f16x8_t* b_cur, f16x8_t* a_nxt, f16x8_t* b_nxt)
        __attribute__((always_inline)) {
      wait_vmcnt<(NS - 3) * PW>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue((kt + NS - 1) % NS, (kt + NS - 1) * DS_BK);
      read_frags(a_nxt, b_nxt, (kt + 1) % NS);
      mfmas(a_cur, b_cur);
      __builtin_amdgcn_sched_group_barrier(0x020, PW, 0);  // DMA first
#pragma unroll
      for (int g = 0; g < FM + FN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      // one fragment read
        __builtin_amdgcn_sched_group_barrier(0x008, (FM * FN) / (FM + FN), 0);  // then MFMAs
      }
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN) * ((FM * FN) / (FM + FN)), 0);
    };
    auto iter = [&](int kt, f16x8_t* a_cur, f16x8_t* b_cur, f16x8_t* a_nxt, f16x8_t* b_nxt)
        __attribute__((always_inline)) {
      if (kt + 1 < nk) {
        stage_ready(kt + 1, nk, NS - 3);
        if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, (kt + NS - 1) * DS_BK);
        read_frags(a_nxt, b_nxt, (kt + 1) % NS);
      }
      mfmas(a_cur, b_cur);
    };
    int kt = 0;
    for (; kt + NS < nk; kt += 2) {
      step(kt, af[0], bw[0], af[1], bw[1]);
      step(kt + 1, af[1], bw[1], af[0], bw[0]);
    }
    static_assert(NS == 4, "the cleanup below covers the last NS k-steps of a 4-stage pipeline");
    if (kt < nk) iter(kt, af[0], bw[0], af[1], bw[1]);
    if (kt + 1 < nk) iter(kt + 1, af[1], bw[1], af[0], bw[0]);
    if (kt + 2 < nk) iter(kt + 2, af[0], bw[0], af[1], bw[1]);
    if (kt + 3 < nk) iter(kt + 3, af[1], bw[1], af[0], bw[0]);
  }


  dma_tile_epilogue<BM, FM, FN, NW, EPI>(ep, acc, smem, M, N, tm, tm + wm * WM, tn + wn * WN, tid, lg, l16);
}

template <int BM, int BN, int WGM, int WGN, bool SB = false>
static void gemm_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep, hipStream_t s,
                          int splits = 1);

template <int BM, int BN, int NS>
static constexpr size_t gemm_dma_lds_bytes() {
  return (size_t)NS * (BM + BN) * DS_BK * sizeof(f16_t);
}

// Returns the number of K slices launched (1 unless split).  A split is aligned to the 64-wide
// k-steps gemm_splitk_count counts in, so the slice count equals the one it returned.
template <int BM, int BN, int WGM, int WGN, int NS, bool SCHED = false>
static int gemm_dma_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep,
                             hipStream_t s, int splits = 1) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int nkb = K / DS_BK;
  const int kb_per = splits > 1 ? 2 * ((((K + 63) / 64) + splits - 1) / splits) : nkb;
  const dim3 grid(tm * tn, (nkb + kb_per - 1) / kb_per);
  const int nt = 64 * WGM * WGN;
  constexpr size_t lds = gemm_dma_lds_bytes<BM, BN, NS>();
  // Above 64 KiB the per-kernel dynamic LDS limit must be raised, once (a function-local static
  // is initialised exactly once even with concurrent callers).
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void*)gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_STORE_F32, SCHED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_RESID, SCHED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_QKV, SCHED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_SWIGLU, SCHED>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)attr;
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_STORE_F32, SCHED>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_RESID:
      launch_k(gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_RESID, SCHED>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_QKV:
      // The staged RoPE rows (BM x d floats, d <= 128) fit only square 4-stage tiles; other
      // tiles hand the q|k|v projection to the register-staged kernel.
      if constexpr (BM == BN && NS >= 4)
        launch_k(gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_QKV, SCHED>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      else
        gemm_dispatch<128, 128, 2, 2>(A, W, M, N, K, ep, s);
      break;
    case EPI_SWIGLU:
      launch_k(gemm_dma_kernel<BM, BN, WGM, WGN, NS, EPI_SWIGLU, SCHED>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
  }
  return (int)grid.y;
}

// ------------------------------------------------------------------ 64-wide DMA stages
//
// As gemm_dma_kernel, with stages of BK = 64.  A tile row is then 128 bytes, one full cache line,
// and a DMA instruction fills 8 whole rows; with the 64-byte rows of 32-wide stages every DMA
// instruction touches 16 half lines, which doubles the cache requests per byte and keeps the
// texture-address unit stalled on the vector cache for much of the kernel.  Two stage buffers:
// while the waves multiply stage s, stage s+1 is landing; the DMA of stage s+2 goes out as soon as
// every wave holds all of stage s in registers (after the barrier in the middle of iteration s),
// so a stage has one whole iteration to land.  Chunk c of row r sits at c ^ (r % 8): the 8 lanes
// of one LDS read cycle (8 consecutive rows, one chunk) hit distinct banks.  K must be a multiple
// of 64 (and K slices even counts of 32-wide k-steps).

constexpr int D64_BK = 64;

__device__ __forceinline__ int d64_off(int r, int c) { return r * D64_BK + ((c ^ (r & 7)) << 3); }

template <int BM, int BN, int WGM, int WGN, int EPI>
__global__ void __launch_bounds__(64 * WGM * WGN) gemm_dma64_kernel(const f16_t* __restrict__ A,
                                                                    const f16_t* __restrict__ W, int M, int N, int K,
                                                                    int tiles_m, int tiles_n, EpiParams ep,
                                                                    int kb_per) {
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int STAGE = (BM + BN) * D64_BK;  // f16 elements per stage
  constexpr int NI = (BM + BN) / 8;          // DMA instructions per stage
  constexpr int PW = NI / NW;                // ... per wave
  static_assert(NI % NW == 0 && PW < 64, "DMA instructions do not split evenly over the waves");

  extern __shared__ __attribute__((aligned(16))) f16_t smem[];

  int tm_idx, tn_idx;
  dma_tile_of(blockIdx.x, tiles_m, tiles_n, tm_idx, tn_idx);
  const int tm = tm_idx * BM, tn = tn_idx * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave offsets in SGPRs
  const int wm = wid / WGN, wn = wid % WGN;
  const int l16 = lane & 15, lg = lane >> 4;

  // K range of this workgroup: kb_per 32-wide k-steps (an even count) from split blockIdx.y.
  const int kb0 = blockIdx.y * kb_per;
  const int kbase = kb0 * DS_BK;

  // Lane l of a DMA instruction takes row l / 8 of its 8-row block and physical chunk l % 8,
  // which holds logical chunk (l % 8) ^ (row % 8).  The wave's first PA instructions fill A
  // blocks, the rest W blocks; each keeps a 32-bit byte offset from the operand's base.
  constexpr int PA = BM / 8 / NW;
  static_assert((BM / 8) % NW == 0, "A blocks do not split evenly over the waves");
  const int dr = lane >> 3;
  const int dc = ((lane & 7) ^ dr) * 8;
  unsigned goff[PW];
  int dst_off[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int blk = wid + NW * i;  // 8-row block of the stage: A blocks first, then W blocks
    if (i < PA) {
      goff[i] = (unsigned)(((size_t)min(tm + blk * 8 + dr, M - 1) * K + kbase + dc) * sizeof(f16_t));
      dst_off[i] = blk * 8 * D64_BK;
    } else {
      const int b = blk - BM / 8;
      goff[i] = (unsigned)(((size_t)min(tn + b * 8 + dr, N - 1) * K + kbase + dc) * sizeof(f16_t));
      dst_off[i] = BM * D64_BK + b * 8 * D64_BK;
    }
  }
  auto issue = [&](int buf, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PW; ++i)
      dma16_asm(i < PA ? A : W, goff[i] + (unsigned)(k0 * sizeof(f16_t)), smem + buf * STAGE + dst_off[i]);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragments of one 32-wide half of a stage (sub = 0 or 1), double-buffered in registers.
  f16x8_t af[2][FM], bw[2][FN];
  auto read_frags = [&](f16x8_t* a, f16x8_t* b, int buf, int sub) __attribute__((always_inline)) {
    const f16_t* As = smem + buf * STAGE;
    const f16_t* Bs = As + BM * D64_BK;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      a[i] = *reinterpret_cast<const f16x8_t*>(&As[d64_off(wm * WM + i * 16 + l16, sub * 4 + lg)]);
#pragma unroll
    for (int jn = 0; jn < FN; ++jn)
      b[jn] = *reinterpret_cast<const f16x8_t*>(&Bs[d64_off(wn * WN + jn * 16 + l16, sub * 4 + lg)]);
  };
  auto mfmas = [&](const f16x8_t* a, const f16x8_t* b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[jn], acc[i][jn], 0, 0, 0);
  };
  // Interleave the half's fragment reads with its MFMAs, products first: the first MFMA then
  // waits only for reads issued in the previous half.
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < FM + FN; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, (FM * FN) / (FM + FN), 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN) * ((FM * FN) / (FM + FN)), 0);
  };

  const int ns = min(kb_per, K / DS_BK - kb0) / 2;
  issue(0, 0);
  if (ns > 1) {
    issue(1, D64_BK);
    wait_vmcnt<PW>();
  } else {
    wait_vmcnt<0>();
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frags(af[0], bw[0], 0, 0);
  // Iteration st: first half on stage st's fragments 0..31 while reading 32..63; then, once
  // stage st+1 has landed and every wave is past its reads of buffer st % 2, the DMA of stage
  // st+2 into that buffer and the second half while reading stage st+1's first fragments.  The
  // steady state (st + 2 < ns) has no branch; the last two iterations are peeled.
  auto first_half = [&](int cur) __attribute__((always_inline)) {
    read_frags(af[1], bw[1], cur, 1);
    mfmas(af[0], bw[0]);
    interleave();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  int st = 0;
  for (; st + 2 < ns; ++st) {
    const int cur = st & 1;
    first_half(cur);
    issue(cur, (st + 2) * D64_BK);
    read_frags(af[0], bw[0], cur ^ 1, 0);
    mfmas(af[1], bw[1]);
    interleave();
  }
  if (st + 1 < ns) {
    first_half(st & 1);
    read_frags(af[0], bw[0], (st & 1) ^ 1, 0);
    mfmas(af[1], bw[1]);
    interleave();
    ++st;
  }
  first_half(st & 1);
  mfmas(af[1], bw[1]);

  dma_tile_epilogue<BM, FM, FN, NW, EPI>(ep, acc, smem, M, N, tm, tm + wm * WM, tn + wn * WN, tid, lg, l16);
}

// Whether a projection can take gemm_dma64_kernel: K a multiple of 64, and every operand byte
// within the 32-bit lane offset its DMA addresses with (kept under 2 GiB).
static bool dma64_ok(int M, int N, int K) {
  return K % D64_BK == 0 && (size_t)std::max(M, N) * (size_t)K * sizeof(f16_t) < ((size_t)1 << 31);
}

// Launches gemm_dma64_kernel; returns the number of K slices (K % 64 == 0).
template <int BM, int BN, int WGM, int WGN>
static int gemm_dma64_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep,
                               hipStream_t s, int splits = 1) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int nkb = K / DS_BK;
  const int kb_per = splits > 1 ? 2 * ((((K + 63) / 64) + splits - 1) / splits) : nkb;
  const dim3 grid(tm * tn, (nkb + kb_per - 1) / kb_per);
  const int nt = 64 * WGM * WGN;
  constexpr size_t lds = (size_t)2 * (BM + BN) * D64_BK * sizeof(f16_t);
  // the q|k|v epilogue stages the tile's RoPE rows (BM x d floats, d <= 128) in the same LDS
  constexpr size_t lds_qkv = std::max(lds, (size_t)BM * 128 * sizeof(float));
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void*)gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_STORE_F32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_RESID>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_QKV>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_qkv);
    (void)hipFuncSetAttribute((const void*)gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_SWIGLU>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)attr;
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_STORE_F32>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_RESID:
      launch_k(gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_RESID>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_QKV:
      launch_k(gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_QKV>, grid, nt, lds_qkv, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_SWIGLU:
      launch_k(gemm_dma64_kernel<BM, BN, WGM, WGN, EPI_SWIGLU>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
  }
  return (int)grid.y;
}

template <int BM, int BN>
static size_t gemm_lds_bytes() {
  return (size_t)2 * (BM + BN) * GEMM_LDK * sizeof(f16_t);
}

template <int BM, int BN, int WGM, int WGN, bool SB>
static void gemm_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep, hipStream_t s,
                          int splits) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int nkb = (K + GEMM_BK - 1) / GEMM_BK;
  const int kb_per = (nkb + splits - 1) / splits;
  const dim3 grid(tm * tn, (nkb + kb_per - 1) / kb_per);
  const int nt = 64 * WGM * WGN;
  const size_t lds = gemm_lds_bytes<BM, BN>();
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_STORE_F32, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_RESID:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_RESID, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_QKV:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_QKV, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_SWIGLU:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_SWIGLU, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
  }
}

template <int BM, int BN, int WGM, int WGN, bool SB = false>
static void gemm_set_lds_limit() {
  const int bytes = (int)gemm_lds_bytes<BM, BN>();
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_STORE_F32, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_RESID, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_QKV, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_SWIGLU, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// Tiles above 64 KiB of LDS need the per-kernel dynamic limit raised once.
static void gemm_init_attributes() {
  static const bool done = [] {
    gemm_set_lds_limit<256, 256, 2, 4, true>();
    gemm_set_lds_limit<128, 128, 2, 2>();
    return true;
  }();
  (void)done;
}

// The epilogue of four consecutive columns n .. n+3 of row m (N % 4 == 0 on the paths that use
// it), so RoPE partners (2j, 2j+1) and SwiGLU gate/up pairs (2c, 2c+1) are together.
// STORE_F32 writes to `out` (a split's slice of the partial sums, or the output).
// Returns whether an fp16 value it stored left fp16's range.
template <int EPI>
__device__ __forceinline__ bool epi_apply4(const EpiParams& ep, float* out, int m, int n, const float (&a)[4]) {
  if (EPI == EPI_QKV && (ep.head_dim & 3) == 0) return qkv_store4(ep, m, n, a);
  bool bad = false;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (EPI == EPI_STORE_F32) out[(size_t)m * ep.ld + n + c] = a[c];
    else if (EPI == EPI_RESID) ep.out_f32[(size_t)m * ep.ld + n + c] += a[c];
    else if (EPI == EPI_QKV) bad |= epi_qkv<f16_t>(ep, m, n + c, a[c], a[c ^ 1]);
    else if (EPI == EPI_SWIGLU && (c & 1) == 0) bad |= epi_swiglu<f16_t>(ep, m, (n + c) >> 1, a[c], a[c + 1]);
  }
  return bad;
}

// Split-K second pass: out = epilogue(sum over the splits of part[s][m][n]), summed in split
// order.  One thread per 4 consecutive columns (N % 4 == 0).
template <int EPI>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                            EpiParams ep) {
  const size_t i4 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t slice = (size_t)M * N;
  if (i4 * 4 >= slice) return;
  const size_t e = i4 * 4;
  const int m = (int)(e / N), n = (int)(e % N);
  float4 v = *reinterpret_cast<const float4*>(part + e);
  for (int sp = 1; sp < splits; ++sp) {
    const float4 w = *reinterpret_cast<const float4*>(part + (size_t)sp * slice + e);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const float a[4] = {v.x, v.y, v.z, v.w};
  raise_range_error(ep, epi_apply4<EPI>(ep, ep.out_f32, m, n, a));
}

// Split-K reduction of a residual projection fused with the RMSNorm that consumes its result:
// x[m] += (sum over the splits of part[s][m], in split order), then
// a[m] = fp16(x[m] / sqrt(mean(x[m]^2) + eps) * w), fp32 statistics summed in a fixed order.
// One 1024-thread workgroup per row, V4 float4 of the row per thread (N % 4 == 0,
// N <= 4096 V4), so a row's loads all go out at once.
template <int V4>
__global__ void __launch_bounds__(1024) splitk_resid_norm_kernel(const float* __restrict__ part, int splits, int M,
                                                                 int N, float* __restrict__ x, int ldx,
                                                                 const float* __restrict__ w, float eps,
                                                                 f16_t* __restrict__ a, int* err) {
  __shared__ float red[16];
  const int m = blockIdx.x;
  const size_t slice = (size_t)M * N;
  float* xr = x + (size_t)m * ldx;
  f32x4_t v[V4];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i = (threadIdx.x + 1024 * j) * 4;
    if (i < N) {
      float4 p = *reinterpret_cast<const float4*>(part + (size_t)m * N + i);
      for (int sp = 1; sp < splits; ++sp) {
        const float4 q = *reinterpret_cast<const float4*>(part + (size_t)sp * slice + (size_t)m * N + i);
        p.x += q.x; p.y += q.y; p.z += q.z; p.w += q.w;
      }
      const float4 xo = *reinterpret_cast<const float4*>(xr + i);
      v[j] = f32x4_t{xo.x + p.x, xo.y + p.y, xo.z + p.z, xo.w + p.w};
      *reinterpret_cast<float4*>(xr + i) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
      ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
    }
  }
  ss = wave_sum(ss);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)N + eps);
  f16_t* ar = a + (size_t)m * N;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i = (threadIdx.x + 1024 * j) * 4;
    if (i < N) {
      const f32x4_t g = *reinterpret_cast<const f32x4_t*>(w + i);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float y = v[j][k] * inv * g[k];
        bad |= f16_out_of_range(y);
        ar[i + k] = from_f32<f16_t>(y);
      }
    }
  }
  if (bad) atomicOr(err, LLM_DEVERR_RANGE_BIT);
}

// Weight-streaming GEMM for batches of at most 64 rows (batched decode).  Such a projection is
// bound by the weight stream, and on this GPU one CU streams at most about 22 GB/s from HBM
// (measured: 224 workgroups of 128 weight rows, one per CU, reach 4.6 TB/s with or without
// deeper pipelines; 448 workgroups of 64 rows over all 256 CUs reach 5.6).  So the grid is
// sized to give every CU one equal share: an N tile of 16 * FN weight rows over one K slice,
// FN and the slice count chosen per shape (stream_plan), e.g. 256 tiles of 112 rows for the
// 28672-row gate-up projection.  Any FN works because the 4 waves split each stage's K instead
// of its columns:
//  - a stage holds BK = 128 k of the 64 activation rows and the BN weight rows, as 256-byte
//    row pieces (whole 128-byte lines) brought in by LDS DMA, 16-byte chunk c of row r at
//    position c ^ (r % 16) (fragment reads of 8 consecutive rows hit distinct banks);
//  - wave w multiplies k-quarter w of every stage into its own 64 x BN accumulators;
//  - at the end the four partial tiles meet in LDS, are summed in wave order (deterministic)
//    and go through the epilogue 4 columns per thread: the output itself when K is not split,
//    else this slice's partial sums for the reduction pass (splitk_reduce_kernel, or
//    splitk_resid_norm_kernel when the RMSNorm that follows rides along).
constexpr int ST_BK = 128;

template <int FN, int NS>
static constexpr size_t stream_lds_bytes() {
  return std::max((size_t)NS * (64 + 16 * FN) * ST_BK * sizeof(f16_t), (size_t)4 * 64 * 16 * FN * sizeof(float));
}

template <int FN, int NS, int EPI>
__global__ void __launch_bounds__(256) gemm_stream_kernel(const f16_t* __restrict__ A, const f16_t* __restrict__ W,
                                                          int M, int N, int K, EpiParams ep, int kb_per) {
  constexpr int BM = 64, BN = 16 * FN, ROWS = BM + BN;
  constexpr int STAGE = ROWS * ST_BK;  // f16 elements per stage
  constexpr int NI = ROWS / 4;         // DMA instructions per stage: 4 rows x 256 bytes each
  constexpr int PW = NI / 4;           // ... per wave
  static_assert(NI % 4 == 0, "DMA instructions do not split evenly over the waves");
  static_assert(NS >= 3 && NS <= 4 && (NS - 2) * PW < 64, "stages");

  extern __shared__ __attribute__((aligned(16))) f16_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int tn = blockIdx.x * BN;
  const int kb0 = blockIdx.y * kb_per;  // first stage (of ST_BK k) of this slice
  const int nk = min(kb_per, K / ST_BK - kb0);

  // DMA: instruction j of a stage covers tile rows 4j .. 4j+3 (activation rows first); lane l
  // lands at row 4j + l/16, physical chunk l % 16, and so loads logical chunk (l % 16) ^ (row % 16).
  const f16_t* src[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int j = wid * PW + i;
    const int r = 4 * j + (lane >> 4);
    const int col = ((lane & 15) ^ (r & 15)) * 8 + kb0 * ST_BK;
    src[i] = r < BM ? A + (size_t)min(r, M - 1) * K + col : W + (size_t)min(tn + r - BM, N - 1) * K + col;
  }
  auto issue = [&](int buf, int kt) {
    f16_t* base = smem + buf * STAGE + wid * PW * 4 * ST_BK;
#pragma unroll
    for (int i = 0; i < PW; ++i)
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(src[i] + kt * ST_BK),
                                       (void __attribute__((address_space(3)))*)(base + i * 4 * ST_BK), 16, 0, 0);
  };

  f32x4_t acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) acc[i][jn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) issue(st, st);
  // Logical chunk of this lane's fragments: k-quarter wid of the stage, 8 k per lane group.
  const int fc = ((4 * wid + lg) ^ l16) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt is in LDS once at most min(NS - 2, nk - 1 - kt) later stages are outstanding.
    const int later = min(NS - 2, nk - 1 - kt);
    if (later >= 2) wait_vmcnt<2 * PW>();
    else if (later == 1) wait_vmcnt<PW>();
    else wait_vmcnt<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // The buffer of stage kt - 1 is free: every wave finished reading it before this barrier.
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
    const f16_t* As = smem + (kt % NS) * STAGE;
    const f16_t* Ws = As + BM * ST_BK;
    f16x8_t af[4], bw[FN];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const f16x8_t*>(As + (i * 16 + l16) * ST_BK + fc);
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) bw[jn] = *reinterpret_cast<const f16x8_t*>(Ws + (jn * 16 + l16) * ST_BK + fc);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jn = 0; jn < FN; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bw[jn], acc[i][jn], 0, 0, 0);
  }

  // The four waves' partial tiles meet in LDS ([wave][row][col] floats over the stage buffers).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jn = 0; jn < FN; ++jn)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wid * BM + i * 16 + lg * 4 + r) * BN + jn * 16 + l16] = acc[i][jn][r];
  __syncthreads();
  float* out = EPI == EPI_STORE_F32 ? ep.out_f32 + (size_t)blockIdx.y * M * ep.ld : ep.out_f32;
  bool bad = false;
  for (int g = tid; g < BM * BN / 4; g += 256) {
    const int m = g / (BN / 4), c4 = (g % (BN / 4)) * 4;
    if (m >= M || tn + c4 >= N) continue;
    float4 v = *reinterpret_cast<const float4*>(red + m * BN + c4);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 u = *reinterpret_cast<const float4*>(red + (w * BM + m) * BN + c4);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    const float a[4] = {v.x, v.y, v.z, v.w};
    bad |= epi_apply4<EPI>(ep, out, m, tn + c4, a);
  }
  raise_range_error(ep, bad);
}

// Launch over N / (16 FN) tiles and `splits` K slices (whole stages of ST_BK each); returns the
// slice count.  Requires M <= 64, K % ST_BK == 0 and N % 4 == 0.
template <int FN, int NS>
static int gemm_stream_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep,
                                hipStream_t s, int splits) {
  constexpr int BN = 16 * FN;
  const int nkb = K / ST_BK;
  const int kb_per = (nkb + splits - 1) / splits;
  const dim3 grid((N + BN - 1) / BN, (nkb + kb_per - 1) / kb_per);
  constexpr size_t lds = stream_lds_bytes<FN, NS>();
  static const bool attr = [] {
    (void)hipFuncSetAttribute((const void*)gemm_stream_kernel<FN, NS, EPI_STORE_F32>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_stream_kernel<FN, NS, EPI_RESID>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_stream_kernel<FN, NS, EPI_QKV>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)hipFuncSetAttribute((const void*)gemm_stream_kernel<FN, NS, EPI_SWIGLU>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    return true;
  }();
  (void)attr;
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemm_stream_kernel<FN, NS, EPI_STORE_F32>, grid, 256, lds, s, A, W, M, N, K, ep, kb_per);
      break;
    case EPI_RESID:
      launch_k(gemm_stream_kernel<FN, NS, EPI_RESID>, grid, 256, lds, s, A, W, M, N, K, ep, kb_per);
      break;
    case EPI_QKV:
      launch_k(gemm_stream_kernel<FN, NS, EPI_QKV>, grid, 256, lds, s, A, W, M, N, K, ep, kb_per);
      break;
    case EPI_SWIGLU:
      launch_k(gemm_stream_kernel<FN, NS, EPI_SWIGLU>, grid, 256, lds, s, A, W, M, N, K, ep, kb_per);
      break;
  }
  return (int)grid.y;
}

// Plan of the weight-streaming kernel for 8 < M <= 64: FN (tile of 16 FN weight rows) and the
// K slice count S, over the tiles that divide N.  The rule, from a sweep of the Llama-3-8B
// projections at 64 and 40 rows on MI355X (weights rotated over copies so HBM is measured):
// the most workgroups up to 256 (one per CU; fewer leave CUs idle, more queue behind them),
// then tiles of at least 48 rows (narrower ones re-read the activations for too few weights:
// down on 32-row tiles 3.5 TB/s against 4.2 on 64), then the fewest slices (each slice adds
// a pass over fp32 partial sums).  E.g. q|k|v 3 x 2 slices 3.9 TB/s (was 2.9), wo 4 x 4
// slices 2.9 (2.5), gate-up 7 unsplit 4.6 (4.3), down 4 x 4 slices 4.2 (3.8).  Returns false
// when no plan gives more than 128 workgroups or the shape does not fit (K % 128, N % 4).
struct StreamPlan {
  int fn;
  int splits;
};

static bool stream_plan(int M, int N, int K, StreamPlan& p) {
  if (M <= 8 || M > 64 || K % ST_BK != 0 || N % 4 != 0) return false;
  static const int fns[] = {2, 3, 4, 6, 7, 8};
  const int nkb = K / ST_BK;
  bool found = false;
  long best[3] = {0, 0, 0};  // (workgroups, tile of >= 48 rows, -slices), compared in order
  for (int sp = 1; sp <= 8; sp *= 2) {
    if (nkb / sp < 4) break;
    for (int fn : fns) {
      if (N % (16 * fn) != 0) continue;
      const long wg = (long)(N / (16 * fn)) * sp;
      if (wg > 256 || wg <= 128) continue;
      const long key[3] = {wg, fn >= 3, -sp};
      if (!found || std::lexicographical_compare(best, best + 3, key, key + 3)) {
        std::copy(key, key + 3, best);
        p = {fn, sp};
        found = true;
      }
    }
  }
  return found;
}

// Launch a stream plan; returns the number of K slices (partial sums to reduce when > 1).
static int gemm_stream_run(const StreamPlan& p, const f16_t* A, const f16_t* W, int M, int N, int K,
                           const EpiParams& ep, hipStream_t s) {
  switch (p.fn) {
    case 2: return gemm_stream_dispatch<2, 3>(A, W, M, N, K, ep, s, p.splits);
    case 3: return gemm_stream_dispatch<3, 3>(A, W, M, N, K, ep, s, p.splits);
    case 4: return gemm_stream_dispatch<4, 3>(A, W, M, N, K, ep, s, p.splits);
    case 6: return gemm_stream_dispatch<6, 3>(A, W, M, N, K, ep, s, p.splits);
    case 7: return gemm_stream_dispatch<7, 3>(A, W, M, N, K, ep, s, p.splits);
    default: return gemm_stream_dispatch<8, 3>(A, W, M, N, K, ep, s, p.splits);
  }
}

// Number of K splits for a GEMM: only small-M shapes (weight streaming) whose 64 x 64
// tiles give fewer than 256 workgroups (one per CU) are split: the smallest power of two
// giving at least 384 of them, at most 8 and at least 4 K steps of 64 per split.  From a sweep
// at M = 16, 64 and 128 on MI355X with the weights streamed from HBM (rotating copies): at 64
// rows, q|k|v streams at 3.1 TB/s in 4 slices, wo at 2.5 in 4 or 8, down at 3.8 in 8 (on
// 64 x 128 tiles), while the 448-tile gate-up projection is fastest unsplit.
int gemm_splitk_count(int M, int N, int K) {
  if (M <= 0 || M > 128 || N % 4 != 0) return 1;
  const long tiles = (long)((M + 63) / 64) * ((N + 63) / 64);
  if (tiles >= 256) return 1;
  const int nkb = (K + GEMM_BK - 1) / GEMM_BK;
  int sp = 2;
  while (sp < 8 && tiles * sp < 384) sp *= 2;
  sp = std::min(sp, nkb / 4);
  if (sp < 2) return 1;
  const int per = (nkb + sp - 1) / sp;
  return (nkb + per - 1) / per;
}

// Prefill row counts (M > 128) whose large tiles cannot fill the GPU: 256 x 256 tiles when they
// number at least 192; else, with K >= 4096, 256 x 256 tiles in 2 K slices when that gives 192
// to 320 workgroups (not for q|k|v); else 256 x 128 (not for q|k|v) when they number at least
// 192; otherwise K is split over the 256 x 256 or 256 x 128 tiles with at least 1024 k per
// slice and at most 320 workgroups, taking the most workgroups up to 256, then the fewest
// slices, then the larger tile.  From sweeps of the Llama-3-8B projections on MI355X: down at
// M = 512, 498 TFLOP/s unsplit on 64 x 64 tiles, 841 on 256 x 128 tiles in 4 slices; down at
// M = 2048, 280 us on 256 x 128 tiles against 212 on 256 x 256 tiles in 2 slices.  A residual
// projection with K < 8192 (wo) skips the 2-slice plan: since its tile epilogue keeps all residual
// loads in flight, wo at M = 2048 takes 77.5 us on unsplit 256 x 128 tiles against 84.6 in 2
// slices with their reduction (down, K = 14336, stays split: 215 against 253 us unsplit).
struct BigPlan {
  int tile;  // 0: 256 x 256, 1: 256 x 128
  int splits;
};

static bool big_tile_plan(int M, int N, int K, bool qkv, BigPlan& p, bool resid = false) {
  if (M <= 128 || K % DS_BK != 0) return false;
  auto tiles = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(256, 256) >= 192) { p = {0, 1}; return true; }
  if (!qkv && !(resid && K < 8192) && K >= 4096 && N % 4 == 0 && tiles(256, 256) * 2 >= 192 && tiles(256, 256) * 2 <= 320) {
    p = {0, 2};
    return true;
  }
  if (!qkv && tiles(256, 128) >= 192) { p = {1, 1}; return true; }
  long best = 0;
  bool found = false;
  for (int sp = 2; sp <= 8; sp *= 2) {
    if (K / sp < 1024 || N % 4 != 0) break;
    for (int t = 0; t < 2; ++t) {
      const long wg = tiles(256, t == 0 ? 256 : 128) * sp;
      if (wg > 320) continue;
      const long score = std::min<long>(wg, 256);
      if (!found || score > best) { best = score; p = {t, sp}; found = true; }
    }
  }
  return found;
}

size_t gemm_splitk_floats(int M, int N, int K) {
  BigPlan bp;
  // The q|k|v projection is the only one with N = (H + 2 G) d; which projection it is matters
  // only for the tile choice, so both readings are sized for.
  size_t need = 0;
  for (bool qkv : {false, true})
    if (big_tile_plan(M, N, K, qkv, bp) && bp.splits > 1) need = std::max(need, (size_t)bp.splits * M * N);
  const int sp = gemm_splitk_count(M, N, K);
  if (sp > 1) need = std::max(need, (size_t)sp * M * N);
  StreamPlan st;
  if (stream_plan(M, N, K, st) && st.splits > 1) need = std::max(need, (size_t)st.splits * M * N);
  return need;
}

// Compute units of the current device (read once; 256 on MI355X).
static int gemm_cu_count() {
  static const int n = [] {
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipGetLastError();
    return c > 0 ? c : 256;
  }();
  return n;
}

// 256 x 256 tiles that do not come in whole waves over the CUs leave the last wave partly idle: at
// M = 2048 the gate-up projection has 896 tiles, 3.5 waves on 256 CUs, so it takes 4 tile times.
// Then the columns of the whole waves stay on 256 x 256 tiles and the rest go to a second GEMM,
// when that is at most one wave of 256 x 128 tiles (at M = 2048: 768 tiles, then a 4096-column
// GEMM).  Returns the first column of that tail, or N for no split.
static int big_tile_tail_split(int M, int N) {
  const long cus = gemm_cu_count();
  if (N % 256 != 0) return N;
  const long tm = (M + 255) / 256, tn = N / 256, t = tm * tn;
  if (t < cus || t % cus == 0) return N;
  const long full = t / cus * cus;
  if (full % tm != 0) return N;
  const long n_main = full / tm;
  if (tm * (tn - n_main) * 2 > cus) return N;
  return (int)(n_main * 256);
}

// Tile choice from sweeps of the Llama-3-8B projection shapes at M = 16 .. 8192 on MI355X.
// 8 < M <= 64 with K % 128 == 0 streams the weights through gemm_stream_kernel (stream_plan).
// Other shapes with K % 32 == 0 use the LDS-DMA kernel: M <= 128 split over K on 64 x 64 tiles
// (gemm_splitk_count); larger M as big_tile_plan says (256 x 256 or 256 x 128 tiles, split
// over K when they are too few), then 128 x 128 with at least 192 tiles, else 64 x 64.  Other
// K use the register-staged kernel.
void launch_gemm_f16(const void* A, const void* W, int M, int N, int K, const EpiParams& ep, float* splitk_ws,
                     size_t splitk_ws_floats, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  gemm_init_attributes();
  const f16_t* a = (const f16_t*)A;
  const f16_t* w = (const f16_t*)W;
  auto tiles = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  auto reduce = [&](int ns) {
    const size_t n4 = (size_t)M * N / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    switch (ep.kind) {
      case EPI_STORE_F32: launch_k(splitk_reduce_kernel<EPI_STORE_F32>, grid, 256, 0, s, splitk_ws, ns, M, N, ep); break;
      case EPI_RESID: launch_k(splitk_reduce_kernel<EPI_RESID>, grid, 256, 0, s, splitk_ws, ns, M, N, ep); break;
      case EPI_QKV: launch_k(splitk_reduce_kernel<EPI_QKV>, grid, 256, 0, s, splitk_ws, ns, M, N, ep); break;
      case EPI_SWIGLU: launch_k(splitk_reduce_kernel<EPI_SWIGLU>, grid, 256, 0, s, splitk_ws, ns, M, N, ep); break;
    }
  };
  if (ep.kind == EPI_SWIGLU && M > 128 && dma64_ok(M, N, K) && tiles(256, 256) >= 192) {
    // The SwiGLU projection's columns beyond its whole waves of 256 x 256 tiles go to a second GEMM,
    // planned on its own (at M = 2048: 256 x 256 tiles in two K slices); output column = weight
    // row / 2.
    const int nt = big_tile_tail_split(M, N);
    if (nt < N) {
      launch_gemm_f16(A, W, M, nt, K, ep, splitk_ws, splitk_ws_floats, s);
      EpiParams et = ep;
      et.out_act = (f16_t*)ep.out_act + nt / 2;
      launch_gemm_f16(A, w + (size_t)nt * K, M, N - nt, K, et, splitk_ws, splitk_ws_floats, s);
      return;
    }
  }
  {
    BigPlan bp;
    if (big_tile_plan(M, N, K, ep.kind == EPI_QKV, bp, ep.kind == EPI_RESID) && bp.splits > 1 && splitk_ws &&
        (size_t)bp.splits * M * N <= splitk_ws_floats) {
      EpiParams pe = ep;
      pe.kind = EPI_STORE_F32;
      pe.out_f32 = splitk_ws;
      pe.ld = N;
      const int ns = dma64_ok(M, N, K)
                         ? (bp.tile == 0 ? gemm_dma64_dispatch<256, 256, 2, 4>(a, w, M, N, K, pe, s, bp.splits)
                                         : gemm_dma64_dispatch<256, 128, 4, 2>(a, w, M, N, K, pe, s, bp.splits))
                         : (bp.tile == 0 ? gemm_dma_dispatch<256, 256, 2, 4, 4, true>(a, w, M, N, K, pe, s, bp.splits)
                                         : gemm_dma_dispatch<256, 128, 4, 2, 4, true>(a, w, M, N, K, pe, s, bp.splits));
      reduce(ns);
      return;
    }
  }
  {
    StreamPlan st;
    if (stream_plan(M, N, K, st) && (st.splits == 1 || (splitk_ws && (size_t)st.splits * M * N <= splitk_ws_floats))) {
      if (st.splits == 1) {
        gemm_stream_run(st, a, w, M, N, K, ep, s);
      } else {
        EpiParams pe = ep;
        pe.kind = EPI_STORE_F32;
        pe.out_f32 = splitk_ws;
        pe.ld = N;
        reduce(gemm_stream_run(st, a, w, M, N, K, pe, s));
      }
      return;
    }
  }
  const int sp = gemm_splitk_count(M, N, K);
  if (sp > 1 && splitk_ws && (size_t)sp * M * N <= splitk_ws_floats) {
    EpiParams pe = ep;
    pe.kind = EPI_STORE_F32;
    pe.out_f32 = splitk_ws;
    pe.ld = N;
    int ns = sp;
    if (K % DS_BK == 0 && K >= 8192)  // long rows (down): 64 x 128 tiles, 3.8 TB/s against 3.2
      ns = gemm_dma_dispatch<64, 128, 1, 4, 4>(a, w, M, N, K, pe, s, sp);
    else if (K % DS_BK == 0)
      ns = gemm_dma_dispatch<64, 64, 2, 2, 4>(a, w, M, N, K, pe, s, sp);
    else
      gemm_dispatch<64, 64, 2, 2>(a, w, M, N, K, pe, s, sp);
    reduce(ns);
    return;
  }
  // The DMA kernel's q|k|v epilogue handles prefill rows whose RoPE table rows (BM x d floats)
  // fit its stage buffers: BM = BN square tiles with 4 stages hold d <= 128.
  const bool qkv = ep.kind == EPI_QKV;
  const bool dma_qkv_ok = ep.row_pos == nullptr && ep.head_dim <= 128;
  // Unsplit row counts up to 128 stream the weights, and wider tiles re-read the activations
  // less: at most 64 rows, 64 x 128 tiles when there are 256 to 1024 of 64 x 64 (gate-up: 4.3
  // TB/s against 3.5 on 64 x 64 tiles); above 64 rows, 64 x 256 tiles when they number 192 to
  // 512 (gate-up at 128 rows: 3.2 TB/s against 2.7).  Wider N (a batch's LM head) stays on the
  // register-staged 64 x 64 kernel up to 64 rows (5.2 TB/s) and on 128 x 128 tiles above.
  if (M <= 128 && K % DS_BK == 0 && !qkv) {
    const long t64 = tiles(64, 64), t256 = tiles(64, 256);
    if (M <= 64 && t64 >= 256 && t64 <= 1024) {
      gemm_dma_dispatch<64, 128, 1, 4, 4>(a, w, M, N, K, ep, s);
      return;
    }
    if (M > 64 && t256 >= 192 && t256 <= 512) {
      gemm_dma_dispatch<64, 256, 1, 4, 4>(a, w, M, N, K, ep, s);
      return;
    }
  }
  if (M > 64 && K % DS_BK == 0 && (!qkv || dma_qkv_ok)) {
    // The big tiles take 64-wide stages when K allows (whole cache lines per DMA row).
    if (M > 128 && tiles(256, 256) >= 192) {
      // 256 x 192 tiles when they fill the CUs in fewer tile-widths of waves (q|k|v at M = 2048:
      // 256 tiles, one wave, against 192 of 256 x 256 that leave a quarter of the CUs idle)
      const long cus = gemm_cu_count();
      auto wave_cost = [&](int bn) { return (tiles(256, bn) + cus - 1) / cus * bn; };
      if (dma64_ok(M, N, K) && N % 192 == 0 && wave_cost(192) < wave_cost(256)) {
        gemm_dma64_dispatch<256, 192, 2, 4>(a, w, M, N, K, ep, s);
      } else if (dma64_ok(M, N, K)) {
        gemm_dma64_dispatch<256, 256, 2, 4>(a, w, M, N, K, ep, s);
      } else {
        gemm_dma_dispatch<256, 256, 2, 4, 4, true>(a, w, M, N, K, ep, s);
      }
    } else if (M > 128 && !qkv && tiles(256, 128) >= 192) {
      if (dma64_ok(M, N, K)) gemm_dma64_dispatch<256, 128, 4, 2>(a, w, M, N, K, ep, s);
      else gemm_dma_dispatch<256, 128, 4, 2, 4, true>(a, w, M, N, K, ep, s);
    } else if (M > 64 && tiles(128, 128) >= 192) {
      gemm_dma_dispatch<128, 128, 2, 2, 4>(a, w, M, N, K, ep, s);
    } else {
      gemm_dma_dispatch<64, 64, 2, 2, 4>(a, w, M, N, K, ep, s);
    }
    return;
  }
  // The q|k|v epilogue (RoPE table reads, cache addressing) does not fit the register-staged
  // 256 x 256 tile's registers (it spills), so that projection stays on 128 x 128 tiles.
  if (M > 128 && ep.kind != EPI_QKV && tiles(256, 256) >= 192)
    gemm_dispatch<256, 256, 2, 4, true>(a, w, M, N, K, ep, s);
  else if (M > 64 && tiles(128, 128) >= 256)
    gemm_dispatch<128, 128, 2, 2>(a, w, M, N, K, ep, s);
  else
    gemm_dispatch<64, 64, 2, 2>(a, w, M, N, K, ep, s);
}


// x += A W^T (a residual projection, ep.kind == EPI_RESID) followed by a = rmsnorm(x) * norm_w in
// fp16, for shapes the weight-streaming plan splits over K: the reduction pass of the partial
// sums also applies the RMSNorm, which saves a launch.  Returns false, enqueueing nothing, for
// other shapes; the caller then runs the projection and the RMSNorm separately.
bool launch_gemm_f16_resid_norm(const void* A, const void* W, int M, int N, int K, const EpiParams& ep,
                                const float* norm_w, float eps, void* a_out, float* splitk_ws,
                                size_t splitk_ws_floats, hipStream_t s) {
  if (ep.kind != EPI_RESID || M <= 0 || N % 4 != 0 || N > 8192 || ep.ld != N || !splitk_ws) return false;
  StreamPlan st;
  if (!stream_plan(M, N, K, st) || st.splits < 2 || (size_t)st.splits * M * N > splitk_ws_floats) return false;
  EpiParams pe = ep;
  pe.kind = EPI_STORE_F32;
  pe.out_f32 = splitk_ws;
  pe.ld = N;
  const int ns = gemm_stream_run(st, (const f16_t*)A, (const f16_t*)W, M, N, K, pe, s);
  f16_t* a = (f16_t*)a_out;
  if (N <= 4096)
    launch_k(splitk_resid_norm_kernel<1>, M, 1024, 0, s, splitk_ws, ns, M, N, ep.out_f32, ep.ld, norm_w, eps, a,
             ep.err);
  else
    launch_k(splitk_resid_norm_kernel<2>, M, 1024, 0, s, splitk_ws, ns, M, N, ep.out_f32, ep.ld, norm_w, eps, a,
             ep.err);
  return true;
}

}  // namespace llm
