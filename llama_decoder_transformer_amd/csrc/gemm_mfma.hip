// Projections on the matrix cores: C[m][n] = sum_k A[m][k] * W[n][k] with fp16
// operands and fp32 accumulation, A = activations [M][K], W = weights [N][K]
// (both K-major, so both operands are staged into LDS with 16-byte row loads).
// The bf16 weights are held as fp16 (converted exactly at init) and activations
// are rounded to fp16 rather than bf16: same bytes and MFMA rate, 8x finer
// rounding, which keeps 32 layers within the bf16 parity bar.
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

template <int BM, int BN, int WGM, int WGN, int EPI, int NPART = 1, bool SB = false>
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

  // The next stage's global loads are split into NPART parts, one per k-step of
  // 32, so only 1/NPART of a stage sits in registers at a time.
  static_assert((BK / 32) % NPART == 0 && A_LD % NPART == 0 && B_LD % NPART == 0, "bad NPART");
  constexpr int PA = A_LD / NPART, PB = B_LD / NPART;
  u32x4_t ra[PA], rb[PB];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // Out-of-range rows / columns load from a clamped in-range address and are then
  // replaced by zero with a select, so the loads stay branch-free.
  auto gload = [&](int k0, int part) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int idx = tid + (part * PA + i) * NT, r = idx >> 3, c = (idx & 7) * 8;
      const int gm = tm + r, gk = k0 + c;
      const bool ok = gm < M && gk < K;
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(A + (size_t)min(gm, M - 1) * K + min(gk, K - 8));
      ra[i] = ok ? v : zero;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int idx = tid + (part * PB + i) * NT, r = idx >> 3, c = (idx & 7) * 8;
      const int gn = tn + r, gk = k0 + c;
      const bool ok = gn < N && gk < K;
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(W + (size_t)min(gn, N - 1) * K + min(gk, K - 8));
      rb[i] = ok ? v : zero;
    }
  };
  auto sstore = [&](int stage, int part) {
    f16_t* As = smem + stage * STAGE;
    f16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int idx = tid + (part * PA + i) * NT, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&As[lds_off(r, c >> 3)]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int idx = tid + (part * PB + i) * NT, r = idx >> 3, c = (idx & 7) * 8;
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
#pragma unroll
  for (int part = 0; part < NPART; ++part) {
    gload(kbase, part);
    sstore(0, part);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const f16_t* As = smem + cur * STAGE;
    const f16_t* Bs = As + BM * LDK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      constexpr int KS_PER_PART = (BK / 32) / NPART;
      if (more && ks % KS_PER_PART == 0) gload(kbase + (kt + 1) * BK, ks / KS_PER_PART);
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
      if (more && ks % KS_PER_PART == KS_PER_PART - 1) sstore(cur ^ 1, ks / KS_PER_PART);
    }
    __syncthreads();
  }

  // Epilogue.  A split-K workgroup stores its partial sums to slice blockIdx.y.
  float* const out_f32 = ep.out_f32 + (size_t)blockIdx.y * M * ep.ld;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int jn = 0; jn < FN; ++jn) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = tm + wm * WM + i * 16 + lg * 4 + r;
        const int n = tn + wn * WN + jn * 16 + l16;
        const float v = acc[i][jn][r];
        if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
          const float vp = __shfl_xor(v, 1);
          if (m < M && n < N) {
            if (EPI == EPI_QKV) epi_qkv<f16_t>(ep, m, n, v, vp);
            else if ((n & 1) == 0) epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
          }
        } else if (m < M && n < N) {
          if (EPI == EPI_STORE_F32) out_f32[(size_t)m * ep.ld + n] = v;
          else out_f32[(size_t)m * ep.ld + n] += v;
        }
      }
    }
  }
}

template <int BM, int BN>
static size_t gemm_lds_bytes() {
  return (size_t)2 * (BM + BN) * GEMM_LDK * sizeof(f16_t);
}

template <int BM, int BN, int WGM, int WGN, int NPART = 1, bool SB = false>
static void gemm_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep, hipStream_t s,
                          int splits = 1) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  const int nkb = (K + GEMM_BK - 1) / GEMM_BK;
  const int kb_per = (nkb + splits - 1) / splits;
  const dim3 grid(tm * tn, (nkb + kb_per - 1) / kb_per);
  const int nt = 64 * WGM * WGN;
  const size_t lds = gemm_lds_bytes<BM, BN>();
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_STORE_F32, NPART, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_RESID:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_RESID, NPART, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_QKV:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_QKV, NPART, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
    case EPI_SWIGLU:
      launch_k(gemm_f16_kernel<BM, BN, WGM, WGN, EPI_SWIGLU, NPART, SB>, grid, nt, lds, s, A, W, M, N, K, tm, tn, ep, kb_per);
      break;
  }
}

template <int BM, int BN, int WGM, int WGN, int NPART = 1, bool SB = false>
static void gemm_set_lds_limit() {
  const int bytes = (int)gemm_lds_bytes<BM, BN>();
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_STORE_F32, NPART, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_RESID, NPART, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_QKV, NPART, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  (void)hipFuncSetAttribute((const void*)gemm_f16_kernel<BM, BN, WGM, WGN, EPI_SWIGLU, NPART, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// Tiles above 64 KiB of LDS need the per-kernel dynamic limit raised once.
static void gemm_init_attributes() {
  static bool done = false;
  if (done) return;
  done = true;
  gemm_set_lds_limit<256, 256, 2, 4, 1, true>();
  gemm_set_lds_limit<128, 128, 2, 2>();
}

// Tile choice from a sweep of the Llama-3-8B projection shapes at M = 512, 2048
// and 8192 on MI355X: the 8-wave 256 x 256 tile when it still yields at least 192
// tiles, then 128 x 128 with at least 256 tiles (one per CU), else 64 x 64.
// Split-K second pass: out = epilogue(sum over the splits of part[s][m][n]), summed in split
// order.  One thread per 4 consecutive columns (N % 4 == 0), so RoPE partners (2j, 2j+1)
// and SwiGLU gate/up pairs (2c, 2c+1) are in the same thread.
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
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (EPI == EPI_STORE_F32) ep.out_f32[(size_t)m * ep.ld + n + c] = a[c];
    else if (EPI == EPI_RESID) ep.out_f32[(size_t)m * ep.ld + n + c] += a[c];
    else if (EPI == EPI_QKV) epi_qkv<f16_t>(ep, m, n + c, a[c], a[c ^ 1]);
    else if ((c & 1) == 0) epi_swiglu<f16_t>(ep, m, (n + c) >> 1, a[c], a[c + 1]);
  }
}

// Number of K splits for a GEMM: only small-M shapes (weight streaming) whose 64 x 64
// tiles give fewer than 1024 workgroups are split, aiming at about 1024 workgroups, at
// most 8 splits and at least 4 K steps of 64 per split.
int gemm_splitk_count(int M, int N, int K) {
  if (M <= 0 || M > 128 || N % 4 != 0) return 1;
  const long tiles = (long)((M + 63) / 64) * ((N + 63) / 64);
  if (tiles >= 1024) return 1;
  const int nkb = (K + GEMM_BK - 1) / GEMM_BK;
  int sp = (int)std::min<long>(8, (1024 + tiles - 1) / tiles);
  sp = std::min(sp, nkb / 4);
  if (sp < 2) return 1;
  const int per = (nkb + sp - 1) / sp;
  return (nkb + per - 1) / per;
}

size_t gemm_splitk_floats(int M, int N, int K) {
  const int sp = gemm_splitk_count(M, N, K);
  return sp > 1 ? (size_t)sp * M * N : 0;
}

// Tile choice from a sweep of the Llama-3-8B projection shapes at M = 512, 2048
// and 8192 on MI355X: the 8-wave 256 x 256 tile when it still yields at least 192
// tiles, then 128 x 128 with at least 256 tiles (one per CU), else 64 x 64, split
// over K when even those are too few.
void launch_gemm_f16(const void* A, const void* W, int M, int N, int K, const EpiParams& ep, float* splitk_ws,
                     size_t splitk_ws_floats, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  gemm_init_attributes();
  const f16_t* a = (const f16_t*)A;
  const f16_t* w = (const f16_t*)W;
  auto tiles = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int sp = gemm_splitk_count(M, N, K);
  if (sp > 1 && splitk_ws && (size_t)sp * M * N <= splitk_ws_floats) {
    EpiParams pe = ep;
    pe.kind = EPI_STORE_F32;
    pe.out_f32 = splitk_ws;
    pe.ld = N;
    gemm_dispatch<64, 64, 2, 2>(a, w, M, N, K, pe, s, sp);
    const size_t n4 = (size_t)M * N / 4;
    const dim3 grid((unsigned)((n4 + 255) / 256));
    switch (ep.kind) {
      case EPI_STORE_F32: launch_k(splitk_reduce_kernel<EPI_STORE_F32>, grid, 256, 0, s, splitk_ws, sp, M, N, ep); break;
      case EPI_RESID: launch_k(splitk_reduce_kernel<EPI_RESID>, grid, 256, 0, s, splitk_ws, sp, M, N, ep); break;
      case EPI_QKV: launch_k(splitk_reduce_kernel<EPI_QKV>, grid, 256, 0, s, splitk_ws, sp, M, N, ep); break;
      case EPI_SWIGLU: launch_k(splitk_reduce_kernel<EPI_SWIGLU>, grid, 256, 0, s, splitk_ws, sp, M, N, ep); break;
    }
    return;
  }
  // The q|k|v epilogue (RoPE table reads, cache addressing) does not fit the 256 x 256
  // tile's registers (it spills), so that projection stays on 128 x 128 tiles.
  if (M > 128 && ep.kind != EPI_QKV && tiles(256, 256) >= 192)
    gemm_dispatch<256, 256, 2, 4, 1, true>(a, w, M, N, K, ep, s);
  else if (M > 64 && tiles(128, 128) >= 256)
    gemm_dispatch<128, 128, 2, 2>(a, w, M, N, K, ep, s);
  else
    gemm_dispatch<64, 64, 2, 2>(a, w, M, N, K, ep, s);
}

}  // namespace llm
