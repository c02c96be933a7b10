// Small-M projections (decode steps, tiny prefills): y[m][n] = sum_k a[m][k] * W[n][k].
//
// Batch-1 decode is bound by streaming each weight matrix from HBM once.  A
// 256-thread block owns R consecutive weight rows; its 4 waves split K into
// 512-element chunks taken round-robin, each lane loading 16 bytes of every row
// per chunk (a wave reads 1 KiB of a row per load instruction).  Two chunks are
// in flight at a time, so 2 * R loads per lane are outstanding.  Partial sums are reduced
// across the wave with xor shuffles and across the 4 waves through LDS, and the
// epilogue (RoPE / cache write, SwiGLU, residual add, fp32 store) runs on the
// R * MR finished values.
//
// With NORM the input is the fp32 residual stream x and the RMSNorm is fused:
// the block accumulates sum_k W[n][k] * (x[k] * g[k]) and sum_k x[k]^2 in the
// same pass and scales by 1 / sqrt(mean(x^2) + eps) at the end (the "rms_norm"
// of the "Building llama3 from scratch" page, distributed over the dot product).
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace llm {

// fp16 pair (round to nearest even) as a 32-bit word.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  f16x2_t h;
  h.x = (f16_t)a;
  h.y = (f16_t)b;
  return __builtin_bit_cast(uint32_t, h);
}

template <typename T, int MR, int R, int EPI, bool NORM>
__global__ void __launch_bounds__(256) gemv_kernel(const void* __restrict__ Ain, const T* __restrict__ W,
                                                   const float* __restrict__ gnorm, float eps, int M, int N, int K,
                                                   EpiParams ep) {
  constexpr int KW = WAVE * 8;
  __shared__ float s_acc[4][MR][R];
  __shared__ float s_ss[4][MR];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n0 = blockIdx.x * R;
  const int m0 = blockIdx.y * MR;
  const int mrows = min(MR, M - m0);

  const T* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = W + (size_t)min(n0 + r, N - 1) * K;

  float acc[MR][R];
  float ss[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;
  }

  const int nchunks = (K + KW - 1) / KW;
#pragma unroll 2
  for (int c = wid; c < nchunks; c += 4) {
    const int k = c * KW + lane * 8;
    if (k < K) {
      float w[R][8];
#pragma unroll
      for (int r = 0; r < R; ++r) load8(wr[r] + k, w[r]);
      float g[8];
      if (NORM) load8(gnorm + k, g);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        if (i < mrows) {
          float a[8];
          if (NORM) {
            load8(reinterpret_cast<const float*>(Ain) + (size_t)(m0 + i) * K + k, a);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              ss[i] = fmaf(a[e], a[e], ss[i]);
              a[e] *= g[e];
            }
          } else {
            load8(reinterpret_cast<const T*>(Ain) + (size_t)(m0 + i) * K + k, a);
          }
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][r] = fmaf(a[e], w[r][e], acc[i][r]);
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MR; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = wave_sum(acc[i][r]);
    if (NORM) ss[i] = wave_sum(ss[i]);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_acc[wid][i][r] = acc[i][r];
      s_ss[wid][i] = ss[i];
    }
  }
  __syncthreads();

  const int t = threadIdx.x;
  if (t < MR * R) {
    const int i = t / R, r = t % R;
    const int m = m0 + i, n = n0 + r;
    if (i < mrows && n < N) {
      float v = s_acc[0][i][r] + s_acc[1][i][r] + s_acc[2][i][r] + s_acc[3][i][r];
      float vp = s_acc[0][i][r ^ 1] + s_acc[1][i][r ^ 1] + s_acc[2][i][r ^ 1] + s_acc[3][i][r ^ 1];
      if (NORM) {
        const float tot = s_ss[0][i] + s_ss[1][i] + s_ss[2][i] + s_ss[3][i];
        const float inv = 1.0f / sqrtf(tot / (float)K + eps);
        v *= inv;
        vp *= inv;
      }
      if (EPI == EPI_STORE_F32) {
        ep.out_f32[(size_t)m * ep.ld + n] = v;
      } else if (EPI == EPI_RESID) {
        ep.out_f32[(size_t)m * ep.ld + n] += v;
      } else if (EPI == EPI_QKV) {
        epi_qkv<T>(ep, m, n, v, vp);
      } else if (EPI == EPI_SWIGLU) {
        if ((r & 1) == 0) epi_swiglu<T>(ep, m, n >> 1, v, vp);
      }
    }
  }
}

// fp16 weights (the bf16-weight path): the same scheme with the weights kept as
// raw 16-byte words until use, so two chunks x R rows of loads (2R per lane) are
// issued before any math.  The products use the packed fp16 dot instruction (two
// products per lane per instruction, fp32 accumulation): fp16 activations are
// used as loaded, and with the fused norm x * g is rounded to fp16 once, as the
// separate RMSNorm of the matrix-core path rounds its output.

template <int MR, int R, int EPI, bool NORM>
__global__ void __launch_bounds__(256) gemv_h_kernel(const void* __restrict__ Ain, const f16_t* __restrict__ W,
                                                        const float* __restrict__ gnorm, float eps, int M, int N,
                                                        int K, EpiParams ep) {
  constexpr int KW = WAVE * 8;
  __shared__ float s_acc[4][MR][R];
  __shared__ float s_ss[4][MR];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n0 = blockIdx.x * R;
  const int m0 = blockIdx.y * MR;
  const int mrows = min(MR, M - m0);

  // Epilogue inputs that do not depend on the dot products (the residual being
  // added to, RoPE position / slot / cos / sin) are fetched before the weight
  // stream so they do not add a dependent round trip after it.
  const int et = threadIdx.x;
  const int ei = et / R, er = et % R;
  const bool ethread = et < MR * R && ei < mrows && n0 + er < N;
  float e_resid = 0.f;
  QkvPrep e_qkv = {};
  if (ethread) {
    if (EPI == EPI_RESID) e_resid = ep.out_f32[(size_t)(m0 + ei) * ep.ld + n0 + er];
    if (EPI == EPI_QKV) e_qkv = qkv_prepare(ep, m0 + ei, n0 + er);
  }

  const f16_t* wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wr[r] = W + (size_t)min(n0 + r, N - 1) * K;

  float acc[MR][R];
  float ss[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    ss[i] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;
  }
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  const int nchunks = (K + KW - 1) / KW;
  for (int c0 = wid; c0 < nchunks; c0 += 8) {
    int kk[2];
    bool ok[2];
    u32x4_t wraw[2][R];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kk[u] = (c0 + 4 * u) * KW + lane * 8;
      ok[u] = kk[u] < K;
#pragma unroll
      for (int r = 0; r < R; ++r)
        wraw[u][r] = ok[u] ? *reinterpret_cast<const u32x4_t*>(wr[r] + kk[u]) : zero;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!ok[u]) continue;
      float g[8];
      if (NORM) load8(gnorm + kk[u], g);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        if (i < mrows) {
          // the 8 activations of this lane as 4 fp16 pairs
          uint32_t ah[4];
          if (NORM) {
            float a[8];
            load8(reinterpret_cast<const float*>(Ain) + (size_t)(m0 + i) * K + kk[u], a);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss[i] = fmaf(a[e], a[e], ss[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ah[e] = pack_h2(a[2 * e] * g[2 * e], a[2 * e + 1] * g[2 * e + 1]);
          } else {
            const u32x4_t raw =
                *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const f16_t*>(Ain) + (size_t)(m0 + i) * K + kk[u]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ah[e] = raw[e];
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t wv = wraw[u][r][e];
              acc[i][r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ah[e]), __builtin_bit_cast(f16x2_t, wv),
                                                 acc[i][r], false);
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MR; ++i) {
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = wave_sum(acc[i][r]);
    if (NORM) ss[i] = wave_sum(ss[i]);
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_acc[wid][i][r] = acc[i][r];
      s_ss[wid][i] = ss[i];
    }
  }
  __syncthreads();

  if (ethread) {
    const int i = ei, r = er;
    const int m = m0 + i, n = n0 + r;
    float v = s_acc[0][i][r] + s_acc[1][i][r] + s_acc[2][i][r] + s_acc[3][i][r];
    float vp = s_acc[0][i][r ^ 1] + s_acc[1][i][r ^ 1] + s_acc[2][i][r ^ 1] + s_acc[3][i][r ^ 1];
    if (NORM) {
      const float tot = s_ss[0][i] + s_ss[1][i] + s_ss[2][i] + s_ss[3][i];
      const float inv = 1.0f / sqrtf(tot / (float)K + eps);
      v *= inv;
      vp *= inv;
    }
    if (EPI == EPI_STORE_F32) {
      ep.out_f32[(size_t)m * ep.ld + n] = v;
    } else if (EPI == EPI_RESID) {
      ep.out_f32[(size_t)m * ep.ld + n] = e_resid + v;
    } else if (EPI == EPI_QKV) {
      qkv_store<f16_t>(ep, e_qkv, m, n, v, vp);
    } else if (EPI == EPI_SWIGLU) {
      if ((r & 1) == 0) epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
    }
  }
}

template <int MR, int R, bool NORM>
static void gemv_h_dispatch(const void* A, const f16_t* W, const float* g, float eps, int M, int N, int K,
                               const EpiParams& ep, hipStream_t s) {
  dim3 grid((N + R - 1) / R, (M + MR - 1) / MR);
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemv_h_kernel<MR, R, EPI_STORE_F32, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep);
      break;
    case EPI_RESID: launch_k(gemv_h_kernel<MR, R, EPI_RESID, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
    case EPI_QKV: launch_k(gemv_h_kernel<MR, R, EPI_QKV, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
    case EPI_SWIGLU: launch_k(gemv_h_kernel<MR, R, EPI_SWIGLU, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
  }
}

template <typename T, int MR, int R, bool NORM>
static void gemv_dispatch(const void* A, const T* W, const float* g, float eps, int M, int N, int K,
                          const EpiParams& ep, hipStream_t s) {
  dim3 grid((N + R - 1) / R, (M + MR - 1) / MR);
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemv_kernel<T, MR, R, EPI_STORE_F32, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep);
      break;
    case EPI_RESID: launch_k(gemv_kernel<T, MR, R, EPI_RESID, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
    case EPI_QKV: launch_k(gemv_kernel<T, MR, R, EPI_QKV, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
    case EPI_SWIGLU: launch_k(gemv_kernel<T, MR, R, EPI_SWIGLU, NORM>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
  }
}

template <bool NORM>
static void gemv_h_pick(const void* A, const f16_t* W, const float* g, float eps, int M, int N, int K,
                           const EpiParams& ep, hipStream_t s) {
  // Rows per block for M = 1, from a sweep of the Llama-3-8B projection shapes on MI355X:
  // LM head (N >= 64K) 16, gate-up (N >= 16K) 8, long-K down projection 2, q|k|v 8, wo 2.
  if (M == 1) {
    if (N >= 65536) gemv_h_dispatch<1, 16, NORM>(A, W, g, eps, M, N, K, ep, s);
    else if (N >= 16384) gemv_h_dispatch<1, 8, NORM>(A, W, g, eps, M, N, K, ep, s);
    else if (K >= 8192) gemv_h_dispatch<1, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
    else if (N >= 6144) gemv_h_dispatch<1, 8, NORM>(A, W, g, eps, M, N, K, ep, s);
    else gemv_h_dispatch<1, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
  } else if (M <= 4) {
    gemv_h_dispatch<4, 4, NORM>(A, W, g, eps, M, N, K, ep, s);
  } else {
    gemv_h_dispatch<8, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
  }
}

template <bool NORM>
static void gemv_f32_pick(const void* A, const float* W, const float* g, float eps, int M, int N, int K,
                          const EpiParams& ep, hipStream_t s) {
  if (M == 1) gemv_dispatch<float, 1, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
  else if (M <= 4) gemv_dispatch<float, 4, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
  else gemv_dispatch<float, 8, 2, NORM>(A, W, g, eps, M, N, K, ep, s);
}

void launch_gemv(int dtype, const void* A, const void* W, const float* norm_w, float eps, int M, int N, int K,
                 const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (dtype == 1) {
    if (norm_w) gemv_h_pick<true>(A, (const f16_t*)W, norm_w, eps, M, N, K, ep, s);
    else gemv_h_pick<false>(A, (const f16_t*)W, nullptr, eps, M, N, K, ep, s);
  } else {
    if (norm_w) gemv_f32_pick<true>(A, (const float*)W, norm_w, eps, M, N, K, ep, s);
    else gemv_f32_pick<false>(A, (const float*)W, nullptr, eps, M, N, K, ep, s);
  }
}

}  // namespace llm
