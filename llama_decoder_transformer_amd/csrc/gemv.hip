// Small-M projections (decode steps, tiny prefills): y[m][n] = sum_k a[m][k] * W[n][k].
//
// Batch-1 decode is bound by streaming the weight matrix from HBM once, so each
// wave owns RPW consecutive weight rows and walks K with 16-byte loads per lane
// (a wave reads 1 KiB of one row per load instruction), keeping RPW * UNROLL
// loads in flight.  The activations (at most MR rows) are re-read from L1/L2.
// Partial sums are reduced across the wave with xor shuffles; the epilogue
// (RoPE / cache write, SwiGLU, residual add, fp32 store) is applied by one lane
// per output.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace llm {

template <typename T, int MR, int RPW, int EPI>
__global__ void __launch_bounds__(256) gemv_kernel(const T* __restrict__ A, const T* __restrict__ W, int M,
                                                   int N, int K, EpiParams ep) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int n0 = wave * RPW;
  if (n0 >= N) return;
  const int m0 = blockIdx.y * MR;
  const int mrows = min(MR, M - m0);

  const T* wr[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) wr[r] = W + (size_t)min(n0 + r, N - 1) * K;

  float acc[MR][RPW];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[i][r] = 0.f;

#pragma unroll 2
  for (int k = lane * 8; k < K; k += WAVE * 8) {
    float w[RPW][8];
#pragma unroll
    for (int r = 0; r < RPW; ++r) load8(wr[r] + k, w[r]);
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      if (i < mrows) {
        float a[8];
        load8(A + (size_t)(m0 + i) * K + k, a);
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[i][r] = fmaf(a[e], w[r][e], acc[i][r]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[i][r] = wave_sum(acc[i][r]);

#pragma unroll
  for (int i = 0; i < MR; ++i) {
    if (i >= mrows) break;
    const int m = m0 + i;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int n = n0 + r;
      if (lane != (i * RPW + r) % WAVE || n >= N) continue;
      const float v = acc[i][r];
      if (EPI == EPI_STORE_F32) {
        ep.out_f32[(size_t)m * ep.ld + n] = v;
      } else if (EPI == EPI_RESID) {
        ep.out_f32[(size_t)m * ep.ld + n] += v;
      } else if (EPI == EPI_QKV) {
        epi_qkv<T>(ep, m, n, v, acc[i][r ^ 1]);
      } else if (EPI == EPI_SWIGLU) {
        if ((r & 1) == 0) epi_swiglu<T>(ep, m, n >> 1, v, acc[i][r + 1]);
      }
    }
  }
}

template <typename T, int MR, int RPW>
static void gemv_dispatch(const T* A, const T* W, int M, int N, int K, const EpiParams& ep, hipStream_t s) {
  const int waves = (N + RPW - 1) / RPW;
  dim3 grid((waves + 3) / 4, (M + MR - 1) / MR);
  switch (ep.kind) {
    case EPI_STORE_F32: gemv_kernel<T, MR, RPW, EPI_STORE_F32><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_RESID: gemv_kernel<T, MR, RPW, EPI_RESID><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_QKV: gemv_kernel<T, MR, RPW, EPI_QKV><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_SWIGLU: gemv_kernel<T, MR, RPW, EPI_SWIGLU><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
  }
}

void launch_gemv(int dtype, const void* A, const void* W, int M, int N, int K, const EpiParams& ep,
                 hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (dtype == 1) {
    if (M == 1)
      gemv_dispatch<bf16_t, 1, 4>((const bf16_t*)A, (const bf16_t*)W, M, N, K, ep, s);
    else if (M <= 4)
      gemv_dispatch<bf16_t, 4, 4>((const bf16_t*)A, (const bf16_t*)W, M, N, K, ep, s);
    else
      gemv_dispatch<bf16_t, 8, 2>((const bf16_t*)A, (const bf16_t*)W, M, N, K, ep, s);
  } else {
    if (M == 1)
      gemv_dispatch<float, 1, 4>((const float*)A, (const float*)W, M, N, K, ep, s);
    else if (M <= 4)
      gemv_dispatch<float, 4, 4>((const float*)A, (const float*)W, M, N, K, ep, s);
    else
      gemv_dispatch<float, 8, 2>((const float*)A, (const float*)W, M, N, K, ep, s);
  }
}

}  // namespace llm
