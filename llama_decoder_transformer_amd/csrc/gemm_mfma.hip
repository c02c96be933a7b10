// Projections on the matrix cores: C[m][n] = sum_k A[m][k] * W[n][k] with fp16
// operands and fp32 accumulation, A = activations [M][K], W = weights [N][K]
// (both K-major, so both operands are staged into LDS with 16-byte row loads).
// The bf16 weights are held as fp16 (converted exactly at init) and activations
// are rounded to fp16 rather than bf16: same bytes and MFMA rate, 8x finer
// rounding, which keeps 32 layers within the bf16 parity bar.
//
// Tiling: BM x BN output tile per 256-thread workgroup (4 waves as 2 x 2), BK =
// 64 per stage, v_mfma_f32_16x16x32_f16 on 16x16 blocks.  A lane feeds row
// (lane % 16) and the 8 k-values starting at 8 * (lane / 16) of a 16x32 block;
// it receives rows 4 * (lane / 16) + r, r = 0..3, of column lane % 16 of the
// 16x16 result.  The epilogue therefore sees RoPE partners (columns 2j, 2j+1)
// and SwiGLU gate/up pairs (packed columns 2c, 2c+1) in lanes l and l ^ 1.
// LDS rows are padded by 16 bytes so the fragment reads of 16 consecutive rows
// spread over the banks.
#include "common.h"
#include "epilogue.h"
#include "launch.h"

namespace llm {

template <int BM, int BN, int EPI>
__global__ void __launch_bounds__(256) gemm_f16_kernel(const f16_t* __restrict__ A, const f16_t* __restrict__ W,
                                                        int M, int N, int K, EpiParams ep) {
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;  // padded LDS row (144 bytes)
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * BK / 8 / 256;  // 16-byte loads per thread per stage
  constexpr int B_LD = BN * BK / 8 / 256;
  static_assert(A_LD >= 1 && B_LD >= 1, "tile too small for 256 threads");

  __shared__ __attribute__((aligned(16))) f16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) f16_t Bs[BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tm = blockIdx.y * BM, tn = blockIdx.x * BN;
  const int l16 = lane & 15, lg = lane >> 4;

  u32x4_t ra[A_LD], rb[B_LD];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + i * 256, r = idx >> 3, c = (idx & 7) * 8;
      const int gm = tm + r, gk = k0 + c;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const u32x4_t*>(A + (size_t)gm * K + gk) : zero;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + i * 256, r = idx >> 3, c = (idx & 7) * 8;
      const int gn = tn + r, gk = k0 + c;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const u32x4_t*>(W + (size_t)gn * K + gk) : zero;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int idx = tid + i * 256, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&As[r * LDK + c]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int idx = tid + i * 256, r = idx >> 3, c = (idx & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&Bs[r * LDK + c]) = rb[i];
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      f16x8_t af[FM], bw[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const f16x8_t*>(&As[(wm * WM + i * 16 + l16) * LDK + ks * 32 + lg * 8]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bw[j] = *reinterpret_cast<const f16x8_t*>(&Bs[(wn * WN + j * 16 + l16) * LDK + ks * 32 + lg * 8]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bw[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = tm + wm * WM + i * 16 + lg * 4 + r;
        const int n = tn + wn * WN + j * 16 + l16;
        const float v = acc[i][j][r];
        if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
          const float vp = __shfl_xor(v, 1);
          if (m < M && n < N) {
            if (EPI == EPI_QKV) epi_qkv<f16_t>(ep, m, n, v, vp);
            else if ((n & 1) == 0) epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
          }
        } else if (m < M && n < N) {
          if (EPI == EPI_STORE_F32) ep.out_f32[(size_t)m * ep.ld + n] = v;
          else ep.out_f32[(size_t)m * ep.ld + n] += v;
        }
      }
    }
  }
}

template <int BM, int BN>
static void gemm_dispatch(const f16_t* A, const f16_t* W, int M, int N, int K, const EpiParams& ep, hipStream_t s) {
  dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM);
  switch (ep.kind) {
    case EPI_STORE_F32: gemm_f16_kernel<BM, BN, EPI_STORE_F32><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_RESID: gemm_f16_kernel<BM, BN, EPI_RESID><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_QKV: gemm_f16_kernel<BM, BN, EPI_QKV><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
    case EPI_SWIGLU: gemm_f16_kernel<BM, BN, EPI_SWIGLU><<<grid, 256, 0, s>>>(A, W, M, N, K, ep); break;
  }
}

void launch_gemm_f16(const void* A, const void* W, int M, int N, int K, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (M > 64 && tiles128 >= 512)
    gemm_dispatch<128, 128>((const f16_t*)A, (const f16_t*)W, M, N, K, ep, s);
  else
    gemm_dispatch<64, 64>((const f16_t*)A, (const f16_t*)W, M, N, K, ep, s);
}

}  // namespace llm
