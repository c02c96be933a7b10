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
// With NORM the input is the fp32 residual stream x and the RMSNorm is fused (the
// "rms_norm" of the "Building llama3 from scratch" page): the fp32 kernel accumulates
// sum_k W[n][k] * (x[k] * g[k]) and sum_k x[k]^2 in the same pass and scales by
// 1 / sqrt(mean(x^2) + eps) at the end; the fp16 kernel first takes sum_k x[k]^2 of
// its rows and then multiplies by the normalised activations, rounded to fp16 as the
// separate RMSNorm kernel rounds them.
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
// raw 16-byte words until use, so U chunks x R rows of loads (U R per lane) are
// issued before any math.  The products use the packed fp16 dot instruction (two
// products per lane per instruction, fp32 accumulation) on fp16 activations.
//
// With the fused norm, the block first sums x^2 over its rows (fp32, through LDS),
// with the first chunks' weight loads already in flight, and the loop then uses
// fp16(x * inv_rms * g), as the separate RMSNorm kernel of the matrix-core path
// rounds its output, so a large residual cannot overflow fp16 before it is scaled
// down.  A normalised value outside fp16's range raises LLM_DEVERR_RANGE.

template <int MR, int R, int EPI, bool NORM, int U>
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
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;
  const int nchunks = (K + KW - 1) / KW;
  // Wave w takes chunks w, w + 4, ..., w + 4 (U - 1) of 512 elements per round (U chunks x R
  // rows of weights in flight per lane).
  int kk[U];
  bool ok[U];
  u32x4_t wraw[U][R];
  // The round's other operands travel with its weights: the norm weight (with the norm) or the
  // fp16 activations (without, up to 2 rows: more would cost occupancy), issued first so they
  // land first.  Loaded inside the product loop, under its chunk test, each cost a round trip of
  // its own after the weights had landed.
  constexpr bool HOIST_A = !NORM && MR <= 2;
  f32x4_t graw[NORM ? U : 1][2];
  u32x4_t araw[HOIST_A ? U : 1][HOIST_A ? MR : 1];
  // Every load below is unconditional, from an address clamped into the row (K % 8 == 0), and
  // a chunk past the row's end is skipped at use: with no load under a branch the compiler
  // counts the loads in flight exactly and waits only for the ones it needs.
  auto load_w = [&](int c0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kk[u] = (c0 + 4 * u) * KW + lane * 8;
      ok[u] = kk[u] < K;
      const int kc = min(kk[u], K - 8);
      if constexpr (NORM) {
        graw[u][0] = *reinterpret_cast<const f32x4_t*>(gnorm + kc);
        graw[u][1] = *reinterpret_cast<const f32x4_t*>(gnorm + kc + 4);
      } else if constexpr (HOIST_A) {
#pragma unroll
        for (int i = 0; i < MR; ++i)
          araw[u][i] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const f16_t*>(Ain) +
                                                         (size_t)(m0 + min(i, mrows - 1)) * K + kc);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) wraw[u][r] = *reinterpret_cast<const u32x4_t*>(wr[r] + kc);
    }
  };
  const float* const xin = reinterpret_cast<const float*>(Ain);

  // With the norm: this lane's residual values of the first round's U chunks are loaded
  // first (the loop's element mapping, kept in registers for it), then the weights.  Loads
  // complete in issue order, so the statistics below wait for x only, not for the weights.
  float xa[NORM ? MR : 1][NORM ? U : 1][8];
  if (NORM) {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = min((wid + 4 * u) * KW + lane * 8, K - 8);
        load8(xin + (size_t)(m0 + min(i, mrows - 1)) * K + k, xa[i][u]);
      }
  }
  load_w(min(wid, nchunks - 1));

  float inv[MR];
  bool range_bad = false;
  if (NORM) {
    float ss[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      ss[i] = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if ((wid + 4 * u) * KW + lane * 8 >= K) continue;  // clamped duplicate of another chunk
#pragma unroll
        for (int e = 0; e < 8; ++e) ss[i] = fmaf(xa[i][u][e], xa[i][u][e], ss[i]);
      }
      // rows longer than one round: the rest of this lane's chunks
      if (i < mrows) {
        for (int c = wid + 4 * U; c < nchunks; c += 4) {
          const int k = c * KW + lane * 8;
          if (k < K) {
            float a[8];
            load8(xin + (size_t)(m0 + i) * K + k, a);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss[i] = fmaf(a[e], a[e], ss[i]);
          }
        }
      }
      ss[i] = wave_sum(ss[i]);
    }
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < MR; ++i) s_ss[wid][i] = ss[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      const float tot = s_ss[0][i] + s_ss[1][i] + s_ss[2][i] + s_ss[3][i];
      inv[i] = 1.0f / sqrtf(tot / (float)K + eps);
    }
  }

  for (int c0 = wid; c0 < nchunks; c0 += 4 * U) {
    const bool first = c0 == wid;
    if (!first) load_w(c0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;
      float g[8];
      if (NORM) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[e] = graw[u][0][e];
          g[4 + e] = graw[u][1][e];
        }
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        if (i < mrows) {
          // the 8 activations of this lane as 4 fp16 pairs
          uint32_t ah[4];
          if (NORM) {
            float a[8];
            if (first) {
#pragma unroll
              for (int e = 0; e < 8; ++e) a[e] = xa[i][u][e];
            } else {
              load8(xin + (size_t)(m0 + i) * K + kk[u], a);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              a[e] = a[e] * inv[i] * g[e];
              range_bad |= f16_out_of_range(a[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ah[e] = pack_h2(a[2 * e], a[2 * e + 1]);
          } else {
            u32x4_t raw;
            if constexpr (HOIST_A)
              raw = araw[u][i];
            else
              raw = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const f16_t*>(Ain) + (size_t)(m0 + i) * K +
                                                      kk[u]);
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
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < MR; ++i) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_acc[wid][i][r] = acc[i][r];
    }
  }
  __syncthreads();

  unsigned long long akey = 0ull;
  if (ethread) {
    const int i = ei, r = er;
    const int m = m0 + i, n = n0 + r;
    const float v = s_acc[0][i][r] + s_acc[1][i][r] + s_acc[2][i][r] + s_acc[3][i][r];
    const float vp = s_acc[0][i][r ^ 1] + s_acc[1][i][r ^ 1] + s_acc[2][i][r ^ 1] + s_acc[3][i][r ^ 1];
    if (EPI == EPI_STORE_F32) {
      ep.out_f32[(size_t)m * ep.ld + n] = v;
      akey = argmax_key(v, n);
    } else if (EPI == EPI_RESID) {
      ep.out_f32[(size_t)m * ep.ld + n] = e_resid + v;
    } else if (EPI == EPI_QKV) {
      range_bad |= qkv_store<f16_t>(ep, e_qkv, m, n, v, vp);
    } else if (EPI == EPI_SWIGLU) {
      if ((r & 1) == 0) range_bad |= epi_swiglu<f16_t>(ep, m, n >> 1, v, vp);
    }
  }
  // The LM head of a generation step: the best (logit, index) of each row's R logits here goes
  // into one of the row's AMAX_REP keys (the epilogue threads of a row are R consecutive lanes of
  // wave 0, R a power of two).
  if (EPI == EPI_STORE_F32 && ep.amax_keys && et < 64) {
#pragma unroll
    for (int o = 1; o < R; o <<= 1) {
      const unsigned long long other = __shfl_xor(akey, o);
      akey = other > akey ? other : akey;
    }
    if (ethread && er == 0) ep.amax_keys[(size_t)(m0 + ei) * gridDim.x + blockIdx.x] = akey;
  }
  raise_range_error(ep, range_bad);
}

template <int MR, int R, bool NORM, int U = 2>
static void gemv_h_dispatch(const void* A, const f16_t* W, const float* g, float eps, int M, int N, int K,
                               const EpiParams& ep, hipStream_t s) {
  dim3 grid((N + R - 1) / R, (M + MR - 1) / MR);
  switch (ep.kind) {
    case EPI_STORE_F32:
      launch_k(gemv_h_kernel<MR, R, EPI_STORE_F32, NORM, U>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep);
      break;
    case EPI_RESID:
      launch_k(gemv_h_kernel<MR, R, EPI_RESID, NORM, U>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep);
      break;
    case EPI_QKV: launch_k(gemv_h_kernel<MR, R, EPI_QKV, NORM, U>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep); break;
    case EPI_SWIGLU:
      launch_k(gemv_h_kernel<MR, R, EPI_SWIGLU, NORM, U>, grid, 256, 0, s, A, W, g, eps, M, N, K, ep);
      break;
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

// Rows per block (and chunks per round) of the fp16 GEMV.  For M = 1, from sweeps of the
// Llama-3-8B projection shapes on MI355X in the full decode step: LM head (N >= 64K) 16; gate-up
// (N >= 16K) 6 (36.58 us against 36.83 with 8, 38.1-39.0 with 4, 12 or 16, or 8 rows one chunk per
// round); long-K down projection 2 rows with the whole row, 7 chunks, in one round (19.48 us
// against 20.11 with 4 chunks per round, 20.3-20.9 with 1 or 4 rows or 2 chunks per round);
// q|k|v 8, wo 2.  (Before the activations travelled with the weights, 4 chunks per round was the
// better down projection: 20.4 us against 22.0.)
enum class GemvPlan { M1_R16, M1_R6, M1_R8, M1_R2_U7, M1_R2, M4_R4, M8_R2 };

static GemvPlan gemv_h_plan(int M, int N, int K) {
  if (M == 1) {
    if (N >= 65536) return GemvPlan::M1_R16;
    if (N >= 16384) return GemvPlan::M1_R6;
    if (K >= 8192) return GemvPlan::M1_R2_U7;
    if (N >= 6144) return GemvPlan::M1_R8;
    return GemvPlan::M1_R2;
  }
  return M <= 4 ? GemvPlan::M4_R4 : GemvPlan::M8_R2;
}

int gemv_h_blocks(int M, int N, int K) {
  switch (gemv_h_plan(M, N, K)) {
    case GemvPlan::M1_R16: return (N + 15) / 16;
    case GemvPlan::M1_R6: return (N + 5) / 6;
    case GemvPlan::M1_R8: return (N + 7) / 8;
    case GemvPlan::M4_R4: return (N + 3) / 4;
    default: return (N + 1) / 2;
  }
}

template <bool NORM>
static void gemv_h_pick(const void* A, const f16_t* W, const float* g, float eps, int M, int N, int K,
                           const EpiParams& ep, hipStream_t s) {
  switch (gemv_h_plan(M, N, K)) {
    case GemvPlan::M1_R16: gemv_h_dispatch<1, 16, NORM>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M1_R6: gemv_h_dispatch<1, 6, NORM>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M1_R8: gemv_h_dispatch<1, 8, NORM>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M1_R2_U7: gemv_h_dispatch<1, 2, NORM, 7>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M1_R2: gemv_h_dispatch<1, 2, NORM>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M4_R4: gemv_h_dispatch<4, 4, NORM>(A, W, g, eps, M, N, K, ep, s); break;
    case GemvPlan::M8_R2: gemv_h_dispatch<8, 2, NORM>(A, W, g, eps, M, N, K, ep, s); break;
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
