// Embedding gather, RMSNorm, greedy argmax and small bookkeeping kernels.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace llm {

// ---------------------------------------------------------------- embedding
// Row m of the residual stream is row tok[m] of tok_embeddings, widened to fp32
// (embedding lookup of the "Building llama3 from scratch" page).
template <typename TW>
__global__ void __launch_bounds__(256) embed_kernel(const TW* __restrict__ emb, const int* __restrict__ tok,
                                                    int dim, int vocab, float* __restrict__ x, int* err, int* zero,
                                                    int n_zero, int zero_stride) {
  const int m = blockIdx.x;
  if (m == 0)
    for (int i = threadIdx.x; i < n_zero; i += blockDim.x) zero[(size_t)i * zero_stride] = 0;
  const int t = tok[m];
  float* xr = x + (size_t)m * dim;
  if (t < 0 || t >= vocab) {
    if (threadIdx.x == 0) atomicOr(err, 1);
    for (int i = threadIdx.x; i < dim; i += blockDim.x) xr[i] = 0.f;
    return;
  }
  const TW* er = emb + (size_t)t * dim;
  // 16-byte loads, UN of them per thread per pass, all issued before any is stored (indices
  // clamped into the row; dim % 8 == 0): a Llama-3-8B row (4096 fp16) is one pass of one round
  // trip instead of four dependent ones.
  constexpr int EPL = 16 / sizeof(TW), UN = 4;
  const int step = blockDim.x * EPL;
  for (int i0 = threadIdx.x * EPL; i0 < dim; i0 += UN * step) {
    u32x4_t raw[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) raw[u] = *reinterpret_cast<const u32x4_t*>(er + min(i0 + u * step, dim - EPL));
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = i0 + u * step;
      if (i >= dim) continue;
      float f[EPL];
      if constexpr (sizeof(TW) == 2) {
        f16x8_to_f32(raw[u], f);
      } else {
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          const uint32_t w = raw[u][k];  // through a scalar (see f16x8_to_f32)
          f[k] = __uint_as_float(w);
        }
      }
#pragma unroll
      for (int k = 0; k < EPL; ++k) xr[i + k] = f[k];
    }
  }
}

void launch_embed(int dtype, const void* emb, const int* tokens, int M, int dim, int vocab, float* x,
                  int* err, hipStream_t s, int* zero, int n_zero, int zero_stride) {
  if (M <= 0) return;
  if (!zero) n_zero = 0;
  if (dtype == 1)
    launch_k(embed_kernel<f16_t>, M, 256, 0, s, (const f16_t*)emb, tokens, dim, vocab, x, err, zero, n_zero,
             zero_stride);
  else
    launch_k(embed_kernel<float>, M, 256, 0, s, (const float*)emb, tokens, dim, vocab, x, err, zero, n_zero,
             zero_stride);
}

// ---------------------------------------------------------------- RMSNorm
// y = x / sqrt(mean(x^2) + eps) * w per row ("rms_norm" on the "Building llama3
// from scratch" page), fp32 statistics, one rounding to the output dtype.  One 256-thread
// workgroup per row; thread t holds float4 j of the row at element 4 (t + 256 j) in registers
// (V4 of them, dim <= 1024 V4), so all of a row's loads, and the norm weight's, are in flight
// together and x is read once.
template <typename TO, int V4>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                      int dim, float eps, TO* __restrict__ y, int* err) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * dim;
  f32x4_t v[V4], g[V4];
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i = (threadIdx.x + 256 * j) * 4;
    v[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    g[j] = v[j];
    if (i < dim) {
      v[j] = *reinterpret_cast<const f32x4_t*>(xr + i);
      g[j] = *reinterpret_cast<const f32x4_t*>(w + i);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < V4; ++j) ss += v[j][0] * v[j][0] + v[j][1] * v[j][1] + v[j][2] * v[j][2] + v[j][3] * v[j][3];
  ss = wave_sum(ss);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)dim + eps);
  TO* yr = y + (size_t)m * dim;
  bool bad = false;
#pragma unroll
  for (int j = 0; j < V4; ++j) {
    const int i = (threadIdx.x + 256 * j) * 4;
    if (i < dim) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float o = v[j][k] * inv * g[j][k];
        bad |= store_out_of_range<TO>(o);
        yr[i + k] = from_f32<TO>(o);
      }
    }
  }
  if (bad) atomicOr(err, LLM_DEVERR_RANGE_BIT);
}

// Rows wider than the register version holds (dim > 16384): the same arithmetic in loops.
template <typename TO>
__global__ void __launch_bounds__(256) rmsnorm_loop_kernel(const float* __restrict__ x, const float* __restrict__ w,
                                                           int dim, float eps, TO* __restrict__ y, int* err) {
  __shared__ float red[8];
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * dim;
  float ss = 0.f;
  for (int i = threadIdx.x * 4; i < dim; i += 256 * 4) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(xr + i);
    ss += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
  }
  ss = wave_sum(ss);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)dim + eps);
  TO* yr = y + (size_t)m * dim;
  bool bad = false;
  for (int i = threadIdx.x * 4; i < dim; i += 256 * 4) {
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(xr + i);
    f32x4_t g = *reinterpret_cast<const f32x4_t*>(w + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float o = v[k] * inv * g[k];
      bad |= store_out_of_range<TO>(o);
      yr[i + k] = from_f32<TO>(o);
    }
  }
  if (bad) atomicOr(err, LLM_DEVERR_RANGE_BIT);
}

template <typename TO>
static void rmsnorm_dispatch(const float* x, const float* w, int M, int dim, float eps, TO* out, int* err,
                             hipStream_t s) {
  if (dim <= 1024) launch_k(rmsnorm_kernel<TO, 1>, M, 256, 0, s, x, w, dim, eps, out, err);
  else if (dim <= 2048) launch_k(rmsnorm_kernel<TO, 2>, M, 256, 0, s, x, w, dim, eps, out, err);
  else if (dim <= 4096) launch_k(rmsnorm_kernel<TO, 4>, M, 256, 0, s, x, w, dim, eps, out, err);
  else if (dim <= 8192) launch_k(rmsnorm_kernel<TO, 8>, M, 256, 0, s, x, w, dim, eps, out, err);
  else if (dim <= 16384) launch_k(rmsnorm_kernel<TO, 16>, M, 256, 0, s, x, w, dim, eps, out, err);
  else launch_k(rmsnorm_loop_kernel<TO>, M, 256, 0, s, x, w, dim, eps, out, err);
}

void launch_rmsnorm(int dtype, const float* x, const float* w, int M, int dim, float eps, void* out, int* err,
                    hipStream_t s) {
  if (M <= 0) return;
  if (dtype == 1)
    rmsnorm_dispatch(x, w, M, dim, eps, (f16_t*)out, err, s);
  else
    rmsnorm_dispatch(x, w, M, dim, eps, (float*)out, err, s);
}

// ---------------------------------------------------------------- small helpers
template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ src, float* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = to_f32<T>(src[i]);
}

void launch_to_f32(int dtype, const void* src, float* dst, size_t n, hipStream_t s) {
  if (n == 0) return;
  unsigned g = (unsigned)((n + 255) / 256);
  if (dtype == 1)
    launch_k(to_f32_kernel<bf16_t>, g, 256, 0, s, (const bf16_t*)src, dst, n);
  else
    launch_k(to_f32_kernel<float>, g, 256, 0, s, (const float*)src, dst, n);
}

// Weight packing for the bf16-weight path: rows of a bf16 matrix are stored as fp16
// (round to nearest even) at destination row r * row_mult + row_off.  The conversion
// is exact for bf16 values whose magnitude lies in fp16's normal range
// [2^-14, 65504]; smaller magnitudes keep fewer significant bits (fp16 subnormals),
// and a magnitude above 65504 (or a non-finite weight) becomes +-inf and raises
// LLM_DEVERR_RANGE.
__global__ void pack_rows_kernel(const bf16_t* __restrict__ src, f16_t* __restrict__ dst, size_t rows, int cols,
                                 int row_mult, int row_off, int* err) {
  const size_t n = rows * (size_t)cols;
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
    const size_t r = i / cols, c = i % cols;
    const float v = bf16_to_f32(src[i]);
    bad |= f16_out_of_range(v);
    dst[(r * row_mult + row_off) * (size_t)cols + c] = (f16_t)v;
  }
  if (bad) atomicOr(err, LLM_DEVERR_RANGE_BIT);
}

void launch_pack_rows(const void* src, void* dst, size_t rows, int cols, int row_mult, int row_off, int* err,
                      hipStream_t s) {
  const size_t n = rows * (size_t)cols;
  if (n == 0) return;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 16384);  // grid-stride beyond 4M elements
  launch_k(pack_rows_kernel, blocks, 256, 0, s, (const bf16_t*)src, (f16_t*)dst, rows, cols, row_mult, row_off,
           err);
}

// Gather of whole rows (the last row of each sequence of a batched prefill).
__global__ void gather_rows_kernel(const float* __restrict__ src, const int* __restrict__ idx, int dim,
                                   float* __restrict__ dst) {
  const int i = blockIdx.x;
  const float* sr = src + (size_t)idx[i] * dim;
  float* dr = dst + (size_t)i * dim;
  for (int c = threadIdx.x; c < dim; c += blockDim.x) dr[c] = sr[c];
}

void launch_gather_rows(const float* src, const int* idx, int n, int dim, float* dst, hipStream_t s) {
  if (n <= 0) return;
  launch_k(gather_rows_kernel, n, 256, 0, s, src, idx, dim, dst);
}

// Batched-prefill metadata from the kernel arguments: workgroup b writes the positions and
// slot of sequence first + b's rows, its last row index and its descriptor.
__global__ void __launch_bounds__(256) seq_meta_kernel(SeqMetaChunk c, int* __restrict__ row_pos,
                                                       int* __restrict__ row_slot, int* __restrict__ last_idx,
                                                       SeqDesc* __restrict__ table) {
  const int b = blockIdx.x;
  const SeqDesc sd = c.d[b];
  for (int i = threadIdx.x; i < sd.n; i += blockDim.x) {
    row_pos[sd.row0 + i] = sd.start + i;
    row_slot[sd.row0 + i] = sd.slot;
  }
  if (threadIdx.x == 0) {
    last_idx[c.first + b] = sd.row0 + sd.n - 1;
    table[c.first + b] = sd;
  }
}

void launch_seq_meta(const SeqMetaChunk& c, int* row_pos, int* row_slot, int* last_idx, SeqDesc* table,
                     hipStream_t s) {
  if (c.count <= 0) return;
  launch_k(seq_meta_kernel, c.count, 256, 0, s, c, row_pos, row_slot, last_idx, table);
}

__global__ void fill_i32_kernel(int* p, int v, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

void launch_fill_i32(int* p, int v, size_t n, hipStream_t s) {
  if (n == 0) return;
  launch_k(fill_i32_kernel, (unsigned)((n + 255) / 256), 256, 0, s, p, v, n);
}

__global__ void advance_kernel(int* positions, const int* tokens, int* out_tokens, int* step, int batch) {
  const int b = threadIdx.x;
  const int st = *step;
  __syncthreads();
  if (b < batch) {
    positions[b] += 1;
    out_tokens[(size_t)st * batch + b] = tokens[b];
  }
  if (b == 0) *step = st + 1;
}

void launch_advance(int* positions, const int* tokens, int* out_tokens, int* step_counter, int batch,
                    hipStream_t s) {
  launch_k(advance_kernel, 1, 1024, 0, s, positions, tokens, out_tokens, step_counter, batch);
}

// One 1024-thread workgroup: per row, the maximum of the LM-head workgroups' keys.
__global__ void __launch_bounds__(1024) advance_keys_kernel(const unsigned long long* __restrict__ keys, int nblk,
                                                            int* positions, int* tokens, int* out_tokens, int* step,
                                                            int batch) {
  __shared__ unsigned long long s_k[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int st = *step;
  for (int b = 0; b < batch; ++b) {
    unsigned long long k = 0ull;
    // 8 loads per thread in flight at a time (from clamped indices; a clamped repeat of a key
    // cannot change the maximum)
    for (int j0 = 0; j0 < nblk; j0 += 8 * 1024) {
      unsigned long long kj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kj[u] = keys[(size_t)b * nblk + min(j0 + u * 1024 + t, nblk - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) k = kj[u] > k ? kj[u] : k;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const unsigned long long other = __shfl_xor(k, o);
      k = other > k ? other : k;
    }
    if (lane == 0) s_k[w] = k;
    __syncthreads();
    if (t == 0) {
      for (int i = 1; i < 16; ++i) k = s_k[i] > k ? s_k[i] : k;
      // no key: every logit was NaN, which the argmax kernels leave at index 0x7FFFFFFF
      const int tok = k ? (int)~(uint32_t)k : 0x7FFFFFFF;
      tokens[b] = tok;
      positions[b] += 1;
      out_tokens[(size_t)st * batch + b] = tok;
    }
    __syncthreads();
  }
  if (t == 0) *step = st + 1;
}

void launch_advance_keys(const unsigned long long* keys, int nblk, int* positions, int* tokens, int* out_tokens,
                         int* step_counter, int batch, hipStream_t s) {
  launch_k(advance_keys_kernel, 1, 1024, 0, s, keys, nblk, positions, tokens, out_tokens, step_counter, batch);
}

// ---------------------------------------------------------------- argmax
// Token with the highest logit, lowest index on ties ("Predicción de tokens").
// Pass 1: each block reduces ARGMAX_CHUNK entries of one row to (value, index);
// pass 2: one wave per row reduces the block results.
constexpr int ARGMAX_CHUNK = 1024;  // about 128 blocks per row at a 128K vocabulary

int argmax_blocks(int vocab) { return (vocab + ARGMAX_CHUNK - 1) / ARGMAX_CHUNK; }

__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float v = __shfl_xor(bv, o);
    int i = __shfl_xor(bi, o);
    better(bv, bi, v, i);
  }
}

__global__ void __launch_bounds__(256) argmax_pass1(const float* __restrict__ logits, int vocab, int nblk,
                                                    float* __restrict__ pv, int* __restrict__ pi) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int row = blockIdx.y, blk = blockIdx.x;
  const float* lr = logits + (size_t)row * vocab;
  const int lo = blk * ARGMAX_CHUNK;
  const int hi = min(vocab, lo + ARGMAX_CHUNK);
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = lo + threadIdx.x; i < hi; i += 256) better(bv, bi, lr[i], i);
  wave_argmax(bv, bi);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sv[wid] = bv; si[wid] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    bv = sv[0]; bi = si[0];
    for (int w = 1; w < 4; ++w) better(bv, bi, sv[w], si[w]);
    pv[(size_t)row * nblk + blk] = bv;
    pi[(size_t)row * nblk + blk] = bi;
  }
}

__global__ void __launch_bounds__(64) argmax_pass2(const float* __restrict__ pv, const int* __restrict__ pi,
                                                   int nblk, int* __restrict__ out) {
  const int row = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < nblk; i += 64) better(bv, bi, pv[(size_t)row * nblk + i], pi[(size_t)row * nblk + i]);
  wave_argmax(bv, bi);
  if (threadIdx.x == 0) out[row] = bi;
}

void launch_argmax(const float* logits, int rows, int vocab, void* partial, int* out, hipStream_t s) {
  if (rows <= 0) return;
  const int nblk = argmax_blocks(vocab);
  float* pv = (float*)partial;
  int* pi = (int*)(pv + (size_t)rows * nblk);
  launch_k(argmax_pass1, dim3(nblk, rows), 256, 0, s, logits, vocab, nblk, pv, pi);
  launch_k(argmax_pass2, rows, 64, 0, s, pv, pi, nblk, out);
}

__global__ void __launch_bounds__(1024) argmax_rows_kernel(const float* __restrict__ logits, int vocab,
                                                           int* __restrict__ out) {
  __shared__ float sv[16];
  __shared__ int si[16];
  const float* lr = logits + (size_t)blockIdx.x * vocab;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int i = threadIdx.x; i < vocab; i += 1024) better(bv, bi, lr[i], i);
  wave_argmax(bv, bi);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sv[wid] = bv; si[wid] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    bv = sv[0]; bi = si[0];
    for (int w = 1; w < 16; ++w) better(bv, bi, sv[w], si[w]);
    out[blockIdx.x] = bi;
  }
}

void launch_argmax_rows(const float* logits, int rows, int vocab, int* out, hipStream_t s) {
  if (rows <= 0) return;
  launch_k(argmax_rows_kernel, rows, 1024, 0, s, logits, vocab, out);
}

}  // namespace llm
