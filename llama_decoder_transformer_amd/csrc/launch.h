// Internal launchers of the decoder-pass kernels (host side of each .hip file).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace llm {

// Kernel timing hook.  While a timer is installed on the calling thread (kernel
// timing switched on for a model), every launch takes a start / stop event pair
// from it and records them with the dispatch itself (hipExtLaunchKernelGGL), so
// the measured span is the kernel's own execution, not the queue around it.
struct LaunchTimer {
  virtual bool take(hipEvent_t* start, hipEvent_t* stop) = 0;
  virtual void done(hipEvent_t start, hipEvent_t stop) = 0;
};
extern thread_local LaunchTimer* g_launch_timer;

template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s, Args... args) {
  hipEvent_t a, b;
  if (g_launch_timer && g_launch_timer->take(&a, &b)) {
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, a, b, 0u, args...);
    g_launch_timer->done(a, b);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, s, args...);
  }
}

// What a projection does with its fp32 result C[m][n] = sum_k A[m][k] * W[n][k].
enum EpiKind : int {
  EPI_STORE_F32 = 0,  // out_f32[m*ld + n] = C
  EPI_RESID = 1,      // out_f32[m*ld + n] += C   (residual add into the fp32 stream)
  EPI_QKV = 2,        // RoPE on q/k columns, q -> q_out, k/v -> KV cache
  EPI_SWIGLU = 3      // packed rows (2c, 2c+1) = (w1 row c, w3 row c): out[m*ld + c] = silu(C0) * C1
};

struct EpiParams {
  int kind;
  float* out_f32;   // STORE_F32 / RESID
  void* out_act;    // SWIGLU output or q output (activation dtype)
  int ld;           // leading dimension of out_f32 / out_act
  // QKV
  void* k_cache;    // this layer's K section: [slots][G][max_seq][d]
  void* v_cache;    // this layer's V section
  const int* row_pos;   // device [M] positions, or null -> pos0 + m
  const int* row_slot;  // device [M] slots, or null -> slot0
  int pos0, slot0;
  int n_heads, n_kv_heads, head_dim, max_seq, n_slots;
  const float* rope_cos;  // [max_seq][head_dim/2]
  const float* rope_sin;
  int* err;
  // STORE_F32 on the fp16 GEMV only: also write each workgroup's best (logit, index) of each row
  // as an argmax key (argmax_key) to amax_keys[row][workgroup], or null
  unsigned long long* amax_keys;
};

// Embedding gather: x[m][:] = float(E[tok[m]][:]).  It also clears n_zero ints at zero[i * zero_stride]
// (the decode block's counters of every layer) for the step it starts.
void launch_embed(int dtype, const void* emb, const int* tokens, int M, int dim, int vocab, float* x,
                  int* err, hipStream_t s, int* zero = nullptr, int n_zero = 0, int zero_stride = 1);
// RMSNorm of fp32 rows into the activation dtype (an fp16 result out of range sets err bit 8).
void launch_rmsnorm(int dtype, const float* x, const float* w, int M, int dim, float eps, void* out, int* err,
                    hipStream_t s);
// Widen a [n] vector of the storage dtype to fp32.
void launch_to_f32(int dtype, const void* src, float* dst, size_t n, hipStream_t s);
void launch_fill_i32(int* p, int v, size_t n, hipStream_t s);
// bf16 [rows][cols] -> fp16 rows placed at dst row r * row_mult + row_off (a weight outside fp16's
// range sets err bit 8).
void launch_pack_rows(const void* src, void* dst, size_t rows, int cols, int row_mult, int row_off, int* err,
                      hipStream_t s);
// dst[i][:] = src[idx[i]][:] for i < n (rows of `dim` floats).
void launch_gather_rows(const float* src, const int* idx, int n, int dim, float* dst, hipStream_t s);
// Greedy argmax per row (two passes through `partial`, >= rows*argmax_blocks(vocab)*2 words).
int argmax_blocks(int vocab);
void launch_argmax(const float* logits, int rows, int vocab, void* partial, int* out, hipStream_t s);
// Greedy argmax per row in one pass (one 1024-thread workgroup per row, no scratch).
void launch_argmax_rows(const float* logits, int rows, int vocab, int* out, hipStream_t s);
// After a generation step: positions[b] += 1; out_tokens[step*B + b] = tokens[b]; step++.
void launch_advance(int* positions, const int* tokens, int* out_tokens, int* step_counter, int batch,
                    hipStream_t s);
// The same after an LM head on the fp16 GEMV that left its workgroups' argmax keys in
// keys[b][nblk] (nblk = gemv_h_blocks of the LM head): tokens[b] = the row's greedy token, then
// the advance.  batch <= AMAX_ROWS.
constexpr int AMAX_ROWS = 8;
void launch_advance_keys(const unsigned long long* keys, int nblk, int* positions, int* tokens, int* out_tokens,
                         int* step_counter, int batch, hipStream_t s);

// Projections.
// fp16 MFMA GEMM for M > 8 (A fp16 [M][K], W fp16 [N][K], fp32 accumulation).  Shapes with
// too few output tiles to fill the GPU (small M) split K over several workgroups: fp32
// partials go to `splitk_ws` (gemm_splitk_floats(M, N, K) floats) and a second pass sums
// them in a fixed order and applies the epilogue.  Without enough workspace the GEMM runs
// unsplit.
int gemm_splitk_count(int M, int N, int K);
size_t gemm_splitk_floats(int M, int N, int K);
void launch_gemm_f16(const void* A, const void* W, int M, int N, int K, const EpiParams& ep, float* splitk_ws,
                     size_t splitk_ws_floats, hipStream_t s);
// x += A W^T (ep.kind == EPI_RESID, ep.out_f32 = x with ld N) and then a = fp16(rmsnorm(x) * norm_w)
// in the split-K reduction pass, when the weight-streaming plan splits this shape over K.
// Returns false and enqueues nothing otherwise.
bool launch_gemm_f16_resid_norm(const void* A, const void* W, int M, int N, int K, const EpiParams& ep,
                                const float* norm_w, float eps, void* a_out, float* splitk_ws,
                                size_t splitk_ws_floats, hipStream_t s);
// Vector GEMV for small M.  With norm_w == nullptr, A has the activation dtype; otherwise A
// is the fp32 residual stream and the RMSNorm (weight norm_w, eps) is fused into the pass.
// Workgroups along N of the fp16 GEMV for this shape (its launch's grid.x).
int gemv_h_blocks(int M, int N, int K);
void launch_gemv(int dtype, const void* A, const void* W, const float* norm_w, float eps, int M, int N, int K,
                 const EpiParams& ep, hipStream_t s);

// Attention.
// Split-KV decode attention: rows with explicit (slot, pos); q [rows][H*d]; `partial` holds
// attn_decode_partial_floats(...) floats.
int attn_decode_chunk(int rows, int n_kv_heads, int max_seq);
size_t attn_decode_partial_floats(int rows, int n_heads, int head_dim, int max_seq);
// The partial floats the launcher actually uses for `rows` decode rows (its own chunk choice).
size_t attn_decode_partial_floats_used(int dtype, int rows, int n_heads, int n_kv_heads, int head_dim, int max_seq);
void launch_attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                        const int* row_pos, const int* row_slot, int pos0, int slot0, int rows,
                        int n_heads, int n_kv_heads, int head_dim, int max_seq, int n_slots,
                        float* partial, void* out, int* err, hipStream_t s);
// Causal GQA prefill attention on MFMA (fp16, head_dim 128): queries at pos0 + i for one slot.
bool attn_prefill_supported(int head_dim, int n_heads, int n_kv_heads);
void launch_attn_prefill(const void* q, const void* k_cache, const void* v_cache, int slot, int pos0,
                         int n_tokens, int n_heads, int n_kv_heads, int head_dim, int max_seq,
                         void* out, hipStream_t s);

// One sequence of a batched prefill: its rows [row0, row0 + n) of the activations, positions
// start .. start + n - 1 of cache slot `slot`, and the index of its first query block in the
// batched prefill attention's grid (blocks of attn_prefill_block_rows queries).
struct SeqDesc {
  int row0, n, start, slot, blk0, pad[3];
};
// Query rows per workgroup of the prefill attention for sequences of at most max_n tokens.
int attn_prefill_block_rows(int max_n, int n_heads, int n_kv_heads);
// Prefill attention of several sequences in one launch over (sequence, query block) work items:
// seqs (device, nseq entries, blk0 ascending from 0) as above, n_blocks = sum of the sequences'
// query blocks, max_n = the longest sequence (it sets the block size).
void launch_attn_prefill_varlen(const void* q, const void* k_cache, const void* v_cache, const SeqDesc* seqs,
                                int nseq, int n_blocks, int max_n, int n_heads, int n_kv_heads, int head_dim,
                                int max_seq, void* out, hipStream_t s);
// Ints between two cross-workgroup counters of the decode block (one 128-byte line each).
constexpr int DB_SYNC_LINE = 32;
// Batch-1 decode of one layer's attention half in one launch: q|k|v GEMV (RMSNorm fused, RoPE,
// cache write), causal GQA attention over the cache, wo GEMV with the residual add.
struct DecodeBlockParams {
  float* x;                // fp32 residual [dim]: the norm's input, then += o W_o^T
  const float* attn_norm;  // fp32 [dim]
  const _Float16* wqkv;    // [(H + 2G) * 128][dim]
  const _Float16* wo;      // [dim][H * 128]
  _Float16* q;             // [H * 128]
  _Float16* o;             // [H * 128]
  _Float16* kc;            // this layer's K section [slots][G][max_seq][128]
  _Float16* vc;
  const float* rope_cos;   // [max_seq][64]
  const float* rope_sin;
  const int* row_pos;      // device [1]
  const int* row_slot;     // device [1]
  float* partial;          // >= decode_block_partial_floats(H, max_seq) floats
  int* sync;               // this layer's decode_block_sync_ints(G) ints, zero at the launch
  int* err;
  float eps;
  int dim, H, G, max_seq, n_slots;
  int nq, na, nch, qkv_per_group, wo_delay;  // set by the launcher
};
bool decode_block_supported(int dtype, int dim, int n_heads, int n_kv_heads);
int decode_block_sync_ints(int n_kv_heads);
size_t decode_block_partial_floats(int n_heads, int max_seq);
void launch_decode_block(DecodeBlockParams p, hipStream_t s);

// Per-row positions and slots, last-row indices and the device copy of up to SEQ_META_CHUNK
// sequence descriptors, taken from the kernel arguments (no host staging buffer): entries
// first .. first + count - 1 of the batch.
constexpr int SEQ_META_CHUNK = 32;
struct SeqMetaChunk {
  int first, count, pad[2];
  SeqDesc d[SEQ_META_CHUNK];
};
void launch_seq_meta(const SeqMetaChunk& c, int* row_pos, int* row_slot, int* last_idx, SeqDesc* table,
                     hipStream_t s);

}  // namespace llm
