/*
 * llm.h -- C ABI of the MI355X (gfx950) Llama-2/3 decoder forward pass.
 *
 * The pass follows the model walked through on the pages
 *   "Resumen de una implementación desde cero del modelo LLaMA-3" (GeekNews, es),
 *   "Model Llama 3 yang Diimplementasikan dengan NumPy Murni" (GeekNews, id),
 *   "Building llama3 from scratch" (downcodes, ar) and "LLaMA2" (downcodes, fr):
 * token embedding -> n_layers x [RMSNorm -> separate wq/wk/wv projections ->
 * RoPE on q and k -> KV-cache write -> causal grouped-query attention -> wo and
 * residual add -> RMSNorm -> SwiGLU feed-forward (w1/w3 gate-up, w2 down) and
 * residual add] -> final RMSNorm -> output projection (last position only in a
 * prefill) -> greedy argmax.  Prefill runs a whole prompt; a decode step runs
 * one new token per sequence against its KV cache ("Generasi" section of the
 * NumPy page).
 *
 * Conventions shared by every call:
 *  - Pointers documented as "device" point to GPU memory owned by the caller
 *    (for example torch tensors).  The library never allocates or frees device
 *    memory and keeps no device pointer beyond the buffers handed to
 *    llm_init_weights.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every compute call only enqueues work on that stream and returns; results
 *    are valid once the stream has been synchronised.  No call waits for the
 *    device except llm_init_weights (it synchronises `stream` at its end),
 *    llm_read_device_error (it synchronises `stream`) and the diagnostics
 *    llm_set_kernel_timing / llm_kernel_timing (they wait for the timing events
 *    already recorded).
 *  - Matrices are row-major.  Weights are [out_features, in_features] and a
 *    linear layer computes y = x W^T (printed shapes on the "Building llama3
 *    from scratch" page: wq [4096, 4096], wk/wv [1024, 4096]).  Query head h
 *    owns rows h*head_dim .. h*head_dim+head_dim-1 of wq (per-head view of wq on
 *    the same page); K/V head g likewise owns rows of wk/wv.
 *  - Element types.  An LLM_F32 model takes fp32 weights and computes and
 *    stores everything in fp32.  An LLM_BF16 model takes its weights as raw
 *    bfloat16 bit patterns (uint16); llm_init_weights converts them to fp16
 *    (IEEE binary16) in the packed buffer, and its activations and KV cache are
 *    fp16 too, with fp32 accumulation, an fp32 residual stream and fp32 logits.
 *    The conversion is exact for every bf16 weight whose magnitude lies in
 *    [2^-14, 65504]; smaller magnitudes lose low bits, larger ones raise
 *    LLM_DEVERR_RANGE (as does any fp16 activation or cache value that leaves
 *    fp16's finite range).
 *  - Every call returns an llm_status.  Host-side validation happens before
 *    anything is enqueued, so a failing call leaves the stream untouched.
 *    llm_last_error_message() then describes the failure (thread-local).
 *  - Values read on the device (token ids, decode positions and slots) are
 *    bounds-checked by the kernels: an out-of-range entry makes that row
 *    produce no cache write and zero output, and sets a flag readable with
 *    llm_read_device_error().
 */
#ifndef LLM_H
#define LLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum llm_status {
  LLM_OK = 0,
  LLM_ERR_INVALID_ARG = -1,      /* null pointer, negative size, bad dtype */
  LLM_ERR_CONFIG = -2,           /* inconsistent hyper-parameters */
  LLM_ERR_OUT_OF_RANGE = -3,     /* positions / slots / batch beyond the configured maxima */
  LLM_ERR_BUFFER_TOO_SMALL = -4, /* a caller buffer is smaller than the size query returns */
  LLM_ERR_HIP = -5,              /* a HIP runtime call failed */
  /* Not a status: makes every int32 value a valid llm_status, so that a status read from
   * elsewhere (llm_status_string of an unknown code) is defined behaviour in C++ too. */
  LLM_STATUS_MAX_ENUM = 0x7FFFFFFF
} llm_status;

/* Type of the weights handed to llm_init_weights: LLM_F32 (fp32 everywhere) or
 * LLM_BF16 (bf16 weights, held and computed as fp16; see "Element types" above). */
enum { LLM_F32 = 0, LLM_BF16 = 1 };

/* Device-side error flags (bit mask) reported by llm_read_device_error:
 * TOKEN a token id outside [0, vocab_size); POSITION a decode position outside
 * [0, max_seq_len); SLOT a decode slot outside [0, max_batch); RANGE a value
 * stored as fp16 (a packed weight, a normalised activation, q/k/v, a KV-cache
 * entry or a SwiGLU output) fell outside fp16's finite range or was NaN; SYNC a
 * kernel whose workgroups wait for one another gave up waiting (its wait is bounded,
 * so the kernel always ends; the results of that step are not valid). */
enum { LLM_DEVERR_TOKEN = 1, LLM_DEVERR_POSITION = 2, LLM_DEVERR_SLOT = 4, LLM_DEVERR_RANGE = 8,
       LLM_DEVERR_SYNC = 16 };

/*
 * Model hyper-parameters: the params.json field set printed on the "Building
 * llama3 from scratch" page (dim, n_layers, n_heads, n_kv_heads, vocab_size,
 * norm_eps, rope_theta) with the feed-forward width given explicitly instead of
 * multiple_of / ffn_dim_multiplier, plus the context length (max_seq_len, NumPy
 * page, "Struktur").  Requirements (llm_check_config): every size positive;
 * dim % n_heads == 0 and head_dim = dim / n_heads is 48, 64 or 128;
 * n_heads % n_kv_heads == 0 and n_heads / n_kv_heads is at most 4 or a multiple
 * of 4; dim and ffn_hidden_dim are multiples of 8; rope_theta > 0; norm_eps >= 0;
 * 1 <= max_batch <= 1024; max_seq_len <= 2^20 and max_seq_len * max_batch <= 2^31.
 * max_batch: number of KV-cache slots (= largest decode batch).
 * max_prefill_tokens: largest n_tokens of one llm_prefill / llm_layer_forward, and
 * the largest total of one llm_prefill_batch.
 */
typedef struct llm_config {
  int32_t dim;
  int32_t n_layers;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t vocab_size;
  int32_t max_seq_len;
  int32_t ffn_hidden_dim;
  float rope_theta;
  float norm_eps;
  int32_t dtype;              /* LLM_F32 or LLM_BF16 */
  int32_t max_batch;
  int32_t max_prefill_tokens;
} llm_config;

/*
 * Device pointers to the weights, named as in the checkpoint listing on the
 * "Building llama3 from scratch" page.  All have the config's dtype.  The
 * per-layer members are HOST arrays of n_layers device pointers.  `norm` is the
 * final RMSNorm weight and `output` the (untied) LM head; their names are not
 * printed on the pages.
 *   tok_embeddings [vocab, dim]      output [vocab, dim]      norm [dim]
 *   attention_norm[l], ffn_norm[l] [dim]
 *   wq[l] [n_heads*head_dim, dim]    wk[l], wv[l] [n_kv_heads*head_dim, dim]
 *   wo[l] [dim, n_heads*head_dim]
 *   w1[l], w3[l] [ffn_hidden_dim, dim]    w2[l] [dim, ffn_hidden_dim]
 */
typedef struct llm_weights {
  const void* tok_embeddings;
  const void* const* attention_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* w1;
  const void* const* w3;
  const void* const* w2;
  const void* norm;
  const void* output;
} llm_weights;

typedef struct llm_model llm_model;

/* Check a configuration without touching the GPU.  LLM_OK or LLM_ERR_CONFIG. */
llm_status llm_check_config(const llm_config* cfg);

/* Sizes in bytes of the three device buffers llm_init_weights needs (0 if the
 * config is invalid).  Packed weights: every weight (fp16 for LLM_BF16, fp32 for
 * LLM_F32) plus the fp32 norm weights and RoPE tables.
 * KV cache: row-major [n_layers][2 (K, V)][max_batch (slot)][n_kv_heads]
 * [max_seq_len][head_dim] of fp16 (LLM_BF16) or fp32 (LLM_F32) elements; K is
 * stored after RoPE.  A caller may fill a slot's first positions directly (a
 * cache built elsewhere) and continue it with llm_decode_step or llm_prefill.
 * Workspace: activations for max(max_prefill_tokens, max_batch) rows, attention,
 * split-K and argmax partials (and the generation loop's argmax keys), and
 * batched-prefill descriptors. */
size_t llm_packed_weight_bytes(const llm_config* cfg);
size_t llm_kv_cache_bytes(const llm_config* cfg);
size_t llm_workspace_bytes(const llm_config* cfg);

/*
 * Validate `cfg`, copy and repack the weights into `packed` (q/k/v rows
 * concatenated per layer, w1/w3 rows interleaved, norm weights widened to
 * fp32), build the RoPE cos/sin tables (angle pos * rope_theta^(-2j/head_dim)
 * from an fp64 outer product, "RoPE #1" on the NumPy page) and create a model
 * handle in *out.  The three buffers must stay alive until llm_free; the
 * source weights may be freed once this call returns.  The handle also owns a
 * capture stream, events and graphs, released by llm_free.  The call clears the
 * device error flags and synchronises `stream` before returning; a weight that
 * does not fit fp16 shows as LLM_DEVERR_RANGE in llm_read_device_error.
 * Errors: INVALID_ARG (null pointer), CONFIG, BUFFER_TOO_SMALL (a size below the
 * corresponding query), HIP.
 */
llm_status llm_init_weights(const llm_config* cfg, const llm_weights* weights,
                            void* packed, size_t packed_bytes,
                            void* kv_cache, size_t kv_cache_bytes,
                            void* workspace, size_t workspace_bytes,
                            void* stream, llm_model** out);

/*
 * Prefill ("Generasi": the whole prompt at once): embed tokens_dev[0..n_tokens)
 * (device int32), run every layer at positions start_pos .. start_pos+n_tokens-1
 * writing K/V into cache slot `slot`, and write the logits of the LAST position
 * ("Linear": only the last logit is computed) to logits_dev (device fp32
 * [vocab]).  Errors: INVALID_ARG, OUT_OF_RANGE (slot >= max_batch,
 * n_tokens > max_prefill_tokens, start_pos + n_tokens > max_seq_len).
 */
llm_status llm_prefill(llm_model* m, int32_t slot, const int32_t* tokens_dev, int32_t n_tokens,
                       int32_t start_pos, float* logits_dev, void* stream);

/*
 * Prefill of several sequences in one call, each as llm_prefill would do it: the
 * prompt pass of the "Generasi" section applied to a batch of prompts of their own
 * lengths.  Sequence b has lens_host[b] >= 1 tokens, taken in order from tokens_dev
 * (device int32, sum of the lengths ids), placed at positions starts_host[b] .. of
 * cache slot slots_host[b] (positions before starts_host[b] must already be in that
 * slot's cache).  logits_dev (device fp32 [batch][vocab]) receives the logits of
 * each sequence's last position.  The three host arrays (batch entries each) are
 * read during the call and travel to the device inside kernel arguments, so the
 * call neither stages them in host memory nor waits for the device; they may be
 * reused as soon as it returns.  Projections run once over all rows, and the
 * attention of every sequence runs in one launch.  Results equal separate
 * llm_prefill calls up to rounding.  Errors:
 * INVALID_ARG (null pointer, batch < 1, a length < 1, two sequences with the same
 * slot), OUT_OF_RANGE (batch > max_batch, a slot >= max_batch, start + length >
 * max_seq_len, total tokens > max_prefill_tokens), HIP.
 */
llm_status llm_prefill_batch(llm_model* m, int32_t batch, const int32_t* slots_host, const int32_t* starts_host,
                             const int32_t* lens_host, const int32_t* tokens_dev, float* logits_dev,
                             void* stream);

/*
 * One decoder layer on an explicit residual stream, used to test a layer on its
 * own: x_dev (device fp32 [n_tokens, dim]) is updated in place to the layer's
 * output, at positions start_pos.. and cache slot `slot`.  Same kernels and
 * errors as llm_prefill (plus OUT_OF_RANGE for a bad layer index).
 */
llm_status llm_layer_forward(llm_model* m, int32_t layer, int32_t slot, float* x_dev,
                             int32_t n_tokens, int32_t start_pos, void* stream);

/*
 * One decode step for `batch` independent sequences ("KV cache" and "Generasi"
 * sections: only the newest token is fed, K/V of earlier tokens come from the
 * cache).  Row b: slot slots_dev[b], new token tokens_dev[b] at position
 * positions_dev[b] (= number of tokens already cached in that slot); its K/V
 * are written at that position and attention covers positions 0..positions[b].
 * All three arrays are device int32 [batch]; logits_dev is device fp32
 * [batch, vocab].  Errors: INVALID_ARG, OUT_OF_RANGE (batch > max_batch);
 * device-side range errors are flagged (see llm_read_device_error).
 */
llm_status llm_decode_step(llm_model* m, int32_t batch, const int32_t* slots_dev,
                           const int32_t* positions_dev, const int32_t* tokens_dev,
                           float* logits_dev, void* stream);

/*
 * llm_decode_step for callers that cannot allocate device memory at all (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step and the same results, with the kernels' scratch (the split-KV attention chunk
 * partials, the split-K projection partials, and the batch-1 decode block's partials
 * and counters) in a static device array of the library
 * instead of regions of the model's workspace.  That array holds 32 MiB on each GPU the
 * library runs on, until the process ends; a step whose partials need more (the
 * message states how much) is rejected with LLM_ERR_OUT_OF_RANGE before anything is
 * enqueued.  (A Llama-3-8B-shaped step of 64 rows over an 8193-position cache needs
 * about 14 MB.)  The call enqueues kernels only: no allocation, no synchronisation.
 * Every call on one GPU shares that GPU's array and finds there what the last call left:
 * each partial is written before it is read, and the batch-1 decode's cross-workgroup
 * counters, the only values that must start at zero, are cleared by the step's first
 * kernel.  Calls that overlap on one GPU, from several streams or threads, race on it.
 * Arguments and errors as llm_decode_step.
 */
llm_status llm_decode_step_noalloc(llm_model* m, int32_t batch, const int32_t* slots_dev,
                                   const int32_t* positions_dev, const int32_t* tokens_dev,
                                   float* logits_dev, void* stream);

/*
 * Greedy choice ("Predicción de tokens": the token with the highest logit):
 * out_dev[r] = argmax over logits_dev[r*vocab .. r*vocab+vocab-1], lowest index
 * on ties.  logits_dev device fp32 [rows, vocab]; out_dev device int32 [rows].
 * Needs no model.  Errors: INVALID_ARG.
 */
llm_status llm_argmax(const float* logits_dev, int32_t rows, int32_t vocab, int32_t* out_dev,
                      void* stream);

/*
 * Greedy generation on the device: `n_steps` times { decode step for `batch`
 * rows; argmax into tokens_dev; positions_dev[b] += 1; out_tokens_dev[s*batch+b]
 * = new token }.  tokens_dev / positions_dev are updated in place; logits_dev
 * (device fp32 [batch, vocab]) holds the last step's logits.  One step is
 * captured once into a HIP graph per (batch, buffers) and replayed.  The argmax
 * is llm_argmax's (lowest index on ties, a NaN logit never chosen); for LLM_BF16
 * batches of up to 8 rows it is folded into the LM-head kernel (per-workgroup
 * keys in the workspace) and LLM_K_ARGMAX then times only the reduction of the
 * keys and the advance.  Errors as llm_decode_step.
 */
llm_status llm_generate(llm_model* m, int32_t batch, const int32_t* slots_dev,
                        int32_t* positions_dev, int32_t* tokens_dev, int32_t n_steps,
                        int32_t* out_tokens_dev, float* logits_dev, void* stream);

/* Synchronise `stream`, then return (and clear) the device error flags
 * (LLM_DEVERR_* bits) in *flags.  Errors: INVALID_ARG, HIP. */
llm_status llm_read_device_error(llm_model* m, int32_t* flags, void* stream);

/*
 * Kernel timing (diagnostics).  While enabled, every kernel the library
 * launches directly records a start and a stop hipEvent with its own dispatch
 * (hipExtLaunchKernelGGL), so the measured span is the kernel's execution and
 * excludes queueing and launch gaps; llm_generate then launches directly
 * instead of replaying its graph.  Kernels are charged to LLM_K_* groups (one
 * group invocation may launch several kernels, e.g. a split-K GEMM and its
 * reduce pass).  Enabling resets the totals.  llm_kernel_timing synchronises on
 * the recorded events and returns, for one group, the number of invocations,
 * the number of kernels they dispatched (`kernels` may be NULL) and the summed
 * kernel execution time in milliseconds.  Errors: INVALID_ARG, HIP.
 */
enum {
  LLM_K_EMBED = 0, LLM_K_RMSNORM = 1, LLM_K_QKV = 2, LLM_K_ATTN = 3, LLM_K_WO = 4,
  LLM_K_GATE_UP = 5, LLM_K_DOWN = 6, LLM_K_LM_HEAD = 7, LLM_K_ARGMAX = 8,
  LLM_K_DECODE_BLOCK = 9, /* batch-1 decode: q|k|v, attention and wo in one launch */
  LLM_K_COUNT = 10
};
llm_status llm_set_kernel_timing(llm_model* m, int32_t enable);
llm_status llm_kernel_timing(llm_model* m, int32_t kind, int64_t* launches, int64_t* kernels, double* total_ms);

/* Release the handle and what it owns on the host (stream, events, graphs); no
 * caller-provided device memory is freed.  NULL is allowed. */
void llm_free(llm_model* m);

const char* llm_status_string(llm_status s);
const char* llm_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* LLM_H */
