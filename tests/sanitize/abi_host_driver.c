/*
 * Host-side driver of the C ABI (include/llm.h) for sanitizer builds: it runs every
 * validation path that needs no GPU.  Built and run by tests/test_host_sanitizers.py
 * against a host-only, AddressSanitizer + UndefinedBehaviorSanitizer build of the
 * library.  Exit status 0 when every call returned what the header promises.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "llm.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static llm_config base_config(void) {
  llm_config c;
  memset(&c, 0, sizeof(c));
  c.dim = 288;
  c.n_layers = 6;
  c.n_heads = 6;
  c.n_kv_heads = 6;
  c.vocab_size = 32000;
  c.max_seq_len = 256;
  c.ffn_hidden_dim = 768;
  c.rope_theta = 10000.0f;
  c.norm_eps = 1e-5f;
  c.dtype = LLM_F32;
  c.max_batch = 2;
  c.max_prefill_tokens = 16;
  return c;
}

int main(void) {
  llm_config c = base_config();
  EXPECT(llm_check_config(&c) == LLM_OK);
  EXPECT(llm_check_config(NULL) == LLM_ERR_CONFIG);
  EXPECT(strlen(llm_last_error_message()) > 0);

  /* every requirement of llm_check_config, one broken at a time */
  struct { const char* what; llm_config c; } bad[16];
  int nb = 0;
#define BAD(field, value)            \
  do {                               \
    bad[nb].what = #field "=" #value; \
    bad[nb].c = base_config();       \
    bad[nb].c.field = value;         \
    ++nb;                            \
  } while (0)
  BAD(dim, 290);
  BAD(n_kv_heads, 4);
  BAD(dtype, 7);
  BAD(max_batch, 0);
  BAD(max_batch, 2048);
  BAD(ffn_hidden_dim, 770);
  BAD(rope_theta, -1.0f);
  BAD(norm_eps, -1.0f);
  BAD(max_prefill_tokens, 0);
  BAD(vocab_size, 0);
  BAD(n_layers, -3);
  BAD(max_seq_len, (1 << 20) + 1);
  for (int i = 0; i < nb; ++i) {
    if (llm_check_config(&bad[i].c) != LLM_ERR_CONFIG) {
      fprintf(stderr, "config %s accepted\n", bad[i].what);
      ++failures;
    }
    EXPECT(llm_packed_weight_bytes(&bad[i].c) == 0);
    EXPECT(llm_kv_cache_bytes(&bad[i].c) == 0);
    EXPECT(llm_workspace_bytes(&bad[i].c) == 0);
  }

  /* sizes of both storage types, including the Llama-3-8B shape */
  size_t pw = llm_packed_weight_bytes(&c), kv = llm_kv_cache_bytes(&c), ws = llm_workspace_bytes(&c);
  EXPECT(pw > 0 && kv > 0 && ws > 0);
  EXPECT(kv == (size_t)6 * 2 * 2 * 6 * 256 * 48 * 4);
  llm_config big = base_config();
  big.dim = 4096; big.n_layers = 32; big.n_heads = 32; big.n_kv_heads = 8; big.vocab_size = 128256;
  big.max_seq_len = 8192; big.ffn_hidden_dim = 14336; big.rope_theta = 500000.0f; big.dtype = LLM_BF16;
  big.max_batch = 64; big.max_prefill_tokens = 8192;
  EXPECT(llm_check_config(&big) == LLM_OK);
  EXPECT(llm_kv_cache_bytes(&big) == (size_t)32 * 2 * 64 * 8 * 8192 * 128 * 2);
  EXPECT(llm_packed_weight_bytes(&big) > (size_t)16000000000ULL);
  EXPECT(llm_workspace_bytes(&big) > 0);

  /* llm_init_weights rejects bad arguments before touching the GPU */
  llm_model* m = (llm_model*)0x1;
  char dummy[64];
  const void* layer_ptrs[6] = {dummy, dummy, dummy, dummy, dummy, dummy};
  llm_weights w;
  w.tok_embeddings = dummy; w.norm = dummy; w.output = dummy;
  w.attention_norm = layer_ptrs; w.wq = layer_ptrs; w.wk = layer_ptrs; w.wv = layer_ptrs; w.wo = layer_ptrs;
  w.ffn_norm = layer_ptrs; w.w1 = layer_ptrs; w.w3 = layer_ptrs; w.w2 = layer_ptrs;
  EXPECT(llm_init_weights(&c, &w, dummy, pw, dummy, kv, dummy, ws, NULL, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_init_weights(&bad[0].c, &w, dummy, pw, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_CONFIG);
  EXPECT(m == NULL);
  EXPECT(llm_init_weights(&c, NULL, dummy, pw, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_init_weights(&c, &w, NULL, pw, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_init_weights(&c, &w, dummy, pw - 1, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_BUFFER_TOO_SMALL);
  EXPECT(llm_init_weights(&c, &w, dummy, pw, dummy, kv - 1, dummy, ws, NULL, &m) == LLM_ERR_BUFFER_TOO_SMALL);
  EXPECT(llm_init_weights(&c, &w, dummy, pw, dummy, kv, dummy, ws - 1, NULL, &m) == LLM_ERR_BUFFER_TOO_SMALL);
  const void* with_null[6] = {dummy, dummy, NULL, dummy, dummy, dummy};
  w.w2 = with_null;
  EXPECT(llm_init_weights(&c, &w, dummy, pw, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_INVALID_ARG);
  EXPECT(strstr(llm_last_error_message(), "layer 2") != NULL);
  w.w2 = layer_ptrs;
  w.output = NULL;
  EXPECT(llm_init_weights(&c, &w, dummy, pw, dummy, kv, dummy, ws, NULL, &m) == LLM_ERR_INVALID_ARG);
  EXPECT(m == NULL);

  /* every model call rejects a NULL handle, and the argmax its arguments */
  int32_t ids[4] = {1, 2, 3, 4}, flags = 0;
  float logits[4];
  int64_t launches = 0;
  double ms = 0.0;
  EXPECT(llm_prefill(NULL, 0, ids, 4, 0, logits, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_prefill_batch(NULL, 1, ids, ids, ids, ids, logits, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_layer_forward(NULL, 0, 0, logits, 1, 0, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_decode_step(NULL, 1, ids, ids, ids, logits, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_generate(NULL, 1, ids, ids, ids, 1, ids, logits, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_read_device_error(NULL, &flags, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_set_kernel_timing(NULL, 1) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_kernel_timing(NULL, 0, &launches, NULL, &ms) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_argmax(NULL, 1, 4, ids, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_argmax(logits, 0, 4, ids, NULL) == LLM_ERR_INVALID_ARG);
  EXPECT(llm_argmax(logits, 1, 0, ids, NULL) == LLM_ERR_INVALID_ARG);
  llm_free(NULL);

  const llm_status all[] = {LLM_OK, LLM_ERR_INVALID_ARG, LLM_ERR_CONFIG, LLM_ERR_OUT_OF_RANGE,
                            LLM_ERR_BUFFER_TOO_SMALL, LLM_ERR_HIP, (llm_status)-99};
  for (size_t i = 0; i < sizeof(all) / sizeof(all[0]); ++i) EXPECT(strlen(llm_status_string(all[i])) > 0);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi host driver: all checks passed\n");
  return 0;
}
