// C ABI of the decoder pass: validation, weight packing, buffer layout and the
// per-layer launch sequence.  Declarations and contracts live in include/llm.h.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"
#include "llm.h"

using namespace llm;

// Scratch of llm_decode_step_noalloc: the split-KV attention and split-K projection partials
// of one decode step, in a file-scope device array instead of the caller's workspace, so the
// call needs no allocation by anyone.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses this name as an address: it resolves the array's
// address on each device once (noalloc_scratch_ptr) and passes that to the kernels.
constexpr size_t LLM_NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) char scratch[LLM_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

llm_status fail(llm_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t elem_size(const llm_config& c) { return c.dtype == LLM_BF16 ? 2 : 4; }

bool config_ok(const llm_config* c, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return bad("config is NULL");
  if (c->dim <= 0 || c->n_layers <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->vocab_size <= 0 ||
      c->max_seq_len <= 0 || c->ffn_hidden_dim <= 0)
    return bad("every size must be positive");
  if (c->dtype != LLM_F32 && c->dtype != LLM_BF16) return bad("dtype must be LLM_F32 or LLM_BF16");
  if (c->max_batch < 1 || c->max_batch > 1024) return bad("max_batch must be in [1, 1024]");
  if (c->max_prefill_tokens < 1) return bad("max_prefill_tokens must be >= 1");
  if (c->dim % c->n_heads) return bad("dim must be a multiple of n_heads");
  if (c->n_heads % c->n_kv_heads) return bad("n_heads must be a multiple of n_kv_heads");
  const int hd = c->dim / c->n_heads;
  if (hd != 48 && hd != 64 && hd != 128) return bad("head_dim must be 48, 64 or 128");
  const int hpg = c->n_heads / c->n_kv_heads;
  if (hpg > 4 && hpg % 4) return bad("n_heads / n_kv_heads must be <= 4 or a multiple of 4");
  if (c->dim % 8 || c->ffn_hidden_dim % 8) return bad("dim and ffn_hidden_dim must be multiples of 8");
  if (!(c->rope_theta > 0.f) || !(c->norm_eps >= 0.f)) return bad("rope_theta must be > 0 and norm_eps >= 0");
  if (c->max_seq_len > (1 << 20)) return bad("max_seq_len must be <= 1048576");
  if ((long long)c->max_seq_len * c->max_batch > (1LL << 31)) return bad("max_seq_len * max_batch too large");
  return true;
}

struct Dims {
  int dim, L, H, G, hd, F, V, S, B, P;
  size_t es;
  explicit Dims(const llm_config& c)
      : dim(c.dim), L(c.n_layers), H(c.n_heads), G(c.n_kv_heads), hd(c.dim / c.n_heads), F(c.ffn_hidden_dim),
        V(c.vocab_size), S(c.max_seq_len), B(c.max_batch), P(c.max_prefill_tokens), es(elem_size(c)) {}
  int qkv_rows() const { return (H + 2 * G) * hd; }
  int rows() const { return P > B ? P : B; }
};

// Packed-weight layout.
struct PackedLayout {
  size_t emb, out, norm, cos, sin, layer0, layer_stride;
  size_t l_attn_norm, l_ffn_norm, l_wqkv, l_wo, l_w13, l_w2;
  size_t total;
  explicit PackedLayout(const llm_config& c) {
    Dims d(c);
    size_t o = 0;
    emb = o; o = align256(o + (size_t)d.V * d.dim * d.es);
    out = o; o = align256(o + (size_t)d.V * d.dim * d.es);
    norm = o; o = align256(o + (size_t)d.dim * 4);
    cos = o; o = align256(o + (size_t)d.S * (d.hd / 2) * 4);
    sin = o; o = align256(o + (size_t)d.S * (d.hd / 2) * 4);
    layer0 = o;
    size_t p = 0;
    l_attn_norm = p; p = align256(p + (size_t)d.dim * 4);
    l_ffn_norm = p; p = align256(p + (size_t)d.dim * 4);
    l_wqkv = p; p = align256(p + (size_t)d.qkv_rows() * d.dim * d.es);
    l_wo = p; p = align256(p + (size_t)d.dim * d.H * d.hd * d.es);
    l_w13 = p; p = align256(p + (size_t)2 * d.F * d.dim * d.es);
    l_w2 = p; p = align256(p + (size_t)d.dim * d.F * d.es);
    layer_stride = p;
    total = layer0 + (size_t)d.L * layer_stride;
  }
};

// Workspace layout.
struct WorkLayout {
  size_t flags, x, a, q, o, u, attn, amax, akeys, splitk, splitk_floats, rowmeta, seqtab, last, sync, total;
  explicit WorkLayout(const llm_config& c) {
    Dims d(c);
    const size_t R = (size_t)d.rows();
    size_t p = 0;
    flags = p; p = align256(p + 256);
    const bool mfma_prefill = c.dtype == LLM_BF16 && attn_prefill_supported(d.hd, d.H, d.G);
    const int att_rows = mfma_prefill ? d.B : d.rows();
    x = p; p = align256(p + R * d.dim * 4);
    a = p; p = align256(p + R * d.dim * d.es);
    q = p; p = align256(p + R * d.H * d.hd * d.es);
    o = p; p = align256(p + R * d.H * d.hd * d.es);
    u = p; p = align256(p + R * d.F * d.es);
    attn = p; p = align256(p + std::max(attn_decode_partial_floats(att_rows, d.H, d.hd, d.S),
                                        decode_block_partial_floats(d.H, d.S)) * 4);
    amax = p; p = align256(p + (size_t)d.B * argmax_blocks(d.V) * 8);
    // argmax keys of the LM head of a generation step (one per GEMV workgroup and row)
    akeys = p; p = align256(p + (size_t)AMAX_ROWS * gemv_h_blocks(AMAX_ROWS, d.V, d.dim) * 8);
    // split-K partials of the MFMA projections at row counts whose tiles cannot fill the GPU
    splitk_floats = 0;
    if (c.dtype == LLM_BF16) {
      const int shapes[4][2] = {{d.qkv_rows(), d.dim}, {d.dim, d.H * d.hd}, {2 * d.F, d.dim}, {d.dim, d.F}};
      for (int M = 9; M <= (int)R; ++M)
        for (auto& sh : shapes) splitk_floats = std::max(splitk_floats, gemm_splitk_floats(M, sh[0], sh[1]));
    }
    splitk = p; p = align256(p + splitk_floats * 4);
    // batched prefill: per-row position and slot, per-sequence last row, sequence descriptors,
    // gathered last rows
    rowmeta = p; p = align256(p + (2 * R + (size_t)d.B) * 4);
    seqtab = p; p = align256(p + (size_t)d.B * sizeof(SeqDesc));
    last = p; p = align256(p + (size_t)d.B * d.dim * 4);
    // counters of the batch-1 decode block, per layer
    sync = p; p = align256(p + (size_t)d.L * decode_block_sync_ints(d.G) * 4);
    total = p;
  }
};

size_t kv_bytes(const llm_config& c) {
  Dims d(c);
  return (size_t)d.L * 2 * d.B * d.G * d.S * d.hd * d.es;
}

}  // namespace

struct LayerPtrs {
  float* attn_norm;
  float* ffn_norm;
  void* wqkv;
  void* wo;
  void* w13;
  void* w2;
};

struct GraphEntry {
  int batch;
  const void* ptrs[5];
  hipGraphExec_t exec;
};

struct llm_model {
  llm_config cfg;
  int hd;
  size_t es;
  char* packed;
  void* emb;
  void* out_w;
  float* final_norm;
  float* rope_cos;
  float* rope_sin;
  std::vector<LayerPtrs> layers;
  char* kv;
  size_t kv_half;  // bytes of one K (or V) section of one layer
  int* flags;      // [0] error bits, [1] generation step counter
  float* x;
  void* a;
  void* q;
  void* o;
  void* u;
  float* attn;
  void* amax;
  unsigned long long* akeys;  // device: [rows][LM-head GEMV workgroups] generation argmax keys
  float* splitk;
  size_t splitk_floats;
  int* rowmeta;          // device: [R] positions, [R] slots, [B] last-row indices (batched prefill)
  SeqDesc* seqtab;       // device: [B] sequence descriptors (batched prefill)
  float* last;           // device: [B][dim] gathered last rows (batched prefill)
  int* sync;             // device: decode-block counters, decode_block_sync_ints(G) per layer
  bool mfma_prefill;
  bool decode_block;     // batch-1 decode runs q|k|v, attention and wo as one launch
  hipStream_t cap_stream;
  std::vector<GraphEntry> graphs;
  // kernel timing (llm_set_kernel_timing)
  bool timing = false;
  struct Bracket { int kind; hipEvent_t a, b; };
  std::vector<Bracket> pending;
  std::vector<hipEvent_t> event_pool;
  int64_t t_launches[LLM_K_COUNT] = {};
  int64_t t_kernels[LLM_K_COUNT] = {};
  double t_ms[LLM_K_COUNT] = {};
};

namespace llm {
thread_local LaunchTimer* g_launch_timer = nullptr;
}

namespace {

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

hipEvent_t take_event(llm_model* m) {
  if (!m->event_pool.empty()) {
    hipEvent_t e = m->event_pool.back();
    m->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// While alive (and kernel timing is on), installs a launch timer on this thread:
// each kernel launched in its scope records a start / stop event pair with its
// dispatch, charged to group `kind`.  One Timed scope counts as one invocation.
struct ModelTimer final : LaunchTimer {
  llm_model* m = nullptr;
  int kind = 0;
  bool take(hipEvent_t* a, hipEvent_t* b) override {
    *a = take_event(m);
    if (!*a) return false;
    *b = take_event(m);
    if (!*b) {
      m->event_pool.push_back(*a);
      return false;
    }
    return true;
  }
  void done(hipEvent_t a, hipEvent_t b) override {
    m->pending.push_back({kind, a, b});
    m->t_kernels[kind] += 1;
  }
};

struct Timed {
  ModelTimer timer;
  LaunchTimer* prev = nullptr;
  bool on = false;
  Timed(llm_model* m, int kind, hipStream_t) {
    if (!m->timing) return;
    timer.m = m;
    timer.kind = kind;
    prev = g_launch_timer;
    g_launch_timer = &timer;
    m->t_launches[kind] += 1;
    on = true;
  }
  ~Timed() {
    if (on) g_launch_timer = prev;
  }
};

llm_status resolve_timing(llm_model* m) {
  for (auto& br : m->pending) {
    hipError_t e = hipEventSynchronize(br.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, br.a, br.b);
    if (e != hipSuccess) {
      m->pending.clear();
      return LLM_ERR_HIP;
    }
    m->t_ms[br.kind] += ms;
    m->event_pool.push_back(br.a);
    m->event_pool.push_back(br.b);
  }
  m->pending.clear();
  return LLM_OK;
}

void* k_section(llm_model* m, int l) { return m->kv + (size_t)(2 * l) * m->kv_half; }
void* v_section(llm_model* m, int l) { return m->kv + (size_t)(2 * l + 1) * m->kv_half; }

EpiParams base_epi(llm_model* m) {
  EpiParams e;
  std::memset(&e, 0, sizeof(e));
  e.n_heads = m->cfg.n_heads;
  e.n_kv_heads = m->cfg.n_kv_heads;
  e.head_dim = m->hd;
  e.max_seq = m->cfg.max_seq_len;
  e.n_slots = m->cfg.max_batch;
  e.rope_cos = m->rope_cos;
  e.rope_sin = m->rope_sin;
  e.err = m->flags;
  return e;
}

bool use_mfma(const llm_model* m, int M) { return m->cfg.dtype == LLM_BF16 && M > 8; }

// Scratch of the kernels that merge partial results: the split-KV attention chunks and the
// split-K projection slices.  Normally regions of the caller's workspace; the static device
// array for llm_decode_step_noalloc.
struct Partials {
  float* attn;
  float* splitk;
  size_t splitk_floats;
  int* sync;  // decode-block counters of every layer
};

Partials ws_partials(const llm_model* m) { return Partials{m->attn, m->splitk, m->splitk_floats, m->sync}; }

// y = A W^T with epilogue `ep`.  With norm_w, A is the fp32 residual stream and the
// projection consumes rmsnorm(A) * norm_w: fused into the GEMV, or a separate RMSNorm
// into m->a ahead of the MFMA GEMM.
void project(llm_model* m, const void* A, const void* W, int M, int N, int K, const EpiParams& ep, hipStream_t s,
             const Partials& pt, const float* norm_w = nullptr) {
  const llm_config& c = m->cfg;
  if (use_mfma(m, M)) {
    if (norm_w) {
      launch_rmsnorm(c.dtype, (const float*)A, norm_w, M, K, c.norm_eps, m->a, m->flags, s);
      A = m->a;
    }
    launch_gemm_f16(A, W, M, N, K, ep, pt.splitk, pt.splitk_floats, s);
  } else {
    launch_gemv(c.dtype, A, W, norm_w, c.norm_eps, M, N, K, ep, s);
  }
}

// The sequences of a batched prefill as the attention launch needs them: nseq descriptors on the
// device, n_blocks query blocks in all, the longest sequence max_n.
struct Varlen {
  const SeqDesc* seqs;
  int nseq, n_blocks, max_n;
};

// One decoder block on M rows of m->x.  Rows are either a prefill run
// (row_pos == nullptr: positions pos0.., slot slot0), a batched prefill (`vl`, with per-row
// positions and slots in row_pos / row_slot), or decode rows with their own positions and slots.
// a_ready: m->a already holds rmsnorm(x) with this layer's attention norm (left there by the
// previous layer's down projection).  next_norm: the next layer's attention norm, or null.
// Returns whether m->a now holds rmsnorm(x) with next_norm.  The two RMSNorms ahead of MFMA
// projections ride in the split-K reduction of the wo / down projection when that is split.
bool run_layer(llm_model* m, int l, int M, const int* row_pos, const int* row_slot, int pos0, int slot0,
               bool prefill, hipStream_t s, const Partials& pt, const Varlen* vl = nullptr, bool a_ready = false,
               const float* next_norm = nullptr) {
  const llm_config& c = m->cfg;
  const LayerPtrs& L = m->layers[l];
  const int H = c.n_heads, G = c.n_kv_heads, hd = m->hd, dim = c.dim, F = c.ffn_hidden_dim;

  if (!prefill && M == 1 && m->decode_block && row_pos && row_slot) {
    // q|k|v, attention and wo of the single decode row in one launch
    DecodeBlockParams dp;
    std::memset(&dp, 0, sizeof(dp));
    dp.x = m->x;
    dp.attn_norm = L.attn_norm;
    dp.wqkv = (const _Float16*)L.wqkv;
    dp.wo = (const _Float16*)L.wo;
    dp.q = (_Float16*)m->q;
    dp.o = (_Float16*)m->o;
    dp.kc = (_Float16*)k_section(m, l);
    dp.vc = (_Float16*)v_section(m, l);
    dp.rope_cos = m->rope_cos;
    dp.rope_sin = m->rope_sin;
    dp.row_pos = row_pos;
    dp.row_slot = row_slot;
    dp.partial = pt.attn;
    dp.sync = pt.sync + (size_t)l * decode_block_sync_ints(G);
    dp.err = m->flags;
    dp.eps = c.norm_eps;
    dp.dim = dim;
    dp.H = H;
    dp.G = G;
    dp.max_seq = c.max_seq_len;
    dp.n_slots = c.max_batch;
    {
      Timed t(m, LLM_K_DECODE_BLOCK, s);
      launch_decode_block(dp, s);
    }
    EpiParams g = base_epi(m);
    g.kind = EPI_SWIGLU;
    g.out_act = m->u;
    g.ld = F;
    {
      Timed t(m, LLM_K_GATE_UP, s);
      project(m, m->x, L.w13, M, 2 * F, dim, g, s, pt, L.ffn_norm);
    }
    EpiParams r = base_epi(m);
    r.kind = EPI_RESID;
    r.out_f32 = m->x;
    r.ld = dim;
    {
      Timed t(m, LLM_K_DOWN, s);
      project(m, m->u, L.w2, M, dim, F, r, s, pt);
    }
    return false;
  }

  EpiParams e = base_epi(m);
  e.kind = EPI_QKV;
  e.out_act = m->q;
  e.ld = H * hd;
  e.k_cache = k_section(m, l);
  e.v_cache = v_section(m, l);
  e.row_pos = row_pos;
  e.row_slot = row_slot;
  e.pos0 = pos0;
  e.slot0 = slot0;
  {
    Timed t(m, LLM_K_QKV, s);
    if (a_ready)
      launch_gemm_f16(m->a, L.wqkv, M, (H + 2 * G) * hd, dim, e, pt.splitk, pt.splitk_floats, s);
    else
      project(m, m->x, L.wqkv, M, (H + 2 * G) * hd, dim, e, s, pt, L.attn_norm);
  }

  {
    Timed t(m, LLM_K_ATTN, s);
    if (prefill && m->mfma_prefill && vl) {
      launch_attn_prefill_varlen(m->q, k_section(m, l), v_section(m, l), vl->seqs, vl->nseq, vl->n_blocks, vl->max_n,
                                 H, G, hd, c.max_seq_len, m->o, s);
    } else if (prefill && m->mfma_prefill && !row_pos)
      launch_attn_prefill(m->q, k_section(m, l), v_section(m, l), slot0, pos0, M, H, G, hd, c.max_seq_len, m->o, s);
    else
      launch_attn_decode(c.dtype, m->q, k_section(m, l), v_section(m, l), row_pos, row_slot, pos0, slot0, M, H, G,
                         hd, c.max_seq_len, c.max_batch, pt.attn, m->o, m->flags, s);
  }

  EpiParams r = base_epi(m);
  r.kind = EPI_RESID;
  r.out_f32 = m->x;
  r.ld = dim;
  bool ffn_ready = false;
  {
    Timed t(m, LLM_K_WO, s);
    if (use_mfma(m, M))
      ffn_ready = launch_gemm_f16_resid_norm(m->o, L.wo, M, dim, H * hd, r, L.ffn_norm, c.norm_eps, m->a, pt.splitk,
                                             pt.splitk_floats, s);
    if (!ffn_ready) project(m, m->o, L.wo, M, dim, H * hd, r, s, pt);
  }

  EpiParams g = base_epi(m);
  g.kind = EPI_SWIGLU;
  g.out_act = m->u;
  g.ld = F;
  {
    Timed t(m, LLM_K_GATE_UP, s);
    if (ffn_ready)
      launch_gemm_f16(m->a, L.w13, M, 2 * F, dim, g, pt.splitk, pt.splitk_floats, s);
    else
      project(m, m->x, L.w13, M, 2 * F, dim, g, s, pt, L.ffn_norm);
  }

  bool next_ready = false;
  {
    Timed t(m, LLM_K_DOWN, s);
    if (next_norm && use_mfma(m, M))
      next_ready = launch_gemm_f16_resid_norm(m->u, L.w2, M, dim, F, r, next_norm, c.norm_eps, m->a, pt.splitk,
                                              pt.splitk_floats, s);
    if (!next_ready) project(m, m->u, L.w2, M, dim, F, r, s, pt);
  }
  return next_ready;
}

// All layers over M rows, each passing its successor the attention-normed activations when its
// down projection produced them.
void run_layers(llm_model* m, int M, const int* row_pos, const int* row_slot, int pos0, int slot0, bool prefill,
                hipStream_t s, const Partials& pt, const Varlen* vl = nullptr) {
  const int n = m->cfg.n_layers;
  bool a_ready = false;
  for (int l = 0; l < n; ++l)
    a_ready = run_layer(m, l, M, row_pos, row_slot, pos0, slot0, prefill, s, pt, vl, a_ready,
                        l + 1 < n ? m->layers[l + 1].attn_norm : nullptr);
}

// Device address of `scratch` on the current device, resolved once per device with that device
// current (each GPU holds its own copy at its own address).
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // by device ordinal

hipError_t noalloc_scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Partial floats a decode step of `batch` rows needs: the attention chunks its launcher picks,
// and the largest split-K slice set of its projections (the bound launch_gemm_f16 plans with).
void decode_partials_need(const llm_model* m, int batch, size_t* attn_floats, size_t* splitk_floats,
                          size_t* sync_ints) {
  const llm_config& c = m->cfg;
  const int hd = m->hd, H = c.n_heads, G = c.n_kv_heads;
  *attn_floats = attn_decode_partial_floats_used(c.dtype, batch, H, G, hd, c.max_seq_len);
  *sync_ints = 0;
  if (batch == 1 && m->decode_block) {
    *attn_floats = std::max(*attn_floats, decode_block_partial_floats(H, c.max_seq_len));
    *sync_ints = (size_t)c.n_layers * decode_block_sync_ints(G);
  }
  size_t sk = 0;
  if (use_mfma(m, batch)) {
    const int shapes[5][2] = {{(H + 2 * G) * hd, c.dim}, {c.dim, H * hd}, {2 * c.ffn_hidden_dim, c.dim},
                              {c.dim, c.ffn_hidden_dim}, {c.vocab_size, c.dim}};
    for (auto& sh : shapes) sk = std::max(sk, gemm_splitk_floats(batch, sh[0], sh[1]));
  }
  *splitk_floats = sk;
}

llm_status hip_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LLM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return LLM_OK;
}

// Final RMSNorm of `rows` rows starting at x_row0, then the output projection.
// Whether the LM head of `rows` rows runs on the fp16 GEMV, which can fold the greedy argmax
// into m->akeys as it stores the logits.
bool lm_head_folds_argmax(const llm_model* m, int rows) {
  return m->cfg.dtype == LLM_BF16 && !use_mfma(m, rows) && rows <= AMAX_ROWS;
}

void lm_head(llm_model* m, const float* x_rows, int rows, float* logits, hipStream_t s, const Partials& pt,
             bool fold_argmax = false) {
  const llm_config& c = m->cfg;
  Timed t(m, LLM_K_LM_HEAD, s);
  EpiParams e = base_epi(m);
  e.kind = EPI_STORE_F32;
  e.out_f32 = logits;
  e.ld = c.vocab_size;
  if (fold_argmax && lm_head_folds_argmax(m, rows)) e.amax_keys = m->akeys;
  project(m, x_rows, m->out_w, rows, c.vocab_size, c.dim, e, s, pt, m->final_norm);
}

void enqueue_decode(llm_model* m, int batch, const int* slots, const int* positions, const int* tokens, float* logits,
                    hipStream_t s, const Partials& pt, bool fold_argmax = false) {
  const llm_config& c = m->cfg;
  {
    // the embedding kernel also clears the decode block's counters of every layer
    Timed t(m, LLM_K_EMBED, s);
    const bool blk = batch == 1 && m->decode_block;
    launch_embed(c.dtype, m->emb, tokens, batch, c.dim, c.vocab_size, m->x, m->flags, s, blk ? pt.sync : nullptr,
                 blk ? c.n_layers * decode_block_sync_ints(c.n_kv_heads) / DB_SYNC_LINE : 0, DB_SYNC_LINE);
  }
  run_layers(m, batch, positions, slots, 0, 0, false, s, pt);
  lm_head(m, m->x, batch, logits, s, pt, fold_argmax);
}

// The end of a generation step: the greedy token of each row into tokens_dev, then the advance.
void enqueue_next_token(llm_model* m, int batch, int* positions_dev, int* tokens_dev, int* out_tokens_dev,
                        const float* logits_dev, int* step, hipStream_t s) {
  if (lm_head_folds_argmax(m, batch)) {
    launch_advance_keys(m->akeys, gemv_h_blocks(batch, m->cfg.vocab_size, m->cfg.dim), positions_dev, tokens_dev,
                        out_tokens_dev, step, batch, s);
  } else {
    launch_argmax(logits_dev, batch, m->cfg.vocab_size, m->amax, tokens_dev, s);
    launch_advance(positions_dev, tokens_dev, out_tokens_dev, step, batch, s);
  }
}

}  // namespace

extern "C" {

llm_status llm_check_config(const llm_config* cfg) {
  std::string why;
  if (!config_ok(cfg, &why)) return fail(LLM_ERR_CONFIG, why);
  return LLM_OK;
}

size_t llm_packed_weight_bytes(const llm_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  return PackedLayout(*cfg).total;
}

size_t llm_kv_cache_bytes(const llm_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  return kv_bytes(*cfg);
}

size_t llm_workspace_bytes(const llm_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  return WorkLayout(*cfg).total;
}

llm_status llm_init_weights(const llm_config* cfg, const llm_weights* w, void* packed, size_t packed_bytes,
                            void* kv_cache, size_t kv_cache_bytes, void* workspace, size_t workspace_bytes,
                            void* stream, llm_model** out) {
  if (!out) return fail(LLM_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  std::string why;
  if (!config_ok(cfg, &why)) return fail(LLM_ERR_CONFIG, why);
  if (!w || !packed || !kv_cache || !workspace) return fail(LLM_ERR_INVALID_ARG, "weights or a buffer is NULL");
  const llm_config& c = *cfg;
  Dims d(c);
  if (!w->tok_embeddings || !w->norm || !w->output || !w->attention_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
      !w->ffn_norm || !w->w1 || !w->w3 || !w->w2)
    return fail(LLM_ERR_INVALID_ARG, "a weight pointer is NULL");
  for (int l = 0; l < d.L; ++l)
    if (!w->attention_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->ffn_norm[l] || !w->w1[l] ||
        !w->w3[l] || !w->w2[l])
      return fail(LLM_ERR_INVALID_ARG, "layer " + std::to_string(l) + " has a NULL weight pointer");
  PackedLayout pl(c);
  WorkLayout wl(c);
  if (packed_bytes < pl.total) return fail(LLM_ERR_BUFFER_TOO_SMALL, "packed weight buffer too small");
  if (kv_cache_bytes < kv_bytes(c)) return fail(LLM_ERR_BUFFER_TOO_SMALL, "KV cache buffer too small");
  if (workspace_bytes < wl.total) return fail(LLM_ERR_BUFFER_TOO_SMALL, "workspace buffer too small");

  hipStream_t s = as_stream(stream);
  llm_model* m = new llm_model();
  m->cfg = c;
  m->hd = d.hd;
  m->es = d.es;
  m->packed = (char*)packed;
  m->emb = m->packed + pl.emb;
  m->out_w = m->packed + pl.out;
  m->final_norm = (float*)(m->packed + pl.norm);
  m->rope_cos = (float*)(m->packed + pl.cos);
  m->rope_sin = (float*)(m->packed + pl.sin);
  m->layers.resize(d.L);
  m->kv = (char*)kv_cache;
  m->kv_half = (size_t)d.B * d.G * d.S * d.hd * d.es;
  char* ws = (char*)workspace;
  m->flags = (int*)(ws + wl.flags);
  m->x = (float*)(ws + wl.x);
  m->a = ws + wl.a;
  m->q = ws + wl.q;
  m->o = ws + wl.o;
  m->u = ws + wl.u;
  m->attn = (float*)(ws + wl.attn);
  m->amax = ws + wl.amax;
  m->akeys = (unsigned long long*)(ws + wl.akeys);
  m->splitk = (float*)(ws + wl.splitk);
  m->splitk_floats = wl.splitk_floats;
  m->rowmeta = (int*)(ws + wl.rowmeta);
  m->seqtab = (SeqDesc*)(ws + wl.seqtab);
  m->last = (float*)(ws + wl.last);
  m->sync = (int*)(ws + wl.sync);
  m->decode_block = decode_block_supported(c.dtype, c.dim, c.n_heads, c.n_kv_heads);
  m->mfma_prefill = c.dtype == LLM_BF16 && attn_prefill_supported(d.hd, d.H, d.G);
  m->cap_stream = nullptr;

  const size_t es = d.es;
  const size_t row = (size_t)d.dim * es;
  hipError_t e = hipSuccess;
  const bool h = c.dtype == LLM_BF16;
  // The device error flags start cleared; weight packing may raise LLM_DEVERR_RANGE.
  launch_fill_i32(m->flags, 0, 64, s);
  // Copy rows [0, rows) of src ([rows][cols]) to dst rows r * mult + off.  The fp32
  // path copies as is; bf16 weights are stored as fp16 (exact inside fp16's normal
  // range; an out-of-range weight raises LLM_DEVERR_RANGE).
  auto put = [&](void* dst, const void* src, size_t rows, int cols, int mult, int off) {
    if (e != hipSuccess) return;
    if (h) {
      launch_pack_rows(src, dst, rows, cols, mult, off, m->flags, s);
    } else if (mult == 1) {
      e = hipMemcpyAsync((char*)dst + (size_t)off * cols * 4, src, rows * cols * 4, hipMemcpyDeviceToDevice, s);
    } else {
      e = hipMemcpy2DAsync((char*)dst + (size_t)off * cols * 4, (size_t)mult * cols * 4, src, (size_t)cols * 4,
                           (size_t)cols * 4, rows, hipMemcpyDeviceToDevice, s);
    }
  };
  put(m->emb, w->tok_embeddings, d.V, d.dim, 1, 0);
  put(m->out_w, w->output, d.V, d.dim, 1, 0);
  launch_to_f32(c.dtype, w->norm, m->final_norm, d.dim, s);
  for (int l = 0; l < d.L; ++l) {
    char* base = m->packed + pl.layer0 + (size_t)l * pl.layer_stride;
    LayerPtrs& L = m->layers[l];
    L.attn_norm = (float*)(base + pl.l_attn_norm);
    L.ffn_norm = (float*)(base + pl.l_ffn_norm);
    L.wqkv = base + pl.l_wqkv;
    L.wo = base + pl.l_wo;
    L.w13 = base + pl.l_w13;
    L.w2 = base + pl.l_w2;
    launch_to_f32(c.dtype, w->attention_norm[l], L.attn_norm, d.dim, s);
    launch_to_f32(c.dtype, w->ffn_norm[l], L.ffn_norm, d.dim, s);
    // q|k|v rows concatenated.
    put(L.wqkv, w->wq[l], (size_t)d.H * d.hd, d.dim, 1, 0);
    put((char*)L.wqkv + (size_t)d.H * d.hd * row, w->wk[l], (size_t)d.G * d.hd, d.dim, 1, 0);
    put((char*)L.wqkv + (size_t)(d.H + d.G) * d.hd * row, w->wv[l], (size_t)d.G * d.hd, d.dim, 1, 0);
    put(L.wo, w->wo[l], d.dim, d.H * d.hd, 1, 0);
    // w1 / w3 rows interleaved: packed row 2c = w1 row c, 2c + 1 = w3 row c.
    put(L.w13, w->w1[l], d.F, d.dim, 2, 0);
    put(L.w13, w->w3[l], d.F, d.dim, 2, 1);
    put(L.w2, w->w2[l], d.dim, d.F, 1, 0);
  }
  // RoPE tables: angle(pos, j) = pos * theta^(-2j/hd) in fp64, stored as fp32 cos / sin.
  const int half = d.hd / 2;
  std::vector<float> hc((size_t)d.S * half), hs((size_t)d.S * half);
  for (int j = 0; j < half; ++j) {
    const double f = std::pow((double)c.rope_theta, -2.0 * j / (double)d.hd);
    for (int p = 0; p < d.S; ++p) {
      const double a = (double)p * f;
      hc[(size_t)p * half + j] = (float)std::cos(a);
      hs[(size_t)p * half + j] = (float)std::sin(a);
    }
  }
  if (e == hipSuccess) e = hipMemcpyAsync(m->rope_cos, hc.data(), hc.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemcpyAsync(m->rope_sin, hs.data(), hs.size() * 4, hipMemcpyHostToDevice, s);

  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&m->cap_stream, hipStreamNonBlocking);
  // Resolve llm_decode_step_noalloc's static array on this device now; a failure here is
  // reported by that call (which retries), not by the model's creation.
  void* scratch_dev = nullptr;
  if (e == hipSuccess && noalloc_scratch_ptr(&scratch_dev) != hipSuccess) (void)hipGetLastError();
  if (e != hipSuccess) {
    delete m;
    return fail(LLM_ERR_HIP, std::string("init: ") + hipGetErrorString(e));
  }
  *out = m;
  return LLM_OK;
}

llm_status llm_prefill(llm_model* m, int32_t slot, const int32_t* tokens_dev, int32_t n_tokens, int32_t start_pos,
                       float* logits_dev, void* stream) {
  if (!m || !tokens_dev || !logits_dev) return fail(LLM_ERR_INVALID_ARG, "NULL model, tokens or logits");
  const llm_config& c = m->cfg;
  if (n_tokens < 1) return fail(LLM_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (n_tokens > c.max_prefill_tokens) return fail(LLM_ERR_OUT_OF_RANGE, "n_tokens > max_prefill_tokens");
  if (slot < 0 || slot >= c.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "slot out of range");
  if (start_pos < 0 || (long long)start_pos + n_tokens > c.max_seq_len)
    return fail(LLM_ERR_OUT_OF_RANGE, "start_pos + n_tokens > max_seq_len");
  hipStream_t s = as_stream(stream);
  {
    Timed t(m, LLM_K_EMBED, s);
    launch_embed(c.dtype, m->emb, tokens_dev, n_tokens, c.dim, c.vocab_size, m->x, m->flags, s);
  }
  run_layers(m, n_tokens, nullptr, nullptr, start_pos, slot, true, s, ws_partials(m));
  lm_head(m, m->x + (size_t)(n_tokens - 1) * c.dim, 1, logits_dev, s, ws_partials(m));
  return hip_check("prefill launch");
}

llm_status llm_prefill_batch(llm_model* m, int32_t batch, const int32_t* slots_host, const int32_t* starts_host,
                             const int32_t* lens_host, const int32_t* tokens_dev, float* logits_dev, void* stream) {
  if (!m || !slots_host || !starts_host || !lens_host || !tokens_dev || !logits_dev)
    return fail(LLM_ERR_INVALID_ARG, "NULL model, array or buffer");
  const llm_config& c = m->cfg;
  if (batch < 1) return fail(LLM_ERR_INVALID_ARG, "batch must be >= 1");
  if (batch > c.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "batch > max_batch");
  std::vector<SeqDesc> seqs((size_t)batch);
  std::vector<char> used((size_t)c.max_batch, 0);
  long long total = 0;
  int max_n = 0;
  for (int b = 0; b < batch; ++b) {
    const int slot = slots_host[b], start = starts_host[b], n = lens_host[b];
    if (n < 1) return fail(LLM_ERR_INVALID_ARG, "every sequence needs >= 1 token");
    if (slot < 0 || slot >= c.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "slot out of range");
    if (used[slot]) return fail(LLM_ERR_INVALID_ARG, "two sequences share a slot");
    used[slot] = 1;
    if (start < 0 || (long long)start + n > c.max_seq_len)
      return fail(LLM_ERR_OUT_OF_RANGE, "start + length > max_seq_len");
    if (total + n > c.max_prefill_tokens) return fail(LLM_ERR_OUT_OF_RANGE, "total tokens > max_prefill_tokens");
    std::memset(&seqs[b], 0, sizeof(SeqDesc));
    seqs[b].row0 = (int)total;
    seqs[b].n = n;
    seqs[b].start = start;
    seqs[b].slot = slot;
    total += n;
    max_n = std::max(max_n, n);
  }
  const int T = (int)total;
  // Query blocks of each sequence in the one attention launch.
  int n_blocks = 0;
  if (m->mfma_prefill) {
    const int qb = attn_prefill_block_rows(max_n, c.n_heads, c.n_kv_heads);
    for (SeqDesc& q : seqs) {
      q.blk0 = n_blocks;
      n_blocks += (q.n + qb - 1) / qb;
    }
  }
  const int R = std::max(c.max_prefill_tokens, c.max_batch);
  int* row_pos = m->rowmeta;
  int* row_slot = m->rowmeta + R;
  int* last_idx = m->rowmeta + 2 * R;
  hipStream_t s = as_stream(stream);
  // The per-sequence descriptors travel in kernel arguments, which the launch copies: no host
  // staging buffer, so nothing here waits for the device.
  for (int b0 = 0; b0 < batch; b0 += SEQ_META_CHUNK) {
    SeqMetaChunk ch;
    std::memset(&ch, 0, sizeof(ch));
    ch.first = b0;
    ch.count = std::min(SEQ_META_CHUNK, batch - b0);
    for (int i = 0; i < ch.count; ++i) ch.d[i] = seqs[b0 + i];
    launch_seq_meta(ch, row_pos, row_slot, last_idx, m->seqtab, s);
  }
  {
    Timed t(m, LLM_K_EMBED, s);
    launch_embed(c.dtype, m->emb, tokens_dev, T, c.dim, c.vocab_size, m->x, m->flags, s);
  }
  const Varlen vl{m->seqtab, batch, n_blocks, max_n};
  run_layers(m, T, row_pos, row_slot, 0, 0, true, s, ws_partials(m), &vl);
  launch_gather_rows(m->x, last_idx, batch, c.dim, m->last, s);
  lm_head(m, m->last, batch, logits_dev, s, ws_partials(m));
  return hip_check("batched prefill launch");
}

llm_status llm_layer_forward(llm_model* m, int32_t layer, int32_t slot, float* x_dev, int32_t n_tokens,
                             int32_t start_pos, void* stream) {
  if (!m || !x_dev) return fail(LLM_ERR_INVALID_ARG, "NULL model or x");
  const llm_config& c = m->cfg;
  if (layer < 0 || layer >= c.n_layers) return fail(LLM_ERR_OUT_OF_RANGE, "layer out of range");
  if (n_tokens < 1) return fail(LLM_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (n_tokens > c.max_prefill_tokens) return fail(LLM_ERR_OUT_OF_RANGE, "n_tokens > max_prefill_tokens");
  if (slot < 0 || slot >= c.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "slot out of range");
  if (start_pos < 0 || (long long)start_pos + n_tokens > c.max_seq_len)
    return fail(LLM_ERR_OUT_OF_RANGE, "start_pos + n_tokens > max_seq_len");
  hipStream_t s = as_stream(stream);
  hipError_t e = hipMemcpyAsync(m->x, x_dev, (size_t)n_tokens * c.dim * 4, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return fail(LLM_ERR_HIP, hipGetErrorString(e));
  run_layer(m, layer, n_tokens, nullptr, nullptr, start_pos, slot, true, s, ws_partials(m));
  e = hipMemcpyAsync(x_dev, m->x, (size_t)n_tokens * c.dim * 4, hipMemcpyDeviceToDevice, s);
  if (e != hipSuccess) return fail(LLM_ERR_HIP, hipGetErrorString(e));
  return hip_check("layer launch");
}

llm_status llm_decode_step(llm_model* m, int32_t batch, const int32_t* slots_dev, const int32_t* positions_dev,
                           const int32_t* tokens_dev, float* logits_dev, void* stream) {
  if (!m || !slots_dev || !positions_dev || !tokens_dev || !logits_dev)
    return fail(LLM_ERR_INVALID_ARG, "NULL model or buffer");
  if (batch < 1) return fail(LLM_ERR_INVALID_ARG, "batch must be >= 1");
  if (batch > m->cfg.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "batch > max_batch");
  enqueue_decode(m, batch, slots_dev, positions_dev, tokens_dev, logits_dev, as_stream(stream), ws_partials(m));
  return hip_check("decode launch");
}

llm_status llm_decode_step_noalloc(llm_model* m, int32_t batch, const int32_t* slots_dev,
                                   const int32_t* positions_dev, const int32_t* tokens_dev, float* logits_dev,
                                   void* stream) {
  if (!m || !slots_dev || !positions_dev || !tokens_dev || !logits_dev)
    return fail(LLM_ERR_INVALID_ARG, "NULL model or buffer");
  if (batch < 1) return fail(LLM_ERR_INVALID_ARG, "batch must be >= 1");
  if (batch > m->cfg.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "batch > max_batch");
  size_t attn_f = 0, splitk_f = 0, sync_n = 0;
  decode_partials_need(m, batch, &attn_f, &splitk_f, &sync_n);
  const size_t attn_bytes = align256(attn_f * sizeof(float));
  const size_t splitk_bytes = align256(splitk_f * sizeof(float));
  const size_t need = attn_bytes + splitk_bytes + sync_n * sizeof(int);
  if (need > LLM_NOALLOC_SCRATCH_BYTES)
    return fail(LLM_ERR_OUT_OF_RANGE, "a decode step of " + std::to_string(batch) + " rows needs " +
                                          std::to_string(need) + " bytes of scratch, more than the " +
                                          std::to_string(LLM_NOALLOC_SCRATCH_BYTES) +
                                          " the library holds for llm_decode_step_noalloc");
  void* base = nullptr;
  const hipError_t e = noalloc_scratch_ptr(&base);
  if (e != hipSuccess) return fail(LLM_ERR_HIP, std::string("static scratch address: ") + hipGetErrorString(e));
  const Partials pt{(float*)base, (float*)((char*)base + attn_bytes), splitk_f,
                    (int*)((char*)base + attn_bytes + splitk_bytes)};
  enqueue_decode(m, batch, slots_dev, positions_dev, tokens_dev, logits_dev, as_stream(stream), pt);
  return hip_check("decode launch");
}

llm_status llm_argmax(const float* logits_dev, int32_t rows, int32_t vocab, int32_t* out_dev, void* stream) {
  if (!logits_dev || !out_dev) return fail(LLM_ERR_INVALID_ARG, "NULL logits or out");
  if (rows < 1 || vocab < 1) return fail(LLM_ERR_INVALID_ARG, "rows and vocab must be >= 1");
  launch_argmax_rows(logits_dev, rows, vocab, out_dev, as_stream(stream));
  return hip_check("argmax launch");
}

llm_status llm_generate(llm_model* m, int32_t batch, const int32_t* slots_dev, int32_t* positions_dev,
                        int32_t* tokens_dev, int32_t n_steps, int32_t* out_tokens_dev, float* logits_dev,
                        void* stream) {
  if (!m || !slots_dev || !positions_dev || !tokens_dev || !out_tokens_dev || !logits_dev)
    return fail(LLM_ERR_INVALID_ARG, "NULL model or buffer");
  if (batch < 1 || n_steps < 0) return fail(LLM_ERR_INVALID_ARG, "batch must be >= 1 and n_steps >= 0");
  if (batch > m->cfg.max_batch) return fail(LLM_ERR_OUT_OF_RANGE, "batch > max_batch");
  hipStream_t s = as_stream(stream);
  if (n_steps == 0) return LLM_OK;
  int* step = m->flags + 1;
  launch_fill_i32(step, 0, 1, s);

  const void* key[5] = {slots_dev, positions_dev, tokens_dev, out_tokens_dev, logits_dev};
  hipGraphExec_t exec = nullptr;
  if (!m->timing)
    for (auto& g : m->graphs)
      if (g.batch == batch && !std::memcmp(g.ptrs, key, sizeof(key))) exec = g.exec;
  if (!exec && !m->timing) {
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamBeginCapture(m->cap_stream, hipStreamCaptureModeRelaxed);
    if (e == hipSuccess) {
      enqueue_decode(m, batch, slots_dev, positions_dev, tokens_dev, logits_dev, m->cap_stream, ws_partials(m), true);
      enqueue_next_token(m, batch, positions_dev, tokens_dev, out_tokens_dev, logits_dev, step, m->cap_stream);
      e = hipStreamEndCapture(m->cap_stream, &graph);
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (graph) (void)hipGraphDestroy(graph);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      exec = nullptr;
    } else {
      if (m->graphs.size() >= 8) {
        (void)hipGraphExecDestroy(m->graphs.front().exec);
        m->graphs.erase(m->graphs.begin());
      }
      GraphEntry ge;
      ge.batch = batch;
      std::memcpy(ge.ptrs, key, sizeof(key));
      ge.exec = exec;
      m->graphs.push_back(ge);
    }
  }
  for (int i = 0; i < n_steps; ++i) {
    if (exec) {
      hipError_t e = hipGraphLaunch(exec, s);
      if (e != hipSuccess) return fail(LLM_ERR_HIP, std::string("graph launch: ") + hipGetErrorString(e));
    } else {
      enqueue_decode(m, batch, slots_dev, positions_dev, tokens_dev, logits_dev, s, ws_partials(m), true);
      Timed t(m, LLM_K_ARGMAX, s);
      enqueue_next_token(m, batch, positions_dev, tokens_dev, out_tokens_dev, logits_dev, step, s);
    }
  }
  return hip_check("generate launch");
}

llm_status llm_read_device_error(llm_model* m, int32_t* flags, void* stream) {
  if (!m || !flags) return fail(LLM_ERR_INVALID_ARG, "NULL model or flags");
  hipStream_t s = as_stream(stream);
  int host = 0;
  hipError_t e = hipMemcpyAsync(&host, m->flags, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(LLM_ERR_HIP, hipGetErrorString(e));
  launch_fill_i32(m->flags, 0, 1, s);
  *flags = host;
  return hip_check("clear device error");
}

llm_status llm_set_kernel_timing(llm_model* m, int32_t enable) {
  if (!m) return fail(LLM_ERR_INVALID_ARG, "NULL model");
  if (resolve_timing(m) != LLM_OK) return fail(LLM_ERR_HIP, "timing events failed");
  m->timing = enable != 0;
  for (int k = 0; k < LLM_K_COUNT; ++k) { m->t_launches[k] = 0; m->t_kernels[k] = 0; m->t_ms[k] = 0.0; }
  return LLM_OK;
}

llm_status llm_kernel_timing(llm_model* m, int32_t kind, int64_t* launches, int64_t* kernels, double* total_ms) {
  if (!m || !launches || !total_ms) return fail(LLM_ERR_INVALID_ARG, "NULL model or output");
  if (kind < 0 || kind >= LLM_K_COUNT) return fail(LLM_ERR_INVALID_ARG, "unknown kernel group");
  if (resolve_timing(m) != LLM_OK) return fail(LLM_ERR_HIP, "timing events failed");
  *launches = m->t_launches[kind];
  if (kernels) *kernels = m->t_kernels[kind];
  *total_ms = m->t_ms[kind];
  return LLM_OK;
}

void llm_free(llm_model* m) {
  if (!m) return;
  (void)resolve_timing(m);
  for (auto e : m->event_pool) (void)hipEventDestroy(e);
  for (auto& g : m->graphs) (void)hipGraphExecDestroy(g.exec);
  if (m->cap_stream) (void)hipStreamDestroy(m->cap_stream);
  delete m;
}

const char* llm_status_string(llm_status s) {
  switch ((int)s) {
    case LLM_OK: return "ok";
    case LLM_ERR_INVALID_ARG: return "invalid argument";
    case LLM_ERR_CONFIG: return "invalid configuration";
    case LLM_ERR_OUT_OF_RANGE: return "out of range";
    case LLM_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case LLM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* llm_last_error_message(void) { return g_err.c_str(); }

}  // extern "C"
