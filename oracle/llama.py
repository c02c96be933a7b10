"""Plain NumPy definition of the Llama-2/3 decoder forward pass (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Nothing here is
blocked, fused or reordered beyond what the definition states; matrix products
call ``numpy.matmul`` and everything else is written out.

Sources (web pages, cited by title and section):

* [LLAMA3-NP]  "Model Llama 3 yang Diimplementasikan dengan NumPy Murni"
  (GeekNews, Indonesian): sections Struktur, RoPE #1, RMSNorm, QKV, RoPE #2,
  KV cache, GQA, Scaled Dot-Product Attention, Feed Forward, SwiGLU, Linear,
  Generasi.
* [LLAMA3-SCRATCH]  "Building llama3 from scratch" (downcodes, Arabic): the
  params.json printout, the weight-name listing, the ``rms_norm`` code, the
  printed weight shapes and the per-head view of wq.
* [LLAMA3-ES]  "Resumen de una implementación desde cero del modelo LLaMA-3"
  (GeekNews, Spanish): the bullet walk-through (attention, multi-head,
  feed-forward, repeated layers, token prediction).
* [LLAMA2-FR]  "LLaMA2" (downcodes, French): RMSNorm, SwiGLU, RoPE, GQA/MQA and
  KV-cache paragraphs.

Readings where the pages are silent (each one is listed in the design notes):
attention scale 1/sqrt(head_dim); RoPE frequency theta^(-2j/d) on interleaved
pairs (2j, 2j+1), 0-based positions; query head h reads KV head
h // (n_heads / n_kv_heads); SwiGLU is w2(silu(w1 x) * w3 x); separate final
``norm`` and untied ``output`` weights; greedy ties go to the lowest id.

Precision: the caller picks the matmul dtype (float64 for small models, float32
for the 8B shape); RMSNorm statistics and the softmax are always float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class OracleConfig:
    """Model hyper-parameters: the params.json field set ([LLAMA3-SCRATCH], params.json
    printout) with the FFN width given explicitly and the context length added
    ([LLAMA3-NP], Struktur: max_seq_len)."""

    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int
    ffn_hidden_dim: int
    max_seq_len: int
    rope_theta: float
    norm_eps: float

    @property
    def head_dim(self) -> int:
        # [LLAMA3-SCRATCH], per-head view of wq: head_dim = rows of wq / n_heads.
        return self.dim // self.n_heads


# ----------------------------------------------------------------------------- RMSNorm

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * 1/sqrt(mean(x^2) + eps) * w.

    [LLAMA3-SCRATCH], the ``rms_norm`` function (mean of the squares along the
    last dimension, eps added inside the reciprocal square root, then the
    weight); [LLAMA3-NP], RMSNorm.  Statistics in float64.
    """
    x64 = np.asarray(x, np.float64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    y = x64 / np.sqrt(ms + eps) * np.asarray(w, np.float64)
    return y.astype(np.result_type(x.dtype, np.float32), copy=False)


# ----------------------------------------------------------------------------- RoPE

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotation frequency of pair j: theta^(-2j/head_dim), j = 0..head_dim/2-1 (float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def rope_cos_sin(positions, head_dim: int, theta: float):
    """Precomputed RoPE tables: angles = outer(positions, frequencies), then cos and sin.

    [LLAMA3-NP], RoPE #1: cos and sin are computed up front from an ``np.outer``
    product and reused for Q and K.  float64, shape [len(positions), head_dim/2].
    """
    ang = np.outer(np.asarray(positions, np.float64), rope_inv_freq(head_dim, theta))
    return np.cos(ang), np.sin(ang)


def apply_rope(v: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each pair (v[2j], v[2j+1]) of every head by the angle of its row.

    [LLAMA3-NP], RoPE #2: the input is split into the two members of each pair,
    multiplied by cos and sin, added and subtracted, and put back in place;
    applied to Q and K only.  [LLAMA2-FR], RoPE: a rotation matrix whose angle
    grows with position, so that q.k depends only on the relative offset.
    v: [n, heads, head_dim]; cos, sin: [n, head_dim/2].
    """
    v = np.asarray(v)
    c = cos[:, None, :]
    s = sin[:, None, :]
    x0 = v[..., 0::2]
    x1 = v[..., 1::2]
    out = np.empty(v.shape, np.result_type(v.dtype, np.float32))
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------- attention

def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax with the maximum subtracted first (float64)."""
    s = np.asarray(s, np.float64)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def causal_gqa_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos) -> np.ndarray:
    """Causal grouped-query scaled dot-product attention.

    q: [n, H, d] queries at absolute positions ``q_pos`` ([n]); k, v: [T, G, d]
    keys/values of positions 0..T-1.  For each head h and query i: scores
    q.k_j / sqrt(d) over the keys j <= q_pos[i] (later keys are masked out),
    softmax, then the weighted sum of the values ([LLAMA3-ES], attention and
    multi-head bullets; [LLAMA3-NP], Scaled Dot-Product Attention).  Query head
    h reads KV head h // (H / G) ([LLAMA3-NP], GQA; [LLAMA2-FR], GQA/MQA).
    Returns the heads concatenated head-major: [n, H*d].
    """
    n, H, d = q.shape
    T, G, _ = k.shape
    group = H // G
    q_pos = np.asarray(q_pos, np.int64)
    dt = np.result_type(q.dtype, np.float32)
    out = np.zeros((n, H, d), dt)
    future = np.arange(T)[None, :] > q_pos[:, None]  # [n, T]
    for h in range(H):
        g = h // group
        s = (q[:, h, :] @ k[:, g, :].T).astype(np.float64) / math.sqrt(d)
        s = np.where(future, -np.inf, s)
        p = softmax(s, axis=-1)
        out[:, h, :] = (p @ np.asarray(v[:, g, :], np.float64)).astype(dt)
    return out.reshape(n, H * d)


# ----------------------------------------------------------------------------- feed-forward

def silu(z: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z)
    return z / (1.0 + np.exp(-z))


def feed_forward(b: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """SwiGLU feed-forward of three bias-free linears: w2( silu(b w1^T) * (b w3^T) ).

    [LLAMA3-NP], Feed Forward and SwiGLU: a swish value times the x_V branch,
    then scaled back down by the third linear; [LLAMA3-ES], feed-forward bullet.
    """
    return (silu(b @ w1.T) * (b @ w3.T)) @ w2.T


# ----------------------------------------------------------------------------- layer and model

def decoder_layer(x, lw: dict, cfg: OracleConfig, cache_k, cache_v, positions):
    """One pre-norm decoder block on rows ``x`` ([n, dim]) at absolute ``positions``.

    Steps ([LLAMA3-ES], attention / multi-head / feed-forward bullets;
    [LLAMA3-NP], QKV, RoPE #2, KV cache, GQA):
    a = rmsnorm(x, attention_norm); q = a wq^T, k = a wk^T, v = a wv^T (separate
    projections; head h owns rows h*d..h*d+d-1 of wq); RoPE on q and k; k, v
    written into the cache at their positions; causal GQA attention over cache
    rows 0..max(positions); x += attn wo^T; b = rmsnorm(x, ffn_norm);
    x += feed_forward(b).  ``cache_k``/``cache_v`` ([capacity, G, d]) are updated
    in place.  Returns the new x.
    """
    n = x.shape[0]
    H, G, d = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    positions = np.asarray(positions, np.int64)
    a = rms_norm(x, lw["attention_norm"], cfg.norm_eps)
    q = (a @ lw["wq"].T).reshape(n, H, d)
    k = (a @ lw["wk"].T).reshape(n, G, d)
    v = (a @ lw["wv"].T).reshape(n, G, d)
    cos, sin = rope_cos_sin(positions, d, cfg.rope_theta)
    q = apply_rope(q, cos, sin)
    k = apply_rope(k, cos, sin)
    cache_k[positions] = k
    cache_v[positions] = v
    T = int(positions.max()) + 1
    o = causal_gqa_attention(q, cache_k[:T], cache_v[:T], positions)
    x = x + o @ lw["wo"].T
    b = rms_norm(x, lw["ffn_norm"], cfg.norm_eps)
    return x + feed_forward(b, lw["w1"], lw["w3"], lw["w2"])


def greedy_argmax(logits: np.ndarray) -> np.ndarray:
    """Index of the largest logit per row, lowest index on ties ([LLAMA3-ES], token prediction)."""
    logits = np.asarray(logits)
    if np.isnan(logits).any():
        raise ValueError("NaN logits")
    return np.argmax(logits, axis=-1)


class OracleModel:
    """Whole model: embedding, n_layers decoder blocks, final norm, output projection.

    ``weights`` maps the checkpoint names ([LLAMA3-SCRATCH], model-keys listing:
    ``tok_embeddings.weight``, ``layers.{i}.attention.{wq,wk,wv,wo}.weight``,
    ``layers.{i}.feed_forward.{w1,w3,w2}.weight``,
    ``layers.{i}.{attention_norm,ffn_norm}.weight``; plus ``norm.weight`` and
    ``output.weight``) to arrays shaped [out, in]; a linear is ``x @ W.T``.
    """

    def __init__(self, cfg: OracleConfig, weights: dict, dtype=np.float64):
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        cv = lambda a: np.asarray(a, self.dtype)  # noqa: E731
        self.emb = cv(weights["tok_embeddings.weight"])
        self.layers = []
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            self.layers.append({
                "attention_norm": cv(weights[p + "attention_norm.weight"]),
                "wq": cv(weights[p + "attention.wq.weight"]),
                "wk": cv(weights[p + "attention.wk.weight"]),
                "wv": cv(weights[p + "attention.wv.weight"]),
                "wo": cv(weights[p + "attention.wo.weight"]),
                "ffn_norm": cv(weights[p + "ffn_norm.weight"]),
                "w1": cv(weights[p + "feed_forward.w1.weight"]),
                "w3": cv(weights[p + "feed_forward.w3.weight"]),
                "w2": cv(weights[p + "feed_forward.w2.weight"]),
            })
        self.norm = cv(weights["norm.weight"])
        self.out = cv(weights["output.weight"])

    # -- state
    def new_cache(self, capacity: int | None = None):
        """Per-layer K and V stores [capacity, n_kv_heads, head_dim] ([LLAMA3-NP], KV cache)."""
        cap = capacity or self.cfg.max_seq_len
        shp = (cap, self.cfg.n_kv_heads, self.cfg.head_dim)
        return [(np.zeros(shp, self.dtype), np.zeros(shp, self.dtype)) for _ in range(self.cfg.n_layers)]

    # -- pieces
    def embed(self, tokens) -> np.ndarray:
        """Embedding lookup: row t of tok_embeddings ([LLAMA3-SCRATCH], embedding layer)."""
        return self.emb[np.asarray(tokens, np.int64)].copy()

    def layer(self, l: int, x, cache, positions):
        ck, cvv = cache[l]
        return decoder_layer(x, self.layers[l], self.cfg, ck, cvv, positions)

    def hidden(self, x, cache, positions):
        """All decoder blocks in turn ([LLAMA3-ES], repeat for every layer)."""
        for l in range(self.cfg.n_layers):
            x = self.layer(l, x, cache, positions)
        return x

    def logits_of(self, h) -> np.ndarray:
        """Final RMSNorm, then the output projection ([LLAMA3-ES], token prediction)."""
        y = rms_norm(np.atleast_2d(h), self.norm, self.cfg.norm_eps)
        return y @ self.out.T

    # -- phases ([LLAMA3-NP], Generasi: prefill over the whole input, then decode
    #    steps fed only the last token id; Linear: logits of the last row only)
    def prefill(self, tokens, cache=None, start_pos: int = 0):
        tokens = np.asarray(tokens)
        if cache is None:
            cache = self.new_cache()
        pos = np.arange(start_pos, start_pos + len(tokens))
        h = self.hidden(self.embed(tokens), cache, pos)
        return self.logits_of(h[-1:])[0], cache

    def decode(self, token: int, pos: int, cache):
        h = self.hidden(self.embed([token]), cache, np.array([pos]))
        return self.logits_of(h)[0]

    def forward_all_logits(self, tokens) -> np.ndarray:
        """Logits at every position by one causal pass over a fresh cache (full recompute)."""
        tokens = np.asarray(tokens)
        cache = self.new_cache(max(len(tokens), 1))
        h = self.hidden(self.embed(tokens), cache, np.arange(len(tokens)))
        return self.logits_of(h)

    def generate(self, prompt, steps: int):
        """Greedy generation: t0 = argmax(prefill(prompt)), then ``steps`` decode steps.

        Returns (tokens [steps+1], logits [steps+1, vocab]).
        """
        prompt = np.asarray(prompt)
        logits, cache = self.prefill(prompt)
        toks = [int(greedy_argmax(logits))]
        all_logits = [logits]
        for s in range(steps):
            logits = self.decode(toks[-1], len(prompt) + s, cache)
            all_logits.append(logits)
            toks.append(int(greedy_argmax(logits)))
        return np.array(toks), np.stack(all_logits)
