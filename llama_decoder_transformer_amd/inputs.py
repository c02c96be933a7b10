"""Seeded synthetic inputs for the Llama decoder workloads.

This module only draws numbers: model shapes, random-init weights, token ids,
input activations, KV-cache lengths and KV-cache contents.  It holds none of the
decoder's arithmetic, so both the HIP path and the CPU oracle can take their
inputs from it without sharing any computation.

Random streams.  Every tensor has its own NumPy ``PCG64`` stream keyed by
``[seed, stream_id, *sub_ids, block]`` so tensors can be drawn independently and in
parallel (one block = 2**22 consecutive elements).  Stream ids:

* ``tok_embeddings`` = 0; layer ``l``: ``1 + 7*l + k`` with k = 0 wq, 1 wk, 2 wv,
  3 wo, 4 w1, 5 w3, 6 w2 (the weight order printed in "Building llama3 from
  scratch", model-keys listing); ``output`` = ``1 + 7*n_layers``.
* token ids 1000, input activations 1001, KV lengths 1002, KV contents
  ``2000 + 2*l + (0 for K, 1 for V)`` with sub ids ``[sequence, kv_head]``.

Norm weights are constant 1.0 and draw nothing.  Matrices are ``std * N(0, 1)``
drawn in float32; bf16 tensors are the round-to-nearest-even of that float32
value and are handed out as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK = 1 << 22
WEIGHT_STD = 0.02


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass(frozen=True)
class ModelShape:
    """Hyper-parameters of a Llama decoder (the params.json field set plus F and max_seq_len)."""

    name: str
    dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    ffn_hidden_dim: int
    vocab_size: int
    max_seq_len: int
    rope_theta: float
    norm_eps: float
    dtype: str  # "f32" or "bf16": the storage type of every weight

    @property
    def head_dim(self) -> int:
        return self.dim // self.n_heads

    def replace(self, **kw) -> "ModelShape":
        d = dict(self.__dict__)
        d.update(kw)
        return ModelShape(**d)

    def weight_shapes(self) -> dict:
        """name -> shape for every weight tensor, rows = output features."""
        d, h, g, hd, f, v = (self.dim, self.n_heads, self.n_kv_heads, self.head_dim,
                             self.ffn_hidden_dim, self.vocab_size)
        out = {"tok_embeddings.weight": (v, d)}
        for l in range(self.n_layers):
            p = f"layers.{l}."
            out[p + "attention.wq.weight"] = (h * hd, d)
            out[p + "attention.wk.weight"] = (g * hd, d)
            out[p + "attention.wv.weight"] = (g * hd, d)
            out[p + "attention.wo.weight"] = (d, h * hd)
            out[p + "feed_forward.w1.weight"] = (f, d)
            out[p + "feed_forward.w3.weight"] = (f, d)
            out[p + "feed_forward.w2.weight"] = (d, f)
            out[p + "attention_norm.weight"] = (d,)
            out[p + "ffn_norm.weight"] = (d,)
        out["norm.weight"] = (d,)
        out["output.weight"] = (v, d)
        return out


# stories15M-sized Llama-2 shape (dim 288, 6 layers, 6 heads, vocab 32000, max_seq_len 256).
STORIES15M = ModelShape("stories15M", dim=288, n_layers=6, n_heads=6, n_kv_heads=6,
                        ffn_hidden_dim=768, vocab_size=32000, max_seq_len=256,
                        rope_theta=10000.0, norm_eps=1e-5, dtype="f32")
# Llama-3-8B shape (params.json values: dim 4096, 32 layers, 32 heads, 8 KV heads,
# vocab 128256, rope_theta 500000, eps 1e-5; FFN hidden 14336; context 8192).
LLAMA3_8B = ModelShape("llama3-8b", dim=4096, n_layers=32, n_heads=32, n_kv_heads=8,
                       ffn_hidden_dim=14336, vocab_size=128256, max_seq_len=8192,
                       rope_theta=500000.0, norm_eps=1e-5, dtype="bf16")


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a model shape and what is run on it."""

    key: str
    shape: ModelShape
    prompt_len: int = 0
    decode_steps: int = 0
    batch: int = 1
    kv_len_range: tuple = ()      # batched decode: cached lengths uniform in [lo, hi]
    layer_only: bool = False      # one decoder layer on N(0,1) bf16 activations
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "stories15m": Workload("stories15m", STORIES15M, prompt_len=8, decode_steps=50,
                           notes="fp32, prompt of 8 ids, prefill + 50 greedy decode steps"),
    "llama3-8b-layer": Workload("llama3-8b-layer", LLAMA3_8B.replace(n_layers=1),
                                prompt_len=2048, layer_only=True,
                                notes="one bf16 decoder layer, x ~ N(0,1) bf16 [2048, 4096]"),
    "llama3-8b": Workload("llama3-8b", LLAMA3_8B.replace(max_seq_len=768), prompt_len=512,
                          decode_steps=256,
                          notes="32 layers bf16, prompt 512 ids, 256 greedy KV-cached decode steps"),
    "llama3-8b-batched-decode": Workload("llama3-8b-batched-decode",
                                         LLAMA3_8B.replace(max_seq_len=8193), batch=64,
                                         kv_len_range=(1024, 8192),
                                         notes="64 sequences, cached lengths U{1024..8192}, "
                                               "cache ~ N(0,1) bf16, one decode step"),
    "llama3-8b-long-prefill": Workload("llama3-8b-long-prefill", LLAMA3_8B, prompt_len=8192,
                                       notes="32 layers bf16, prefill 8192 ids, last-position logits"),
}


# ----------------------------------------------------------------------------- numbers

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 values to bfloat16, returned as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _blocked(key: tuple, n: int, fill_block, out: np.ndarray) -> np.ndarray:
    nb = (n + BLOCK - 1) // BLOCK

    def work(b):
        lo = b * BLOCK
        hi = min(n, lo + BLOCK)
        g = np.random.default_rng(list(key) + [b])
        fill_block(g, out, lo, hi)

    if nb <= 1:
        for b in range(nb):
            work(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nb)))
    return out


def normal_f32(key: tuple, n: int, std: float) -> np.ndarray:
    """n draws of std * N(0,1) as float32 from the stream family ``key``."""
    out = np.empty(n, np.float32)

    def fill(g, o, lo, hi):
        g.standard_normal(hi - lo, dtype=np.float32, out=o[lo:hi])
        if std != 1.0:
            o[lo:hi] *= np.float32(std)

    return _blocked(key, n, fill, out)


def normal_bf16_bits(key: tuple, n: int, std: float) -> np.ndarray:
    """Same draws as :func:`normal_f32`, rounded to bfloat16 (uint16 bits)."""
    out = np.empty(n, np.uint16)

    def fill(g, o, lo, hi):
        t = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            t *= np.float32(std)
        o[lo:hi] = f32_to_bf16_bits(t)

    return _blocked(key, n, fill, out)


# ----------------------------------------------------------------------------- weights

_LAYER_SLOT = {"attention.wq.weight": 0, "attention.wk.weight": 1, "attention.wv.weight": 2,
               "attention.wo.weight": 3, "feed_forward.w1.weight": 4,
               "feed_forward.w3.weight": 5, "feed_forward.w2.weight": 6}


def weight_stream_id(shape: ModelShape, name: str) -> int | None:
    """Stream id of a weight, or None for the constant norm weights."""
    if name == "tok_embeddings.weight":
        return 0
    if name == "output.weight":
        return 1 + 7 * shape.n_layers
    if name.endswith("norm.weight"):
        return None
    _, l, rest = name.split(".", 2)
    return 1 + 7 * int(l) + _LAYER_SLOT[rest]


def weight(shape: ModelShape, name: str, seed: int = 0, as_bits: bool | None = None) -> np.ndarray:
    """One weight tensor.

    fp32 shapes give float32 values.  bf16 shapes give uint16 bits when
    ``as_bits`` (the default for bf16), else their exact float32 values.
    """
    shp = shape.weight_shapes()[name]
    n = int(np.prod(shp))
    bf16 = shape.dtype == "bf16"
    if as_bits is None:
        as_bits = bf16
    sid = weight_stream_id(shape, name)
    if sid is None:
        if bf16 and as_bits:
            return np.full(shp, 0x3F80, np.uint16)  # 1.0
        return np.ones(shp, np.float32)
    if bf16:
        bits = normal_bf16_bits((seed, sid), n, WEIGHT_STD).reshape(shp)
        return bits if as_bits else bf16_bits_to_f32(bits)
    if as_bits:
        raise ValueError("fp32 weights have no bf16 bit form")
    return normal_f32((seed, sid), n, WEIGHT_STD).reshape(shp)


def all_weights(shape: ModelShape, seed: int = 0, as_bits: bool | None = None) -> dict:
    return {name: weight(shape, name, seed, as_bits) for name in shape.weight_shapes()}


# ----------------------------------------------------------------------------- other inputs

def token_ids(vocab_size: int, n: int, seed: int = 0, sub: int = 0) -> np.ndarray:
    """n token ids uniform in [0, vocab_size)."""
    g = np.random.default_rng([seed, 1000, sub])
    return g.integers(0, vocab_size, size=n).astype(np.int32)


def activations_bf16_bits(rows: int, dim: int, seed: int = 0) -> np.ndarray:
    """Residual-stream input ~ N(0,1) rounded to bf16 (uint16 bits), shape [rows, dim]."""
    return normal_bf16_bits((seed, 1001), rows * dim, 1.0).reshape(rows, dim)


def kv_lengths(batch: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Cached lengths uniform over the integers lo..hi inclusive."""
    g = np.random.default_rng([seed, 1002])
    return g.integers(lo, hi + 1, size=batch).astype(np.int32)


def kv_contents_bf16_bits(layer: int, which: int, seq: int, kv_head: int, length: int,
                          head_dim: int, seed: int = 0) -> np.ndarray:
    """Cache contents ~ N(0,1) bf16 for one (layer, K or V, sequence, kv head): [length, head_dim]."""
    key = (seed, 2000 + 2 * layer + which, seq, kv_head)
    return normal_bf16_bits(key, length * head_dim, 1.0).reshape(length, head_dim)
