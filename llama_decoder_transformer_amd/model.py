"""A model instance on one GPU: torch allocates the buffers, the HIP library computes.

``LlamaModel`` owns the packed weights, the KV cache and the workspace as torch
uint8 tensors and forwards every computation to the C ABI through
``binding``.  Weights are given as a dict of device tensors keyed by the
checkpoint names (``tok_embeddings.weight``, ``layers.{i}.attention.wq.weight``,
...), float32 or bfloat16.
"""
from __future__ import annotations

import ctypes

import torch

from . import binding as B


def make_config(shape, max_batch: int = 1, max_prefill_tokens: int = 1) -> B.llm_config:
    """llm_config from any object with the ModelShape fields."""
    return B.llm_config(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                        n_kv_heads=shape.n_kv_heads, vocab_size=shape.vocab_size,
                        max_seq_len=shape.max_seq_len, ffn_hidden_dim=shape.ffn_hidden_dim,
                        rope_theta=float(shape.rope_theta), norm_eps=float(shape.norm_eps),
                        dtype=B.LLM_BF16 if shape.dtype == "bf16" else B.LLM_F32,
                        max_batch=max_batch, max_prefill_tokens=max_prefill_tokens)


class LlamaModel:
    def __init__(self, shape, weights: dict, max_batch: int = 1, max_prefill_tokens: int = 1,
                 device="cuda:0", stream=None):
        self.shape = shape
        self.device = torch.device(device)
        self.cfg = make_config(shape, max_batch, max_prefill_tokens)
        B.llm_check_config(self.cfg)
        self.torch_dtype = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        u8 = dict(dtype=torch.uint8, device=self.device)
        self.packed = torch.empty(B.llm_packed_weight_bytes(self.cfg), **u8)
        self.kv = torch.empty(B.llm_kv_cache_bytes(self.cfg), **u8)
        self.workspace = torch.empty(B.llm_workspace_bytes(self.cfg), **u8)
        L = shape.n_layers

        def ptr(name):
            t = weights[name]
            assert t.device == self.device and t.dtype == self.torch_dtype and t.is_contiguous(), name
            return t.data_ptr()

        def arr(fmt):
            return (ctypes.c_void_p * L)(*[ptr(fmt.format(l)) for l in range(L)])

        self._arrays = dict(
            attention_norm=arr("layers.{}.attention_norm.weight"), wq=arr("layers.{}.attention.wq.weight"),
            wk=arr("layers.{}.attention.wk.weight"), wv=arr("layers.{}.attention.wv.weight"),
            wo=arr("layers.{}.attention.wo.weight"), ffn_norm=arr("layers.{}.ffn_norm.weight"),
            w1=arr("layers.{}.feed_forward.w1.weight"), w3=arr("layers.{}.feed_forward.w3.weight"),
            w2=arr("layers.{}.feed_forward.w2.weight"))
        pp = lambda a: ctypes.cast(a, B.PP)  # noqa: E731
        w = B.llm_weights(tok_embeddings=ptr("tok_embeddings.weight"), norm=ptr("norm.weight"),
                          output=ptr("output.weight"),
                          **{k: pp(v) for k, v in self._arrays.items()})
        self.handle = B.llm_init_weights(self.cfg, w, self.packed, self.kv, self.workspace, stream)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            B.llm_free(h)
            self.handle = None

    # ------------------------------------------------------------------ views
    @property
    def cache_dtype(self) -> torch.dtype:
        """Element type of the KV cache: fp16 for bf16-weight models (their compute type), else fp32."""
        return torch.float16 if self.shape.dtype == "bf16" else torch.float32

    def kv_cache_view(self) -> torch.Tensor:
        """[n_layers, 2 (K, V), max_batch, n_kv_heads, max_seq_len, head_dim] view of the cache."""
        s = self.shape
        return self.kv.view(self.cache_dtype).view(s.n_layers, 2, self.cfg.max_batch, s.n_kv_heads,
                                                   s.max_seq_len, s.dim // s.n_heads)

    # ------------------------------------------------------------------ calls
    def prefill(self, tokens: torch.Tensor, slot: int = 0, start_pos: int = 0, logits=None, stream=None):
        n = tokens.numel()
        if logits is None:
            logits = torch.empty(self.shape.vocab_size, dtype=torch.float32, device=self.device)
        B.llm_prefill(self.handle, slot, tokens, n, start_pos, logits, stream)
        return logits

    def prefill_batch(self, tokens: torch.Tensor, slots, starts, lens, logits=None, stream=None):
        """Several prompts at once: tokens holds them back to back; returns [batch, vocab] last-position logits."""
        if logits is None:
            logits = torch.empty(len(lens), self.shape.vocab_size, dtype=torch.float32, device=self.device)
        B.llm_prefill_batch(self.handle, slots, starts, lens, tokens, logits, stream)
        return logits

    def layer_forward(self, layer: int, x: torch.Tensor, slot: int = 0, start_pos: int = 0, stream=None):
        B.llm_layer_forward(self.handle, layer, slot, x, x.shape[0], start_pos, stream)
        return x

    def decode_step(self, slots, positions, tokens, logits=None, stream=None):
        b = tokens.numel()
        if logits is None:
            logits = torch.empty(b, self.shape.vocab_size, dtype=torch.float32, device=self.device)
        B.llm_decode_step(self.handle, b, slots, positions, tokens, logits, stream)
        return logits

    def argmax(self, logits: torch.Tensor, out=None, stream=None):
        rows = 1 if logits.dim() == 1 else logits.shape[0]
        if out is None:
            out = torch.empty(rows, dtype=torch.int32, device=self.device)
        B.llm_argmax(logits, rows, logits.shape[-1], out, stream)
        return out

    def generate(self, slots, positions, tokens, n_steps: int, logits=None, stream=None):
        b = tokens.numel()
        out = torch.empty(n_steps, b, dtype=torch.int32, device=self.device)
        if logits is None:
            logits = torch.empty(b, self.shape.vocab_size, dtype=torch.float32, device=self.device)
        B.llm_generate(self.handle, b, slots, positions, tokens, n_steps, out, logits, stream)
        return out, logits

    def read_device_error(self, stream=None) -> int:
        return B.llm_read_device_error(self.handle, stream)
