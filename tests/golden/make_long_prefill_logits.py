"""Write the oracle's last-position logits for the 8192-token Llama-3-8B prefill.

Expected values for the long-context prefill parity test: the CPU oracle (``oracle/``
only, numpy float32 matmuls, float64 norms and softmax) runs the seeded
Llama-3-8B-shaped model (32 layers, bf16 random-init weights, seed 0) over the
seeded prompt of 8192 token ids and stores the logits of the last position
("Linear" section of "Model Llama 3 yang Diimplementasikan dengan NumPy Murni":
only the last row is projected to the vocabulary; 8192 is the context length in
the Llama 3 vs Llama 2 table of "Building llama3 from scratch").

The layers are run one at a time with each layer's weights drawn just before it
is needed, so the run holds one layer of float32 weights (about 0.9 GB) plus the
[8192, 4096] residual stream.  It takes tens of minutes on a few CPU cores.

Usage: python tests/golden/make_long_prefill_logits.py
Output: tests/golden/llama3_8b_prefill8192_last_logits.npy (float32 [128256])
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from llama_decoder_transformer_amd import inputs  # noqa: E402  (seeded numbers only)
from oracle import OracleConfig, decoder_layer, rms_norm  # noqa: E402

OUT = os.path.join(HERE, "llama3_8b_prefill8192_last_logits.npy")


def main() -> int:
    wl = inputs.WORKLOADS["llama3-8b-long-prefill"]
    shape = wl.shape
    S = wl.prompt_len
    cfg = OracleConfig(dim=shape.dim, n_layers=shape.n_layers, n_heads=shape.n_heads,
                       n_kv_heads=shape.n_kv_heads, vocab_size=shape.vocab_size,
                       ffn_hidden_dim=shape.ffn_hidden_dim, max_seq_len=shape.max_seq_len,
                       rope_theta=shape.rope_theta, norm_eps=shape.norm_eps)
    prompt = inputs.token_ids(shape.vocab_size, S)

    def w(name):
        return inputs.weight(shape, name, as_bits=False)

    t0 = time.time()
    x = w("tok_embeddings.weight")[prompt.astype(np.int64)].copy()
    pos = np.arange(S)
    for l in range(shape.n_layers):
        p = f"layers.{l}."
        lw = {"attention_norm": w(p + "attention_norm.weight"), "wq": w(p + "attention.wq.weight"),
              "wk": w(p + "attention.wk.weight"), "wv": w(p + "attention.wv.weight"),
              "wo": w(p + "attention.wo.weight"), "ffn_norm": w(p + "ffn_norm.weight"),
              "w1": w(p + "feed_forward.w1.weight"), "w3": w(p + "feed_forward.w3.weight"),
              "w2": w(p + "feed_forward.w2.weight")}
        ck = np.zeros((S, shape.n_kv_heads, shape.head_dim), np.float32)
        cv = np.zeros_like(ck)
        x = decoder_layer(x, lw, cfg, ck, cv, pos)
        print(f"layer {l} done at {time.time() - t0:.0f}s", flush=True)
    y = rms_norm(x[-1:], w("norm.weight"), cfg.norm_eps)
    logits = (y @ w("output.weight").T)[0].astype(np.float32)
    np.save(OUT, logits)
    print(f"wrote {OUT}: argmax {int(np.argmax(logits))}, max |logit| {float(np.max(np.abs(logits))):.4f}, "
          f"{time.time() - t0:.0f}s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
