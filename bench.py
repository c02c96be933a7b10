#!/usr/bin/env python3
"""Throughput of the Llama decoder pass on one MI355X.

Default workload: the Llama-3-8B shape (32 layers, dim 4096, 32 query / 8 KV
heads, FFN 14336, vocab 128256, bf16 random-init weights ~ N(0, 0.02)), batch 1,
a prompt of 512 token ids uniform in [0, 128256), prefill, then 256 greedy
KV-cached decode steps.  One step = that whole job; the JSON line reports
tokens/s over it plus prefill tok/s and decode tok/s separately.

Per-kernel durations come from the library's own hipEvent brackets (one
extra, untimed step run with kernel timing on); the roofline object is for the
dominant kernel (the decode gate-up projection, HBM-bound), with the prefill
gate-up GEMM (MFMA-bound) reported next to it.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload and scales it to the full job.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def make_weights(shape, keep_layers: int):
    """Device bf16 weights for every tensor; host float32 copies of a few layers for the CPU sample."""
    import torch

    from llama_decoder_transformer_amd import inputs

    dev, host = {}, {}
    for name in shape.weight_shapes():
        bits = inputs.weight(shape, name)
        dev[name] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        layer = int(name.split(".")[1]) if name.startswith("layers.") else -1
        if layer < keep_layers:
            host[name] = inputs.bf16_bits_to_f32(bits)
    return dev, host


def cpu_baseline(shape, host_w, prompt, n_layers_sample: int, decode_sample: int, decode_steps: int):
    """The oracle (fp32 matmuls) on n_layers_sample of the layers, scaled to the whole model."""
    from oracle import OracleConfig, OracleModel

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    cfg = OracleConfig(dim=shape.dim, n_layers=n_layers_sample, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                       vocab_size=shape.vocab_size, ffn_hidden_dim=shape.ffn_hidden_dim,
                       max_seq_len=shape.max_seq_len, rope_theta=shape.rope_theta, norm_eps=shape.norm_eps)
    om = OracleModel(cfg, host_w, dtype=np.float32)
    cache = om.new_cache()
    n = len(prompt)
    t0 = time.perf_counter()
    h = om.hidden(om.embed(prompt), cache, np.arange(n))
    t1 = time.perf_counter()
    logits = om.logits_of(h[-1:])[0]
    t2 = time.perf_counter()
    tok = int(np.argmax(logits))
    t_dec_layers = 0.0
    t_dec_head = 0.0
    for s in range(decode_sample):
        a = time.perf_counter()
        hd = om.hidden(om.embed([tok]), cache, np.array([n + s]))
        b = time.perf_counter()
        lg = om.logits_of(hd)[0]
        c = time.perf_counter()
        tok = int(np.argmax(lg))
        t_dec_layers += b - a
        t_dec_head += c - b
    scale = shape.n_layers / n_layers_sample
    t_prefill = (t1 - t0) * scale + (t2 - t1)
    t_decode_step = (t_dec_layers * scale + t_dec_head) / decode_sample
    total = t_prefill + decode_steps * t_decode_step
    return {
        "value": round((n + decode_steps) / total, 3),
        "unit": "tok/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"oracle (numpy fp32 matmuls, fp64 norms/softmax) on {n_layers_sample} of {shape.n_layers} layers: "
                   f"prefill of the {n}-token prompt + {decode_sample} decode steps, plus the LM head; layer time "
                   f"scaled by {scale:g} to the full model and decode time by {decode_steps}/{decode_sample}"),
        "prefill_tok_s": round(n / t_prefill, 3),
        "decode_tok_s": round(1.0 / t_decode_step, 4),
        "sample_seconds": round(t2 - t0 + t_dec_layers + t_dec_head, 2),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=4, help="layers in the CPU oracle sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch

    from llama_decoder_transformer_amd import binding as B
    from llama_decoder_transformer_amd import inputs
    from llama_decoder_transformer_amd.model import LlamaModel

    wl = inputs.WORKLOADS["llama3-8b"]
    shape = wl.shape
    P, T = wl.prompt_len, wl.decode_steps
    dev = "cuda:0"
    t0 = time.perf_counter()
    dw, host_w = make_weights(shape, 0 if args.no_cpu_baseline else args.cpu_layers)
    log(f"weights generated and uploaded in {time.perf_counter() - t0:.1f}s")
    model = LlamaModel(shape, dw, max_batch=1, max_prefill_tokens=P, device=dev)
    del dw
    torch.cuda.empty_cache()
    log("model initialised")

    prompt_np = inputs.token_ids(shape.vocab_size, P)
    prompt = torch.as_tensor(prompt_np, device=dev)
    slots = torch.zeros(1, dtype=torch.int32, device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    tok = torch.zeros(1, dtype=torch.int32, device=dev)
    logits1 = torch.empty(shape.vocab_size, dtype=torch.float32, device=dev)
    logitsB = torch.empty(1, shape.vocab_size, dtype=torch.float32, device=dev)
    out = torch.empty(T, 1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    h = model.handle

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        B.llm_prefill(h, 0, prompt, P, 0, logits1, stream)
        B.llm_argmax(logits1, 1, shape.vocab_size, tok, stream)
        if ev:
            ev[1].record(stream)
        pos.fill_(P)
        B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    prefill_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    assert model.read_device_error() == 0
    gen_tokens = out[:, 0].cpu().tolist()
    log(f"timed {args.steps} steps in {wall:.3f}s: prefill {prefill_ms:.3f} ms, decode {decode_ms / T:.3f} ms/token")

    # Per-kernel durations: one prefill and one decode block with the library's event brackets.
    def timed_groups(fn):
        B.llm_set_kernel_timing(h, True)
        fn()
        res = {name: B.llm_kernel_timing(h, k) for k, name in enumerate(B.KERNEL_GROUPS)}
        B.llm_set_kernel_timing(h, False)
        return res

    kt_prefill = timed_groups(lambda: B.llm_prefill(h, 0, prompt, P, 0, logits1, stream))
    torch.cuda.synchronize()
    pos.fill_(P)

    def dec():
        B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream)

    kt_decode = timed_groups(dec)
    torch.cuda.synchronize()

    L, dim, F, V = shape.n_layers, shape.dim, shape.ffn_hidden_dim, shape.vocab_size
    n_up, ms_up = kt_decode["gate_up"]
    up_avg_ms = ms_up / n_up
    up_bytes = 2 * F * dim * 2 + 2 * dim * 4 + F * 2  # w1|w3 weights + fp32 x and norm weight in + SwiGLU row out
    up_gbs = up_bytes / (up_avg_ms * 1e-3) / 1e9
    n_pup, ms_pup = kt_prefill["gate_up"]
    pup_avg_ms = ms_pup / n_pup
    pup_flops = 2.0 * P * (2 * F) * dim
    pup_tflops = pup_flops / (pup_avg_ms * 1e-3) / 1e12

    per_kernel = {}
    for name in B.KERNEL_GROUPS:
        n1, m1 = kt_prefill[name]
        n2, m2 = kt_decode[name]
        per_kernel[name] = {"prefill_launches": n1, "prefill_avg_us": round(m1 / n1 * 1e3, 2) if n1 else None,
                            "decode_launches": n2, "decode_avg_us": round(m2 / n2 * 1e3, 2) if n2 else None}

    # Whole-step HBM bytes of one decode token (weights except the embedding table, + KV read/write).
    hd = dim // shape.n_heads
    kv_pos_bytes = L * shape.n_kv_heads * hd * 2 * 2
    w_bytes = 2 * (L * (dim * (shape.n_heads + 2 * shape.n_kv_heads) * hd + dim * shape.n_heads * hd
                        + 3 * F * dim) + V * dim)
    mean_ctx = P + (T - 1) / 2.0 + 1
    dec_bytes = w_bytes + kv_pos_bytes * mean_ctx
    decode_tok_s = T / (decode_ms * 1e-3)
    prefill_tok_s = P / (prefill_ms * 1e-3)
    value = (P + T) * args.steps / wall

    res = {
        "metric": "prefill tok/s + decode tok/s at Llama-3-8B shape, % of MFMA/HBM roofline",
        "value": round(value, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b: 32-layer Llama-3-8B-shaped bf16 model, batch 1, prefill of 512 ids "
                               "then 256 greedy KV-cached decode steps",
                   "prompt_len": P, "decode_steps": T, "batch": 1, "parallelism": "none (1 GPU)"},
        "prefill_tok_s": round(prefill_tok_s, 1),
        "decode_tok_s": round(decode_tok_s, 2),
        "prefill_ms": round(prefill_ms, 3),
        "decode_ms_per_token": round(decode_ms / T, 4),
        "decode_step_hbm_frac": round(dec_bytes / (decode_ms / T * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"kernel": "decode gate-up projection (w1|w3 GEMV + SwiGLU), M=1", "bound": "hbm",
                     "achieved": round(up_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(up_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": up_bytes, "avg_launch_us": round(up_avg_ms * 1e3, 2)},
        "roofline_prefill": {"kernel": "prefill gate-up GEMM (M=512, N=28672, K=4096) + SwiGLU", "bound": "mfma",
                             "achieved": round(pup_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(pup_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_per_launch": pup_flops, "avg_launch_us": round(pup_avg_ms * 1e3, 2)},
        "per_kernel": per_kernel,
        "generated_first_tokens": gen_tokens[:8],
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        res["cpu_baseline"] = cpu_baseline(shape, host_w, prompt_np, args.cpu_layers, 4, T)
        log(f"cpu baseline took {time.perf_counter() - t0:.1f}s")
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
