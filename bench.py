#!/usr/bin/env python3
"""Throughput of the Llama decoder pass on one MI355X.

Headline workload (``llama3-8b``): the Llama-3-8B shape (32 layers, dim 4096,
32 query / 8 KV heads, FFN 14336, vocab 128256, bf16 random-init weights
~ N(0, 0.02)), batch 1, a prompt of 512 token ids uniform in [0, 128256),
prefill, then 256 greedy KV-cached decode steps replayed from the library's HIP
graph.  One step = that whole job; the JSON line reports tokens/s over it plus
prefill tok/s and decode tok/s separately.

The default run (``--workload all``) prints that headline line and adds, under
``workloads``, one entry per other workload, each with its own steps, timing,
``roofline`` and ``cpu_baseline``:
  stories15m                fp32 stories15M shape: prefill of 8 ids + 50 greedy decode steps
                            (latency / launch bound: us per step and kernels per step)
  llama3-8b-layer           one 8B-shaped layer on x ~ N(0,1) [2048, 4096] (prefill tok/s)
  llama3-8b-long-prefill    prefill of 8192 ids, last-position logits (prefill tok/s)
  llama3-8b-batched-decode  one decode step of 64 sequences, cached lengths U{1024..8192},
                            N(0,1) caches (decode tok/s)
``--workload NAME`` runs one of them alone as the line's headline.

Per-kernel durations come from the library's own hipEvent brackets (one extra,
untimed pass with kernel timing on); ``roofline`` is for the workload's dominant
kernel.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload and scales it to the full job.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all] [--no-cpu-baseline]
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
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16
METRIC = "prefill tok/s + decode tok/s at Llama-3-8B shape, % of MFMA/HBM roofline"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def make_weights(shape, keep_layers: int, keep_head: bool = True):
    """Device bf16 weights for every tensor; host float32 copies of the first layers for the CPU sample."""
    import torch

    from llama_decoder_transformer_amd import inputs

    dev, host = {}, {}
    for name in shape.weight_shapes():
        bits = inputs.weight(shape, name)
        dev[name] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
        layer = int(name.split(".")[1]) if name.startswith("layers.") else -1
        if (layer >= 0 and layer < keep_layers) or (layer < 0 and keep_head):
            host[name] = inputs.bf16_bits_to_f32(bits)
    return dev, host


def oracle_cfg(shape, n_layers: int):
    from oracle import OracleConfig
    return OracleConfig(dim=shape.dim, n_layers=n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                        vocab_size=shape.vocab_size, ffn_hidden_dim=shape.ffn_hidden_dim,
                        max_seq_len=shape.max_seq_len, rope_theta=shape.rope_theta, norm_eps=shape.norm_eps)


def timed_groups(B, h, fn):
    """Run fn with the library's kernel brackets on; return {group: (launches, total_ms)}."""
    B.llm_set_kernel_timing(h, True)
    fn()
    res = {name: B.llm_kernel_timing(h, k) for k, name in enumerate(B.KERNEL_GROUPS)}
    B.llm_set_kernel_timing(h, False)
    return res


def per_kernel_table(groups: dict, label: str) -> dict:
    return {name: {f"{label}_launches": n, f"{label}_avg_us": round(ms / n * 1e3, 2) if n else None}
            for name, (n, ms) in groups.items() if n}


def avg_ms(groups: dict, name: str) -> float:
    n, ms = groups[name]
    return ms / n


def mfma_roofline(kernel: str, flops: float, ms: float) -> dict:
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_PEAK_TFLOPS, 4), "traffic": None, "flops_per_launch": flops,
            "avg_launch_us": round(ms * 1e3, 2)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_fingerprint(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    scaled by the copy-probe factors; None when absent or when the kernel's sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            entry = json.load(f)[key]
        if source_fingerprint(entry["sources"]) != entry["sha256"]:
            return None
        return int(entry["bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def hbm_roofline(kernel: str, nbytes: float, ms: float, traffic=None) -> dict:
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": int(nbytes),
            "avg_launch_us": round(ms * 1e3, 2)}


def layer_flops(shape, S: int) -> tuple[float, float]:
    """(linear, causal attention) flops of one layer over S positions starting at 0."""
    d, H, G, F, hd = shape.dim, shape.n_heads, shape.n_kv_heads, shape.ffn_hidden_dim, shape.head_dim
    lin = 2.0 * S * (d * (H + 2 * G) * hd + H * hd * d + 3 * F * d)
    att = 4.0 * H * hd * S * (S + 1) / 2
    return lin, att


def time_steps(torch, step, steps: int, warmup: int):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


# ----------------------------------------------------------------------------- workloads

def shared_8b_weights(args, inputs, shared):
    """Device bf16 weights of the 32-layer Llama-3-8B shape and host copies of the first
    layers, generated once and shared by the 8B workloads of one run."""
    if "dw" not in shared:
        shape = inputs.LLAMA3_8B if not args.layers else inputs.LLAMA3_8B.replace(n_layers=args.layers)
        t0 = time.perf_counter()
        keep = 0 if args.no_cpu_baseline else min(args.cpu_layers, shape.n_layers)
        shared["dw"], shared["host"] = make_weights(shape, keep, keep_head=not args.no_cpu_baseline)
        log(f"8B weights generated and uploaded in {time.perf_counter() - t0:.1f}s")
    return shared["dw"], shared["host"]


def release(torch):
    """Return the memory of models the caller has just deleted."""
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bench_generate(args, torch, B, inputs, LlamaModel, shared, steps: int, warmup: int) -> dict:
    wl = inputs.WORKLOADS["llama3-8b"]
    shape = wl.shape if not args.layers else wl.shape.replace(n_layers=args.layers)
    P, T = wl.prompt_len, wl.decode_steps
    dev = "cuda:0"
    dw, host_w = shared_8b_weights(args, inputs, shared)
    model = LlamaModel(shape, dw, max_batch=1, max_prefill_tokens=P, device=dev)

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
    evs = []

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        B.llm_prefill(h, 0, prompt, P, 0, logits1, stream)
        B.llm_argmax(logits1, 1, shape.vocab_size, tok, stream)
        ev[1].record(stream)
        pos.fill_(P)
        B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream)
        ev[2].record(stream)
        evs.append(ev)

    wall = time_steps(torch, step, steps, warmup)
    evs = evs[warmup:]
    prefill_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    assert model.read_device_error() == 0
    log(f"llama3-8b: timed {steps} steps in {wall:.3f}s: prefill {prefill_ms:.3f} ms, decode {decode_ms / T:.3f} "
        f"ms/token")

    kt_prefill = timed_groups(B, h, lambda: B.llm_prefill(h, 0, prompt, P, 0, logits1, stream))
    torch.cuda.synchronize()
    pos.fill_(P)
    kt_decode = timed_groups(B, h, lambda: B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream))
    torch.cuda.synchronize()
    first_tokens = out[:8, 0].cpu().tolist()
    del model
    release(torch)

    L, dim, F, V = shape.n_layers, shape.dim, shape.ffn_hidden_dim, shape.vocab_size
    up_bytes = 2 * F * dim * 2 + 2 * dim * 4 + F * 2  # w1|w3 weights + fp32 x and norm weight in + SwiGLU row out
    hd, H, G = shape.head_dim, shape.n_heads, shape.n_kv_heads
    # one decode-block launch (q|k|v GEMV + attention + wo GEMV of a layer): the q|k|v and wo weights
    # (fp16), the layer's cached keys and values at the mean decode context (fp16), x read twice and
    # written once plus the norm weight (fp32)
    mean_ctx_blk = P + (T - 1) / 2.0 + 1
    blk_bytes = 2 * (dim * (H + 2 * G) * hd + H * hd * dim) + G * hd * 2 * 2 * mean_ctx_blk + 4 * dim * 4
    per_kernel = per_kernel_table(kt_prefill, "prefill")
    for k, v in per_kernel_table(kt_decode, "decode").items():
        per_kernel.setdefault(k, {}).update(v)
    hd = shape.head_dim
    kv_pos_bytes = L * shape.n_kv_heads * hd * 2 * 2
    w_bytes = 2 * (L * (dim * (shape.n_heads + 2 * shape.n_kv_heads) * hd + dim * shape.n_heads * hd + 3 * F * dim)
                   + V * dim)
    mean_ctx = P + (T - 1) / 2.0 + 1
    dec_bytes = w_bytes + kv_pos_bytes * mean_ctx
    res = {
        "value": round((P + T) * steps / wall, 3), "unit": "tok/s", "ms_per_step": round(wall / steps * 1e3, 3),
        "config": {"workload": "llama3-8b: 32-layer Llama-3-8B-shaped bf16 model, batch 1, prefill of 512 ids "
                               "then 256 greedy KV-cached decode steps",
                   "prompt_len": P, "decode_steps": T, "batch": 1, "parallelism": "none (1 GPU)"},
        "prefill_tok_s": round(P / (prefill_ms * 1e-3), 1),
        "decode_tok_s": round(T / (decode_ms * 1e-3), 2),
        "prefill_ms": round(prefill_ms, 3),
        "decode_ms_per_token": round(decode_ms / T, 4),
        "decode_step_hbm_frac": round(dec_bytes / (decode_ms / T * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": hbm_roofline("decode gate-up projection (w1|w3 GEMV + fused RMSNorm + SwiGLU), M=1", up_bytes,
                                 avg_ms(kt_decode, "gate_up"), measured_traffic("decode_gate_up_gemv")),
        "roofline_decode_block": hbm_roofline("decode block: q|k|v GEMV + attention + wo GEMV of one layer, M=1",
                                              blk_bytes, avg_ms(kt_decode, "decode_block"),
                                              measured_traffic("decode_block")),
        "roofline_prefill": mfma_roofline("prefill gate-up GEMM (M=512, N=28672, K=4096) + SwiGLU",
                                          2.0 * P * (2 * F) * dim, avg_ms(kt_prefill, "gate_up")),
        "per_kernel": per_kernel,
        "generated_first_tokens": first_tokens,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_generate(shape, host_w, prompt_np, args.cpu_layers, args.cpu_decode_steps, T)
    return res


def cpu_generate(shape, host_w, prompt, n_layers_sample: int, decode_sample: int, decode_steps: int) -> dict:
    from oracle import OracleModel
    om = OracleModel(oracle_cfg(shape, n_layers_sample), host_w, dtype=np.float32)
    cache = om.new_cache()
    n = len(prompt)
    t0 = time.perf_counter()
    h = om.hidden(om.embed(prompt), cache, np.arange(n))
    t1 = time.perf_counter()
    logits = om.logits_of(h[-1:])[0]
    t2 = time.perf_counter()
    tok = int(np.argmax(logits))
    t_layers = t_head = 0.0
    for s in range(decode_sample):
        a = time.perf_counter()
        hd = om.hidden(om.embed([tok]), cache, np.array([n + s]))
        b = time.perf_counter()
        lg = om.logits_of(hd)[0]
        c = time.perf_counter()
        tok = int(np.argmax(lg))
        t_layers += b - a
        t_head += c - b
    scale = shape.n_layers / n_layers_sample
    t_prefill = (t1 - t0) * scale + (t2 - t1)
    t_step = (t_layers * scale + t_head) / decode_sample
    total = t_prefill + decode_steps * t_step
    return {"value": round((n + decode_steps) / total, 3), "unit": "tok/s", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"oracle (numpy fp32 matmuls, fp64 norms/softmax) on {n_layers_sample} of {shape.n_layers} "
                       f"layers: prefill of the {n}-token prompt + {decode_sample} decode steps, plus the LM head; "
                       f"layer time scaled by {scale:g} and decode time by {decode_steps}/{decode_sample}"),
            "prefill_tok_s": round(n / t_prefill, 3), "decode_tok_s": round(1.0 / t_step, 4),
            "sample_seconds": round(t2 - t0 + t_layers + t_head, 2)}


def bench_stories(args, torch, B, inputs, LlamaModel, shared, steps: int, warmup: int) -> dict:
    """stories15M fp32: prefill of 8 ids, then 50 greedy decode steps replayed from the graph.  The
    97.6 MB model sits in the 256 MB memory-side cache, so the job is bound by latency and kernel
    launches: the entry reports us per decode step and kernels per step; its HBM figure is context."""
    wl = inputs.WORKLOADS["stories15m"]
    shape = wl.shape
    P, T = wl.prompt_len, wl.decode_steps
    dev = "cuda:0"
    hw = inputs.all_weights(shape)
    model = LlamaModel(shape, {k: torch.from_numpy(v).to(dev) for k, v in hw.items()}, max_batch=1,
                       max_prefill_tokens=P, device=dev)
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
    evs = []

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        B.llm_prefill(h, 0, prompt, P, 0, logits1, stream)
        B.llm_argmax(logits1, 1, shape.vocab_size, tok, stream)
        ev[1].record(stream)
        pos.fill_(P)
        B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream)
        ev[2].record(stream)
        evs.append(ev)

    wall = time_steps(torch, step, steps, warmup)
    evs = evs[warmup:]
    prefill_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    decode_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    assert model.read_device_error() == 0
    # One more job with the kernel brackets on around the decode steps (direct launches).
    B.llm_prefill(h, 0, prompt, P, 0, logits1, stream)
    B.llm_argmax(logits1, 1, shape.vocab_size, tok, stream)
    t0_gpu = int(tok.item())
    pos.fill_(P)
    B.llm_set_kernel_timing(h, True)
    B.llm_generate(h, 1, slots, pos, tok, T, out, logitsB, stream)
    groups = {name: B.llm_kernel_timing_full(h, k) for k, name in enumerate(B.KERNEL_GROUPS)}
    B.llm_set_kernel_timing(h, False)
    torch.cuda.synchronize()
    gpu_tokens = [t0_gpu] + out[:, 0].cpu().tolist()
    del model
    release(torch)
    kernels_per_step = sum(k for _, k, _ in groups.values()) / T
    kernel_us_per_step = sum(ms for _, _, ms in groups.values()) * 1e3 / T
    L, dim, F, V = shape.n_layers, shape.dim, shape.ffn_hidden_dim, shape.vocab_size
    hd = shape.head_dim
    w_bytes = 4 * (L * (dim * (shape.n_heads + 2 * shape.n_kv_heads) * hd + dim * shape.n_heads * hd + 3 * F * dim)
                   + V * dim)
    us_step = decode_ms / T * 1e3
    res = {"value": round((P + T) * steps / wall, 1), "unit": "tok/s", "ms_per_step": round(wall / steps * 1e3, 3),
           "steps": steps, "warmup": warmup, "dtype": "f32",
           "config": {"workload": "stories15m: stories15M-shaped fp32 Llama (dim 288, 6 layers, 6 heads, vocab "
                                  "32000), batch 1, prefill of 8 ids then 50 greedy KV-cached decode steps",
                      "prompt_len": P, "decode_steps": T, "batch": 1},
           "prefill_us": round(prefill_ms * 1e3, 1), "us_per_decode_step": round(us_step, 2),
           "kernels_per_decode_step": round(kernels_per_step, 2),
           "kernel_us_per_decode_step": round(kernel_us_per_step, 2),
           "roofline": dict(hbm_roofline("whole decode step (latency / launch bound: the weights sit in the "
                                         "memory-side cache; HBM figure is context only)", w_bytes, us_step * 1e-3),
                            bound_note="latency"),
           "generated_tokens": gpu_tokens[:8]}
    if not args.no_cpu_baseline:
        from oracle import OracleModel
        om = OracleModel(oracle_cfg(shape, shape.n_layers), hw, dtype=np.float64)
        times, toks = [], None
        while len(times) < 20 and sum(times) < 5.0:
            t0 = time.perf_counter()
            toks, _ = om.generate(prompt_np, T)
            times.append(time.perf_counter() - t0)
        t = float(np.mean(times))
        res["cpu_baseline"] = {"value": round((P + T) / t, 2), "unit": "tok/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": (f"the whole workload: oracle (numpy fp64) prefill of the 8 ids and 50 "
                                          f"greedy decode steps, mean of {len(times)} passes"),
                               "us_per_decode_step": round(t / (T + 1) * 1e6, 1),
                               "sample_seconds": round(sum(times), 2)}
        res["tokens_match_oracle"] = gpu_tokens == [int(v) for v in toks]
    return res


def bench_layer(args, torch, B, inputs, LlamaModel, shared, steps: int, warmup: int) -> dict:
    wl = inputs.WORKLOADS["llama3-8b-layer"]
    shape = wl.shape.replace(vocab_size=256)  # embedding / LM head unused by the layer
    S = wl.prompt_len
    dw, host_w = make_weights(shape, 1 if not args.no_cpu_baseline else 0, keep_head=False)
    model = LlamaModel(shape, dw, max_batch=1, max_prefill_tokens=S)
    del dw
    release(torch)
    x0 = torch.from_numpy(inputs.bf16_bits_to_f32(inputs.activations_bf16_bits(S, shape.dim))).to("cuda:0")
    x = torch.empty_like(x0)
    stream = torch.cuda.current_stream()
    h = model.handle
    evs = []

    def step():
        x.copy_(x0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        B.llm_layer_forward(h, 0, 0, x, S, 0, stream)
        ev[1].record(stream)
        evs.append(ev)

    wall = time_steps(torch, step, steps, warmup)
    layer_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs[warmup:]]))
    x.copy_(x0)
    kt = timed_groups(B, h, lambda: B.llm_layer_forward(h, 0, 0, x, S, 0, stream))
    del model
    release(torch)
    lin, att = layer_flops(shape, S)
    F, dim = shape.ffn_hidden_dim, shape.dim
    res = {"value": round(S * steps / wall, 1), "unit": "tok/s", "ms_per_step": round(wall / steps * 1e3, 3),
           "steps": steps, "warmup": warmup,
           "config": {"workload": "llama3-8b-layer: one Llama-3-8B-shaped decoder layer, bf16 weights, "
                                  "x ~ N(0,1) bf16 [2048, 4096], positions 0..2047", "seq_len": S, "batch": 1,
                      "parallelism": "none (1 GPU)"},
           "prefill_tok_s": round(S / (layer_ms * 1e-3), 1), "layer_ms": round(layer_ms, 4),
           "layer_mfma_frac": round((lin + att) / (layer_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS, 4),
           "roofline": mfma_roofline("gate-up GEMM (M=2048, N=28672, K=4096) + SwiGLU", 2.0 * S * 2 * F * dim,
                                     avg_ms(kt, "gate_up")),
           "roofline_attention": mfma_roofline("causal GQA prefill attention (S=2048)", att, avg_ms(kt, "attn")),
           "per_kernel": per_kernel_table(kt, "layer")}
    if not args.no_cpu_baseline:
        from oracle import decoder_layer
        lw = {"attention_norm": host_w["layers.0.attention_norm.weight"], "wq": host_w["layers.0.attention.wq.weight"],
              "wk": host_w["layers.0.attention.wk.weight"], "wv": host_w["layers.0.attention.wv.weight"],
              "wo": host_w["layers.0.attention.wo.weight"], "ffn_norm": host_w["layers.0.ffn_norm.weight"],
              "w1": host_w["layers.0.feed_forward.w1.weight"], "w3": host_w["layers.0.feed_forward.w3.weight"],
              "w2": host_w["layers.0.feed_forward.w2.weight"]}
        xs = x0.cpu().numpy()
        ck = np.zeros((S, shape.n_kv_heads, shape.head_dim), np.float32)
        cv = np.zeros_like(ck)
        # the whole workload, repeated until about 8 s of CPU work (at most 10 passes)
        times = []
        while len(times) < 10 and sum(times) < 8.0:
            t0 = time.perf_counter()
            decoder_layer(xs, lw, oracle_cfg(shape, 1), ck, cv, np.arange(S))
            times.append(time.perf_counter() - t0)
        t = sum(times) / len(times)
        res["cpu_baseline"] = {"value": round(S / t, 2), "unit": "tok/s", "cores": blas_threads(), "kind": "oracle",
                               "sample": (f"the whole workload: oracle decoder layer (numpy fp32 matmuls, fp64 "
                                          f"norms/softmax) on the same x, S=2048, mean of {len(times)} passes"),
                               "sample_seconds": round(sum(times), 2)}
    return res


def bench_long_prefill(args, torch, B, inputs, LlamaModel, shared, steps: int, warmup: int) -> dict:
    wl = inputs.WORKLOADS["llama3-8b-long-prefill"]
    shape = wl.shape if not args.layers else wl.shape.replace(n_layers=args.layers)
    S = wl.prompt_len
    n_cpu = 0 if args.no_cpu_baseline else 2
    dw, host_w = shared_8b_weights(args, inputs, shared)
    model = LlamaModel(shape, dw, max_batch=1, max_prefill_tokens=S)
    prompt_np = inputs.token_ids(shape.vocab_size, S)
    prompt = torch.as_tensor(prompt_np, device="cuda:0")
    logits = torch.empty(shape.vocab_size, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    h = model.handle
    wall = time_steps(torch, lambda: B.llm_prefill(h, 0, prompt, S, 0, logits, stream), steps, warmup)
    assert model.read_device_error() == 0
    kt = timed_groups(B, h, lambda: B.llm_prefill(h, 0, prompt, S, 0, logits, stream))
    del model
    release(torch)
    lin, att = layer_flops(shape, S)
    total_flops = shape.n_layers * (lin + att) + 2.0 * shape.dim * shape.vocab_size
    t_step = wall / steps
    F, dim = shape.ffn_hidden_dim, shape.dim
    log(f"llama3-8b-long-prefill: {S * steps / wall:.0f} tok/s")
    res = {"value": round(S * steps / wall, 1), "unit": "tok/s", "ms_per_step": round(t_step * 1e3, 3),
           "steps": steps, "warmup": warmup,
           "config": {"workload": "llama3-8b-long-prefill: 32-layer Llama-3-8B-shaped bf16 model, prefill of 8192 "
                                  "ids, last-position logits", "seq_len": S, "batch": 1,
                      "parallelism": "none (1 GPU)"},
           "prefill_tok_s": round(S / t_step, 1),
           "step_mfma_frac": round(total_flops / t_step / 1e12 / MFMA_PEAK_TFLOPS, 4),
           "roofline": mfma_roofline("gate-up GEMM (M=8192, N=28672, K=4096) + SwiGLU", 2.0 * S * 2 * F * dim,
                                     avg_ms(kt, "gate_up")),
           "roofline_attention": mfma_roofline("causal GQA prefill attention (S=8192)", att, avg_ms(kt, "attn")),
           "per_kernel": per_kernel_table(kt, "prefill")}
    if not args.no_cpu_baseline:
        from oracle import OracleModel
        n = 4096
        om = OracleModel(oracle_cfg(shape.replace(max_seq_len=n), n_cpu), host_w, dtype=np.float32)
        cache = om.new_cache(n)
        t0 = time.perf_counter()
        om.hidden(om.embed(prompt_np[:n]), cache, np.arange(n))
        t = time.perf_counter() - t0
        lin_n, att_n = layer_flops(shape, n)
        scale = (shape.n_layers * (lin + att)) / (n_cpu * (lin_n + att_n))
        res["cpu_baseline"] = {"value": round(S / (t * scale), 3), "unit": "tok/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": (f"oracle prefill of the first {n} ids through {n_cpu} of 32 layers "
                                          f"(numpy fp32 matmuls), scaled by the flop ratio {scale:.1f} to 8192 ids "
                                          f"x 32 layers"), "sample_seconds": round(t, 2)}
    return res


def bench_batched_decode(args, torch, B, inputs, LlamaModel, shared, steps: int, warmup: int) -> dict:
    from concurrent.futures import ThreadPoolExecutor
    wl = inputs.WORKLOADS["llama3-8b-batched-decode"]
    shape = wl.shape if not args.layers else wl.shape.replace(n_layers=args.layers)
    Bn = wl.batch
    lo, hi = wl.kv_len_range
    n_cpu = 0 if args.no_cpu_baseline else min(8, shape.n_layers)
    dw, host_w = shared_8b_weights(args, inputs, shared)
    model = LlamaModel(shape, dw, max_batch=Bn, max_prefill_tokens=1)
    lengths = inputs.kv_lengths(Bn, lo, hi)
    kv = model.kv_cache_view()
    G, hd = shape.n_kv_heads, shape.head_dim
    t0 = time.perf_counter()
    jobs = [(w, b, g) for w in (0, 1) for b in range(Bn) for g in range(G)]
    for l in range(shape.n_layers):
        def gen(job, l=l):
            w, b, g = job
            return job, inputs.kv_contents_bf16_bits(l, w, b, g, int(lengths[b]), hd)
        with ThreadPoolExecutor(16) as ex:
            for (w, b, g), blk in ex.map(gen, jobs):
                kv[l, w, b, g, : lengths[b]] = torch.from_numpy(blk.view(np.int16)).view(torch.bfloat16).to(
                    "cuda:0").to(kv.dtype)
    log(f"llama3-8b-batched-decode: cache contents generated in {time.perf_counter() - t0:.1f}s")
    toks = torch.as_tensor(inputs.token_ids(shape.vocab_size, Bn, sub=4), device="cuda:0")
    slots = torch.arange(Bn, dtype=torch.int32, device="cuda:0")
    pos = torch.as_tensor(lengths, device="cuda:0")
    logits = torch.empty(Bn, shape.vocab_size, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    h = model.handle

    def step():
        B.llm_decode_step(h, Bn, slots, pos, toks, logits, stream)

    wall = time_steps(torch, step, steps, warmup)
    assert model.read_device_error() == 0
    kt = timed_groups(B, h, step)
    del kv, model
    release(torch)
    t_step = wall / steps
    L, dim, F, V = shape.n_layers, shape.dim, shape.ffn_hidden_dim, shape.vocab_size
    w_bytes = 2 * (L * (dim * (shape.n_heads + 2 * G) * hd + dim * shape.n_heads * hd + 3 * F * dim) + V * dim)
    kv_bytes = L * G * hd * 2 * 2 * float(np.sum(lengths.astype(np.int64) + 1))
    att_bytes_per_launch = kv_bytes / L
    log(f"llama3-8b-batched-decode: {Bn * steps / wall:.0f} tok/s")
    res = {"value": round(Bn * steps / wall, 1), "unit": "tok/s", "ms_per_step": round(t_step * 1e3, 3),
           "steps": steps, "warmup": warmup,
           "config": {"workload": "llama3-8b-batched-decode: 32-layer Llama-3-8B-shaped bf16 model, one decode step "
                                  "for 64 sequences with cached lengths U{1024..8192}", "batch": Bn,
                      "parallelism": "none (1 GPU)"},
           "decode_tok_s": round(Bn / t_step, 1),
           "step_hbm_frac": round((w_bytes + kv_bytes) / t_step / 1e9 / HBM_PEAK_GBS, 4),
           "step_bytes": int(w_bytes + kv_bytes),
           "roofline": hbm_roofline("split-KV decode attention + combine (per layer, 64 rows)", att_bytes_per_launch,
                                    avg_ms(kt, "attn")),
           "per_kernel": per_kernel_table(kt, "decode")}
    if not args.no_cpu_baseline:
        from oracle import OracleModel
        om = OracleModel(oracle_cfg(shape.replace(max_seq_len=hi + 1), n_cpu), host_w, dtype=np.float32)
        # 32 of the 64 rows (the longest, the shortest and 30 seeded others), each decoded through n_cpu layers
        # plus the LM head; the layer time is scaled to 32 layers and the 32 rows to the batch of 64.
        rng = np.random.default_rng(5)
        rows = [int(np.argmax(lengths)), int(np.argmin(lengths))]
        rows += [int(r) for r in rng.permutation(Bn) if int(r) not in rows][:30]
        t_layers = t_head = 0.0
        for b in rows:
            Lb = int(lengths[b])
            cache = om.new_cache(Lb + 1)

            def kvgen(job, b=b, Lb=Lb):
                l, w, g = job
                return job, inputs.kv_contents_bf16_bits(l, w, b, g, Lb, hd)
            with ThreadPoolExecutor(16) as ex:
                for (l, w, g), blk in ex.map(kvgen, [(l, w, g) for l in range(n_cpu) for w in (0, 1) for g in range(G)]):
                    cache[l][w][:Lb, g] = inputs.bf16_bits_to_f32(blk)
            t0 = time.perf_counter()
            hdn = om.hidden(om.embed([int(toks[b])]), cache, np.array([Lb]))
            t1 = time.perf_counter()
            om.logits_of(hdn)
            t2 = time.perf_counter()
            t_layers += t1 - t0
            t_head += t2 - t1
        t_batch = (t_layers * (L / n_cpu) + t_head) * (Bn / len(rows))
        res["cpu_baseline"] = {"value": round(Bn / t_batch, 4), "unit": "tok/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": (f"oracle decode of {len(rows)} of the {Bn} rows (the longest, the shortest "
                                          f"and {len(rows) - 2} seeded others) through {n_cpu} of 32 layers plus the "
                                          f"LM head; layer time scaled to 32 layers and the rows to the batch"),
                               "sample_seconds": round(t_layers + t_head, 2)}
    return res


WORKLOAD_FUNS = {"llama3-8b": bench_generate, "stories15m": bench_stories, "llama3-8b-layer": bench_layer,
                 "llama3-8b-long-prefill": bench_long_prefill, "llama3-8b-batched-decode": bench_batched_decode}
# Steps and warm-up of the workloads that ride along with the headline in the default run.
EXTRA_STEPS = {"stories15m": (20, 3), "llama3-8b-layer": (20, 3), "llama3-8b-long-prefill": (5, 1),
               "llama3-8b-batched-decode": (10, 2)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOAD_FUNS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=16, help="layers in the CPU oracle sample (llama3-8b)")
    ap.add_argument("--cpu-decode-steps", type=int, default=100, help="decode steps in the CPU oracle sample (llama3-8b)")
    ap.add_argument("--layers", type=int, default=0,
                    help="profiling aid (8B workloads): build the models with this many layers; every kernel keeps "
                         "its launch shape, but the line is then not the metric")
    ap.add_argument("--copy-probe", action="store_true",
                    help="end with one plain elementwise pass over 1 GiB (torch.neg, fp32: reads 1 GiB, writes "
                         "1 GiB), the reference dispatch that scales the FETCH_SIZE / WRITE_SIZE counters of a "
                         "profiled run")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch

    from llama_decoder_transformer_amd import binding as B
    from llama_decoder_transformer_amd import inputs
    from llama_decoder_transformer_amd.model import LlamaModel

    shared = {}
    head = "llama3-8b" if args.workload == "all" else args.workload
    body = WORKLOAD_FUNS[head](args, torch, B, inputs, LlamaModel, shared, args.steps, args.warmup)
    if args.workload == "all":
        extra = {}
        for name, (k, w) in EXTRA_STEPS.items():
            t0 = time.perf_counter()
            extra[name] = WORKLOAD_FUNS[name](args, torch, B, inputs, LlamaModel, shared, k, w)
            log(f"{name} done in {time.perf_counter() - t0:.1f}s")
        body["workloads"] = extra
    shared.clear()
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    body.pop("steps", None)
    body.pop("warmup", None)
    dtype = body.pop("dtype", "f16")
    res = {"metric": METRIC, "value": body.pop("value"), "unit": body.pop("unit"), "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": body.pop("ms_per_step"), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "dtype_note": ("fp32 throughout" if dtype == "f32" else
                          "fp16 MFMA operands with fp32 accumulation; bf16 weights held as fp16; fp32 residual"),
           "data": "synthetic", "config": body.pop("config")}
    res.update(body)
    if args.layers:
        res["profiling_only"] = f"models built with {args.layers} layers instead of the workload's; not the metric"
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
