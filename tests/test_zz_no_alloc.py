"""llm_decode_step_noalloc: the decode step whose kernel scratch lives in the library's static
device array, against llm_decode_step (scratch in the model's workspace) on the same inputs.

Two calls in a row, the second with a smaller batch (the array keeps the first call's
contents), must each give logits bitwise equal to llm_decode_step's.  The shapes make the
scratch matter: decode batches above 8 rows take the split-K projections, and caches of a
few hundred positions split the attention into chunks merged by a second pass.
"""
import numpy as np
import pytest
import torch

from llama_decoder_transformer_amd import binding as B
from llama_decoder_transformer_amd import inputs

from helpers import device_weights, host_weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

SHAPES = {
    "small": inputs.ModelShape("noalloc-small", dim=512, n_layers=2, n_heads=4, n_kv_heads=2, ffn_hidden_dim=1024,
                               vocab_size=1000, max_seq_len=600, rope_theta=500000.0, norm_eps=1e-5, dtype="bf16"),
    "8b-2layer": inputs.LLAMA3_8B.replace(name="noalloc-8b", n_layers=2, vocab_size=1000, max_seq_len=1100),
}


def _i32(a):
    return torch.as_tensor(np.asarray(a, np.int32), device=DEV)


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_decode_step_noalloc_equals_decode_step(name):
    from llama_decoder_transformer_amd.model import LlamaModel
    shape = SHAPES[name]
    hw = host_weights(shape, seed=21)
    nmax = 24
    m = LlamaModel(shape, device_weights(hw, DEV), max_batch=nmax, max_prefill_tokens=1, device=DEV)
    kv = m.kv_cache_view()
    G, hd = shape.n_kv_heads, shape.head_dim
    lengths = inputs.kv_lengths(nmax, 100, shape.max_seq_len - 2, seed=21)
    for b in range(nmax):
        for l in range(shape.n_layers):
            for which in (0, 1):
                blk = np.stack([inputs.kv_contents_bf16_bits(l, which, b, g, int(lengths[b]), hd, seed=21)
                                for g in range(G)])
                kv[l, which, b, :, : lengths[b]] = torch.from_numpy(blk.view(np.int16)).view(torch.bfloat16).to(
                    DEV).to(kv.dtype)
    toks = inputs.token_ids(shape.vocab_size, nmax, sub=21)
    for batch in (24, 11, 1):
        slots, pos, tk = _i32(np.arange(batch)), _i32(lengths[:batch]), _i32(toks[:batch])
        ref = torch.empty(batch, shape.vocab_size, dtype=torch.float32, device=DEV)
        got = torch.full_like(ref, float("nan"))
        B.llm_decode_step(m.handle, batch, slots, pos, tk, ref)
        ref_np = ref.cpu().numpy()
        # the same step again through the static scratch; the cache entries it rewrites are the same
        B.llm_decode_step_noalloc(m.handle, batch, slots, pos, tk, got)
        got_np = got.cpu().numpy()
        print(f"[noalloc {name} batch={batch}] max |diff| {np.max(np.abs(got_np - ref_np)):.3e}", flush=True)
        assert np.all(np.isfinite(ref_np))
        assert np.array_equal(got_np, ref_np)
    assert m.read_device_error() == 0


def test_decode_step_noalloc_rejects_a_step_beyond_its_scratch():
    """64-dimension heads over a 65536-position cache take the vector decode attention in 512-key
    chunks: 64 rows need 17.3 MB of partials (accepted, and equal to llm_decode_step), 128 rows
    34.6 MB, more than the 32 MiB static array (refused before anything runs)."""
    from llama_decoder_transformer_amd.model import LlamaModel
    shape = SHAPES["small"].replace(name="noalloc-big", n_layers=1, n_heads=8, n_kv_heads=2, max_seq_len=65536)
    assert shape.head_dim == 64
    hw = host_weights(shape, seed=22)
    m = LlamaModel(shape, device_weights(hw, DEV), max_batch=128, max_prefill_tokens=1, device=DEV)
    n = 64
    args = (_i32(np.arange(n)), _i32(np.zeros(n)), _i32(np.arange(n) % shape.vocab_size))
    ref = torch.empty(n, shape.vocab_size, dtype=torch.float32, device=DEV)
    got = torch.full_like(ref, float("nan"))
    B.llm_decode_step(m.handle, n, *args, ref)
    B.llm_decode_step_noalloc(m.handle, n, *args, got)
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())
    n = 128
    logits = torch.empty(n, shape.vocab_size, dtype=torch.float32, device=DEV)
    with pytest.raises(B.LlmError) as e:
        B.llm_decode_step_noalloc(m.handle, n, _i32(np.arange(n)), _i32(np.zeros(n)), _i32(np.zeros(n)), logits)
    assert e.value.status == -3
    assert "scratch" in str(e.value)
    assert m.read_device_error() == 0
