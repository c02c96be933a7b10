"""Host-only checks of the C ABI: the library loads, exports what include/llm.h
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llm.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:llm_status|size_t|void|const char\*)\s+(llm_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def B():
    from llama_decoder_transformer_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from llama_decoder_transformer_amd import build
        build.build()
    return binding


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for n in ("llm_init_weights", "llm_prefill", "llm_decode_step", "llm_argmax"):
        assert n in names


def test_library_exports_every_declared_symbol(B):
    L = B.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(B.EXPORTED)


def _cfg(B, **kw):
    from llama_decoder_transformer_amd import inputs
    from llama_decoder_transformer_amd.model import make_config
    c = make_config(inputs.STORIES15M, max_batch=2, max_prefill_tokens=16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_validation(B):
    B.llm_check_config(_cfg(B))
    bad = [dict(dim=290), dict(n_kv_heads=4), dict(dtype=7), dict(max_batch=0), dict(n_heads=5, dim=300),
           dict(ffn_hidden_dim=770), dict(rope_theta=-1.0), dict(max_prefill_tokens=0), dict(vocab_size=0),
           dict(n_heads=9, n_kv_heads=1, dim=9 * 48)]
    for kw in bad:
        with pytest.raises(B.LlmError) as e:
            B.llm_check_config(_cfg(B, **kw))
        assert e.value.status == -2, kw
        assert B.llm_packed_weight_bytes(_cfg(B, **kw)) == 0


def test_size_queries(B):
    from llama_decoder_transformer_amd import inputs
    c = _cfg(B)
    s = inputs.STORIES15M
    n_params = sum(int(__import__("numpy").prod(v)) for v in s.weight_shapes().values())
    assert B.llm_packed_weight_bytes(c) >= 4 * n_params
    hd = s.dim // s.n_heads
    assert B.llm_kv_cache_bytes(c) == s.n_layers * 2 * 2 * s.n_kv_heads * s.max_seq_len * hd * 4
    assert B.llm_workspace_bytes(c) > 16 * s.dim * 4
    c8 = _cfg(B, dtype=B.LLM_BF16)
    assert B.llm_kv_cache_bytes(c8) * 2 == B.llm_kv_cache_bytes(c)


def test_init_rejects_bad_buffers_before_any_gpu_work(B):
    L = B.lib()
    c = _cfg(B)
    h = ctypes.c_void_p()
    w = B.llm_weights()
    fake = 256
    # null weights struct
    st = L.llm_init_weights(ctypes.byref(c), None, fake, 1 << 40, fake, 1 << 40, fake, 1 << 40, None,
                            ctypes.byref(h))
    assert st == -1
    # null member pointers
    st = L.llm_init_weights(ctypes.byref(c), ctypes.byref(w), fake, 1 << 40, fake, 1 << 40, fake, 1 << 40, None,
                            ctypes.byref(h))
    assert st == -1 and b"NULL" in L.llm_last_error_message()
    # buffers too small (checked before any copy)
    arr = (ctypes.c_void_p * c.n_layers)(*([fake] * c.n_layers))
    pp = ctypes.cast(arr, B.PP)
    w = B.llm_weights(tok_embeddings=fake, norm=fake, output=fake, attention_norm=pp, wq=pp, wk=pp, wv=pp, wo=pp,
                      ffn_norm=pp, w1=pp, w3=pp, w2=pp)
    st = L.llm_init_weights(ctypes.byref(c), ctypes.byref(w), fake, 10, fake, 1 << 40, fake, 1 << 40, None,
                            ctypes.byref(h))
    assert st == -4 and b"packed" in L.llm_last_error_message()
    st = L.llm_init_weights(ctypes.byref(c), ctypes.byref(w), fake, 1 << 40, fake, 10, fake, 1 << 40, None,
                            ctypes.byref(h))
    assert st == -4 and b"KV" in L.llm_last_error_message()
    st = L.llm_init_weights(ctypes.byref(c), ctypes.byref(w), fake, 1 << 40, fake, 1 << 40, fake, 10, None,
                            ctypes.byref(h))
    assert st == -4 and b"workspace" in L.llm_last_error_message()
    bad = _cfg(B, dim=290)
    st = L.llm_init_weights(ctypes.byref(bad), ctypes.byref(w), fake, 1 << 40, fake, 1 << 40, fake, 1 << 40, None,
                            ctypes.byref(h))
    assert st == -2 and h.value is None


def test_calls_reject_null_handles_and_sizes(B):
    L = B.lib()
    assert L.llm_prefill(None, 0, 256, 4, 0, 256, None) == -1
    assert L.llm_layer_forward(None, 0, 0, 256, 4, 0, None) == -1
    one = (ctypes.c_int32 * 1)(1)
    assert L.llm_prefill_batch(None, 1, one, one, one, 256, 256, None) == -1
    assert L.llm_decode_step(None, 1, 256, 256, 256, 256, None) == -1
    assert L.llm_generate(None, 1, 256, 256, 256, 3, 256, 256, None) == -1
    assert L.llm_argmax(None, 1, 10, 256, None) == -1
    assert L.llm_argmax(256, 0, 10, 256, None) == -1
    f = ctypes.c_int32()
    assert L.llm_read_device_error(None, ctypes.byref(f), None) == -1
    L.llm_free(None)
    assert L.llm_status_string(-4) == b"buffer too small"
