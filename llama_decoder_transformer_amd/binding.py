"""ctypes binding of ``libllm.so`` (the C ABI in include/llm.h).

Argument marshalling only: every step of the decoder pass runs in the HIP
library.  Functions keep the C names; torch tensors stand in for device
pointers and ``torch.cuda`` streams for ``hipStream_t``.  Importing this module
never falls back to anything: a missing library raises ``LibraryMissing``.

torch is imported before the library is loaded so that both share torch's HIP
runtime (the library's ``libamdhip64.so.7`` dependency then resolves to the copy
torch already mapped).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_void_p

import torch  # noqa: F401  (must be loaded before libllm.so, see above)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllm.so")

LLM_F32 = 0
LLM_BF16 = 1
STATUS = {0: "LLM_OK", -1: "LLM_ERR_INVALID_ARG", -2: "LLM_ERR_CONFIG", -3: "LLM_ERR_OUT_OF_RANGE",
          -4: "LLM_ERR_BUFFER_TOO_SMALL", -5: "LLM_ERR_HIP"}
DEVERR_TOKEN, DEVERR_POSITION, DEVERR_SLOT, DEVERR_RANGE, DEVERR_SYNC = 1, 2, 4, 8, 16

EXPORTED = ("llm_check_config", "llm_packed_weight_bytes", "llm_kv_cache_bytes", "llm_workspace_bytes",
            "llm_init_weights", "llm_prefill", "llm_prefill_batch", "llm_layer_forward", "llm_decode_step",
            "llm_decode_step_noalloc", "llm_argmax",
            "llm_generate", "llm_read_device_error", "llm_set_kernel_timing", "llm_kernel_timing",
            "llm_free", "llm_status_string", "llm_last_error_message")
KERNEL_GROUPS = ("embed", "rmsnorm", "qkv", "attn", "wo", "gate_up", "down", "lm_head", "argmax", "decode_block")


class LibraryMissing(RuntimeError):
    pass


class LlmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class llm_config(ctypes.Structure):
    _fields_ = [("dim", c_int32), ("n_layers", c_int32), ("n_heads", c_int32), ("n_kv_heads", c_int32),
                ("vocab_size", c_int32), ("max_seq_len", c_int32), ("ffn_hidden_dim", c_int32),
                ("rope_theta", c_float), ("norm_eps", c_float), ("dtype", c_int32), ("max_batch", c_int32),
                ("max_prefill_tokens", c_int32)]


PP = POINTER(c_void_p)


class llm_weights(ctypes.Structure):
    _fields_ = [("tok_embeddings", c_void_p), ("attention_norm", PP), ("wq", PP), ("wk", PP), ("wv", PP),
                ("wo", PP), ("ffn_norm", PP), ("w1", PP), ("w3", PP), ("w2", PP), ("norm", c_void_p),
                ("output", c_void_p)]


_lib = None


def lib():
    """The loaded library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is not built; run `python -m llama_decoder_transformer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = POINTER(llm_config)
        sig = {
            "llm_check_config": (c_int32, [cfgp]),
            "llm_packed_weight_bytes": (c_size_t, [cfgp]),
            "llm_kv_cache_bytes": (c_size_t, [cfgp]),
            "llm_workspace_bytes": (c_size_t, [cfgp]),
            "llm_init_weights": (c_int32, [cfgp, POINTER(llm_weights), c_void_p, c_size_t, c_void_p, c_size_t,
                                           c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
            "llm_prefill": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
            "llm_prefill_batch": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(c_int32), POINTER(c_int32),
                                            c_void_p, c_void_p, c_void_p]),
            "llm_layer_forward": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p]),
            "llm_decode_step": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
            "llm_decode_step_noalloc": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                                  c_void_p]),
            "llm_argmax": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p]),
            "llm_generate": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                       c_void_p, c_void_p]),
            "llm_read_device_error": (c_int32, [c_void_p, POINTER(c_int32), c_void_p]),
            "llm_set_kernel_timing": (c_int32, [c_void_p, c_int32]),
            "llm_kernel_timing": (c_int32, [c_void_p, c_int32, POINTER(ctypes.c_int64), POINTER(ctypes.c_int64),
                                            POINTER(ctypes.c_double)]),
            "llm_free": (None, [c_void_p]),
            "llm_status_string": (c_char_p, [c_int32]),
            "llm_last_error_message": (c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise LlmError(status, lib().llm_last_error_message().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


# ----------------------------------------------------------------------------- C names

def llm_check_config(cfg: llm_config) -> None:
    _check(lib().llm_check_config(ctypes.byref(cfg)))


def llm_packed_weight_bytes(cfg: llm_config) -> int:
    return lib().llm_packed_weight_bytes(ctypes.byref(cfg))


def llm_kv_cache_bytes(cfg: llm_config) -> int:
    return lib().llm_kv_cache_bytes(ctypes.byref(cfg))


def llm_workspace_bytes(cfg: llm_config) -> int:
    return lib().llm_workspace_bytes(ctypes.byref(cfg))


def llm_init_weights(cfg: llm_config, weights: llm_weights, packed, kv_cache, workspace, stream=None) -> int:
    h = c_void_p()
    _check(lib().llm_init_weights(ctypes.byref(cfg), ctypes.byref(weights), _ptr(packed), packed.numel(),
                                  _ptr(kv_cache), kv_cache.numel(), _ptr(workspace), workspace.numel(),
                                  _stream(stream), ctypes.byref(h)))
    return h.value


def llm_prefill(handle: int, slot: int, tokens, n_tokens: int, start_pos: int, logits, stream=None) -> None:
    _check(lib().llm_prefill(handle, slot, _ptr(tokens), n_tokens, start_pos, _ptr(logits), _stream(stream)))


def llm_prefill_batch(handle: int, slots, starts, lens, tokens, logits, stream=None) -> None:
    """slots / starts / lens: host integer sequences of equal length (one entry per sequence)."""
    b = len(lens)
    if len(slots) != b or len(starts) != b:
        raise ValueError("slots, starts and lens must have one entry per sequence")
    arr = c_int32 * max(b, 1)
    _check(lib().llm_prefill_batch(handle, b, arr(*[int(v) for v in slots]), arr(*[int(v) for v in starts]),
                                   arr(*[int(v) for v in lens]), _ptr(tokens), _ptr(logits), _stream(stream)))


def llm_layer_forward(handle: int, layer: int, slot: int, x, n_tokens: int, start_pos: int, stream=None) -> None:
    _check(lib().llm_layer_forward(handle, layer, slot, _ptr(x), n_tokens, start_pos, _stream(stream)))


def llm_decode_step(handle: int, batch: int, slots, positions, tokens, logits, stream=None) -> None:
    _check(lib().llm_decode_step(handle, batch, _ptr(slots), _ptr(positions), _ptr(tokens), _ptr(logits),
                                 _stream(stream)))


def llm_decode_step_noalloc(handle: int, batch: int, slots, positions, tokens, logits, stream=None) -> None:
    _check(lib().llm_decode_step_noalloc(handle, batch, _ptr(slots), _ptr(positions), _ptr(tokens), _ptr(logits),
                                         _stream(stream)))


def llm_argmax(logits, rows: int, vocab: int, out, stream=None) -> None:
    _check(lib().llm_argmax(_ptr(logits), rows, vocab, _ptr(out), _stream(stream)))


def llm_generate(handle: int, batch: int, slots, positions, tokens, n_steps: int, out_tokens, logits,
                 stream=None) -> None:
    _check(lib().llm_generate(handle, batch, _ptr(slots), _ptr(positions), _ptr(tokens), n_steps,
                              _ptr(out_tokens), _ptr(logits), _stream(stream)))


def llm_read_device_error(handle: int, stream=None) -> int:
    f = c_int32(0)
    _check(lib().llm_read_device_error(handle, ctypes.byref(f), _stream(stream)))
    return f.value


def llm_set_kernel_timing(handle: int, enable: bool) -> None:
    _check(lib().llm_set_kernel_timing(handle, 1 if enable else 0))


def llm_kernel_timing(handle: int, kind: int) -> tuple[int, float]:
    """(invocations, total kernel ms) of one kernel group."""
    n, _, ms = llm_kernel_timing_full(handle, kind)
    return n, ms


def llm_kernel_timing_full(handle: int, kind: int) -> tuple[int, int, float]:
    """(invocations, kernels dispatched, total kernel ms) of one kernel group."""
    n = ctypes.c_int64(0)
    k = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().llm_kernel_timing(handle, kind, ctypes.byref(n), ctypes.byref(k), ctypes.byref(ms)))
    return n.value, k.value, ms.value


def llm_free(handle: int) -> None:
    lib().llm_free(handle)
