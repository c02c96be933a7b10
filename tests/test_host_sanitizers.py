"""The library's host code under AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer.

Builds libllm with the sanitizers on its host half only (each ``-fsanitize=`` right after
``-Xarch_host``; the gfx950 code is built as usual), links the C driver
``tests/sanitize/abi_host_driver.c`` against it with the same compiler's runtime, and runs it:
config validation, the size queries (Llama-3-8B shape included), every argument check of
llm_init_weights and the NULL-handle / bad-argument paths of every other entry point.  No GPU
is touched.  The build takes about half a minute on a few cores.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "llama_decoder_transformer_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_host_driver.c")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_abi_host_paths_clean_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *SAN, "-I", INCLUDE, "-I", CSRC]

    def compile_one(f):
        return _run([HIPCC, *flags, "-c", os.path.join(CSRC, f), "-o", str(tmp_path / (f[:-4] + ".o"))])

    with ThreadPoolExecutor(min(4, len(srcs))) as ex:
        list(ex.map(compile_one, srcs))
    lib = tmp_path / "libllm_san.so"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, *[str(tmp_path / (f[:-4] + ".o")) for f in srcs],
          "-o", str(lib)])
    exe = tmp_path / "abi_host_driver"
    _run([CLANG, "-g", "-fsanitize=address,undefined", "-I", INCLUDE, DRIVER, "-L", str(tmp_path), "-lllm_san",
          f"-Wl,-rpath,{tmp_path}", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([str(exe)], env=env)
    assert "all checks passed" in out
    assert "runtime error" not in out and "Sanitizer" not in out
    shutil.rmtree(tmp_path, ignore_errors=True)
