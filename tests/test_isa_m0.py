"""The LDS-DMA inline assembly and M0.

gemm_dma64_kernel issues its global -> LDS loads from inline assembly that sets M0 (the LDS
destination) itself, right before each load.  The compiler also uses M0 for some instructions and
does not promise to honour an M0 clobber, so the asm is only safe in functions where the compiler
generates no M0 access of its own.  This test compiles every kernel source for gfx950 to assembly
and checks, for each function that contains such an asm block, that
  - every asm block that touches M0 is exactly `s_mov_b32 m0, sN` / `s_nop 0` /
    `global_load_lds_dwordx4`, and
  - no instruction outside the asm blocks names M0.
No GPU is needed; the compile takes about half a minute.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "llama_decoder_transformer_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S"]
M0 = re.compile(r"\bm0\b")


def _functions(asm: str):
    """Yield (name, [(in_asm_block, code), ...]) per function of an assembly listing."""
    name, body, in_asm = None, [], False
    for line in asm.split("\n"):
        m = re.match(r"^(_Z[^\s:]+):", line)
        if m:
            if name:
                yield name, body
            name, body, in_asm = m.group(1), [], False
            continue
        if ";;#ASMSTART" in line:
            in_asm = True
            body.append((True, "<asm>"))
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if name and code:
            body.append((in_asm, code))
    if name:
        yield name, body


def _asm_blocks(body):
    blocks, cur = [], None
    for in_asm, code in body:
        if code == "<asm>":
            cur = []
            blocks.append(cur)
        elif in_asm and cur is not None:
            cur.append(code)
    return blocks


def _violations(f: str, asm: str):
    """(functions using the M0 asm, list of problems) for one assembly listing."""
    checked, bad = 0, []
    for name, body in _functions(asm):
        blocks = [b for b in _asm_blocks(body) if any(M0.search(c) for c in b)]
        if not blocks:
            continue
        checked += 1
        for b in blocks:
            if not (len(b) == 3 and re.fullmatch(r"s_mov_b32 m0, s\d+", b[0]) and b[1] == "s_nop 0"
                    and b[2].startswith("global_load_lds_dwordx4 ")):
                bad.append((f, name, "asm block", b))
        outside = [c for in_asm, c in body if not in_asm and c != "<asm>" and M0.search(c)]
        if outside:
            bad.append((f, name, "compiler M0 use", outside[:5]))
    return checked, bad


SYNTHETIC = """_ZN3llm1kEv:                            ; @_ZN3llm1kEv
\ts_load_dwordx2 s[0:1], s[0:1], 0x0
\t;;#ASMSTART
\ts_mov_b32 m0, s6
\ts_nop 0
\tglobal_load_lds_dwordx4 v1, s[0:1]
\t;;#ASMEND
{extra}
\ts_endpgm
"""


def test_m0_checker_flags_compiler_use_and_odd_blocks():
    assert _violations("x", SYNTHETIC.format(extra="")) == (1, [])
    n, bad = _violations("x", SYNTHETIC.format(extra="\ts_mov_b32 m0, -1\n\tds_add_u32 v0, v1"))
    assert n == 1 and bad and bad[0][2] == "compiler M0 use"
    n, bad = _violations("x", SYNTHETIC.format(extra="\t;;#ASMSTART\n\ts_mov_b32 m0, s7\n\t;;#ASMEND"))
    assert n == 1 and bad and bad[0][2] == "asm block"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_m0_is_touched_only_by_the_dma_asm(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        out = tmp_path / (f[:-4] + ".s")
        r = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, f), "-o", str(out)], stdout=subprocess.PIPE,
                           stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-3000:]
        return f, out.read_text()

    with ThreadPoolExecutor(min(4, len(srcs))) as ex:
        listings = list(ex.map(compile_one, srcs))

    checked, bad = 0, []
    for f, asm in listings:
        n, b = _violations(f, asm)
        checked += n
        bad += b
    assert not bad, bad
    # the 256 x 256 and 256 x 128 instances of gemm_dma64_kernel, four epilogues each
    assert checked >= 8, checked
