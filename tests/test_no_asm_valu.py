"""No vector-ALU instruction is written as inline asm in any kernel.

The compiler inserts the wait states that MFMA and other dependent
instructions need after a VGPR is written, but it does not see inside an
inline-asm block: a vector instruction written there can feed an MFMA too
early, and whether it does depends only on how the surrounding code happens
to be scheduled.  (The int4 drafter's code-to-fp16 step once was such a
block; a change elsewhere moved an MFMA closer to it and the results went
wrong.)  Inline asm stays only for what has no compiler form: the direct
global-to-LDS loads with their m0 setup, explicit waits, and empty
statements that pin values to a register class.

Each HIP source is compiled for gfx950 to assembly (device code only, no
GPU needed) and every ASMSTART/ASMEND block is checked.
"""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from lossless_speculative_decoding_vc_amd import build as vcbuild

# instruction prefixes an inline-asm block may hold
ALLOWED = ("s_mov_b32 m0", "global_load_lds_", "buffer_load_", "s_waitcnt", "s_nop")


def _asm_blocks(text):
    blocks, cur = [], None
    for line in text.splitlines():
        t = line.strip()
        if t == ";;#ASMSTART":
            cur = []
        elif t == ";;#ASMEND":
            blocks.append(cur)
            cur = None
        elif cur is not None and t and not t.startswith(";"):
            cur.append(re.sub(r"\s+", " ", t))
    return blocks


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        hipcc = vcbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("vc_asm")
    srcs = [s for s in vcbuild.sources() if s.endswith(".hip")]

    def compile_one(src):
        dst = str(out / (os.path.basename(src) + ".s"))
        r = subprocess.run([hipcc, *vcbuild.CFLAGS, "--offload-device-only", "-S", src, "-o", dst],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"device compile of {src} failed:\n{r.stderr[-3000:]}"
        return os.path.basename(src), open(dst).read()

    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4, 8)) as ex:
        return dict(ex.map(compile_one, srcs))


def test_inline_asm_holds_no_vector_alu(device_asm):
    bad = []
    for name, text in device_asm.items():
        for block in _asm_blocks(text):
            for ins in block:
                if not ins.startswith(ALLOWED):
                    bad.append(f"{name}: {ins}")
    assert not bad, "inline asm outside the allowed loads and waits:\n" + "\n".join(sorted(set(bad))[:40])


def test_the_scan_sees_asm_blocks(device_asm):
    # the direct global->LDS loads are inline asm: the check above is not vacuous
    assert any(_asm_blocks(t) for t in device_asm.values())
