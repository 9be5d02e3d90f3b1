"""ISA checks of the gfx950 build (CPU only: hipcc cross-compiles).

The bf16 dot products of the scoring kernels must feed four different
register pairs to the four packed dot2 instructions of a 16-byte chunk; one
way of writing the bit-casts made the compiler reuse element 0 for all four.
The bf16 attention must use the matrix-core q.k instruction.  No packed-FP32
instruction may be emitted (the build disables them).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "top_sparse_kv_block_amd", "csrc")


def _asm(src):
    from top_sparse_kv_block_amd.build import HIPCC_FLAGS, hipcc
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S", "--cuda-device-only",
           os.path.join(CSRC, src), "-o", "-"]
    return subprocess.run(cmd, capture_output=True, text=True, check=True).stdout


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
@pytest.mark.parametrize("src", ["score.hip", "attention.hip"])
def test_bf16_contractions_and_no_packed_fp32(src):
    asm = _asm(src)
    if src == "score.hip":
        dots = re.findall(r"v_dot2c?_f32_bf16\S*\s+(v\d+),\s*(v\d+),\s*(v\d+)", asm)
        assert dots, "expected packed bf16 dot products"
        for i in range(len(dots) - 3):
            window = dots[i:i + 4]
            if len({d[0] for d in window}) == 1:  # one accumulation chain
                assert len({d[1:] for d in window}) == 4, window
    else:
        assert re.search(r"v_mfma_f32_16x16x32_bf16", asm), "expected bf16 matrix-core q.k"
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)
