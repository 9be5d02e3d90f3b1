"""Build the gfx950 library ``libsparse_kv.so`` in-tree with hipcc.

Run ``python -m top_sparse_kv_block_amd.build`` (or ``__graft_entry__.build()``).
Every HIP source is compiled for gfx950 only; packed-FP32 instructions are
disabled for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsparse_kv.so")
SOURCES = ["abi.hip", "score.hip", "topk.hip", "cache.hip", "attention.hip", "append.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libsparse_kv.so)")


def build(verbose: bool = False, jobs: int = 8, ab_valu: bool = False, out: str | None = None) -> str:
    """Compile every HIP source for gfx950 and link ``libsparse_kv.so``.

    ab_valu=True builds the A/B variant in which bf16 keys are scored and
    bf16 attention logits formed on the vector ALU instead of the matrix
    cores (define SKV_AB_VALU_BF16), into ``out`` (default
    ``libsparse_kv_valu.so`` beside the library); it exists only for the
    kernel-trace comparison of the two and is loaded by setting
    SKV_LIBRARY to its path."""
    cc = hipcc()
    lib = out or (os.path.join(HERE, "libsparse_kv_valu.so") if ab_valu else LIB)
    defines = ["-DSKV_AB_VALU_BF16"] if ab_valu else []
    tmpdir = tempfile.mkdtemp(prefix="skv_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, *defines, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        while procs:
            _wait(procs.pop(0), verbose)
        tmp_lib = lib + ".tmp"
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp_lib, lib)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return lib


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    lines = [ln for ln in (out or "").splitlines() if "packed-fp32-ops" not in ln]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError(f"hipcc failed on {src}")
    if verbose and lines:
        print("\n".join(lines))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, ab_valu="--ab-valu" in sys.argv))
