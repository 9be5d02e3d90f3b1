"""The C ABI library loads and exports every entry point its header declares
(CPU only: no compute call is made)."""
import os
import re
import subprocess

import pytest

from top_sparse_kv_block_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sparse_kv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sparse_\w+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared()
    for fn in ("sparse_kv_score", "sparse_kv_topk", "sparse_kv_cache_update", "sparse_decode_attention"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libsparse_kv.so is not built (run __graft_entry__.build())")
    lib = binding.load()
    for fn in _declared():
        assert hasattr(lib, fn), fn
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert set(_declared()) <= exported
    assert set(binding.EXPORTS) == set(_declared())


def test_status_strings_without_gpu():
    assert binding.status_string(0) == "ok"
    assert "capacity" in binding.status_string(4)
    assert binding.status_string(99) == "unknown status"


def test_host_side_validation_needs_no_gpu():
    # invalid shapes are rejected on the host before any launch
    s = binding.make_shape(1, 8, 3, 64, 1024, "f32")  # Hq % Hkv != 0
    assert binding.sparse_decode_attention_splits(s, 8) == 0
    assert binding.sparse_decode_attention_workspace_bytes(s, 8, 0) == 0
    ok = binding.make_shape(8, 32, 8, 128, 32768, "bf16")
    splits = binding.sparse_decode_attention_splits(ok, 128)
    assert splits == 8  # two workgroups per CU: 512 / 64 rows
    # the per-split partials: rows x splits x G x (D + 2) floats
    assert binding.sparse_decode_attention_workspace_bytes(ok, 128, 0) == 64 * 8 * 4 * 130 * 4
    few = binding.make_shape(1, 64, 8, 128, 1 << 20, "bf16")  # 8 rows: capped at one block per wave
    assert binding.sparse_decode_attention_splits(few, 128) == 16
