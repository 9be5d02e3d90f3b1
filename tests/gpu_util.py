"""Helpers for the GPU parity tests (host <-> device copies, case logging).

Inputs come from ``top_sparse_kv_block_amd.synth`` (seeded) or plain NumPy
generators; expected values come only from the oracle.
"""
import sys

import numpy as np
import torch


def log(*parts):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *parts, file=sys.stderr, flush=True)


def dev(a: np.ndarray, dtype: str | None = None):
    """NumPy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    from top_sparse_kv_block_amd import synth
    return a.astype(np.float32) if dtype == "f32" else synth.f32_to_bf16_bits(a.astype(np.float32))


def max_rel_row_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over (b, h) of max|got - ref| / max|ref| (rows with ref == 0 use abs)."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    num = np.abs(got - ref).max(axis=1)
    return float(np.max(np.where(np.abs(ref).max(axis=1) > 0, num / den, num)))


def topk_swaps_ok(sel_gpu, cnt_gpu, sel_ora, cnt_ora, ora_scores, tol=1e-5, forced=None):
    """Sets equal except for blocks whose oracle score lies within tol of the
    oracle's k-th (lowest admitted non-forced) score."""
    bad = []
    rows = sel_gpu.reshape(-1, sel_gpu.shape[-1])
    rows_o = sel_ora.reshape(-1, sel_ora.shape[-1])
    cg, co = cnt_gpu.reshape(-1), cnt_ora.reshape(-1)
    sc = ora_scores.reshape(-1, ora_scores.shape[-1])
    for r in range(rows.shape[0]):
        if cg[r] != co[r]:
            bad.append((r, "count", int(cg[r]), int(co[r])))
            continue
        a, b = set(rows[r, :cg[r]].tolist()), set(rows_o[r, :co[r]].tolist())
        if a == b:
            continue
        f = forced[r] if forced is not None else set()
        kth = min(sc[r, i] for i in b - f) if b - f else -np.inf
        for blk in a ^ b:
            if abs(sc[r, blk] - kth) > tol:
                bad.append((r, blk, float(sc[r, blk]), float(kth)))
    return bad


def assert_lru_state(slot_block, slot_stamp, lru, msg=""):
    """The device slot table equals the oracle list's, and ordering each row's
    occupied slots by the device's (stamp, block id) gives the list's order
    (least recent first)."""
    rows, cap = lru.rows, lru.cap
    sb = np.asarray(slot_block).reshape(rows, cap)
    st = np.ascontiguousarray(slot_stamp).reshape(rows, cap).view(np.uint32)
    np.testing.assert_array_equal(sb, lru.slot_block(), err_msg=f"slot table {msg}")
    order = lru.order()
    for r in range(rows):
        occ = sorted((s for s in range(cap) if sb[r, s] >= 0), key=lambda s: (int(st[r, s]), int(sb[r, s])))
        assert occ == order[r][order[r] >= 0].tolist(), f"LRU order of row {r} {msg}"


def assert_lists(got: dict, out: dict, rows: int, k: int, msg=""):
    """Step lists (device arrays by name) equal the oracle's bit for bit."""
    for f in ("miss_count", "sel_slot", "sel_hit", "miss_block", "miss_slot"):
        shape = (rows,) if f == "miss_count" else (rows, k)
        np.testing.assert_array_equal(np.asarray(got[f]).reshape(shape), out[f], err_msg=f"{f} {msg}")
