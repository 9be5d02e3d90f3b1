"""Python binding of ``libsparse_kv.so`` (argument marshalling only).

Each function has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, checks dtype / device / contiguity,
passes raw pointers and torch's current HIP stream, and raises
:class:`SparseKVError` on a non-OK status.  Every step of the computation
runs in the library's kernels; there is no fallback of any kind: if the
library is not built, loading it raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SKV_LIBRARY may name another build of the same library (e.g. the A/B
# variant from ``build.py --ab-valu``); by default the in-tree build.
LIB_PATH = os.environ.get("SKV_LIBRARY") or os.path.join(_HERE, "libsparse_kv.so")

SKV_F32, SKV_BF16 = 0, 1
SKV_SCORE_BLOCKMAX, SKV_SCORE_QUEST = 0, 1
SKV_SRC_DEVICE, SKV_SRC_HOST_MAPPED = 0, 1

STATUS = {
    0: "SKV_OK", 1: "SKV_ERR_NULL", 2: "SKV_ERR_SHAPE", 3: "SKV_ERR_DTYPE", 4: "SKV_ERR_CAPACITY",
    5: "SKV_ERR_WORKSPACE", 6: "SKV_ERR_UNSUPPORTED", 7: "SKV_ERR_HIP", 8: "SKV_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 8 << 20  # SKV_NOALLOC_SCRATCH_BYTES

EXPORTS = (
    "sparse_kv_score", "sparse_kv_topk", "sparse_kv_cache_update", "sparse_decode_attention",
    "sparse_decode_attention_splits", "sparse_decode_attention_workspace_bytes", "sparse_kv_quest_meta",
    "sparse_kv_host_alloc", "sparse_kv_host_free", "sparse_kv_status_string", "sparse_kv_select_attend",
    "sparse_kv_select_attend_splits", "sparse_kv_cache_update_importance", "sparse_kv_append", "sparse_kv_select",
    "sparse_kv_select_attend_noalloc", "sparse_kv_stream_read", "sparse_kv_topk_workspace_bytes",
    "sparse_kv_workspace_bytes", "sparse_kv_check_state",
)


class SparseKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {status_string(status)}")


class skv_shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("block_size", C.c_int32), ("max_ctx", C.c_int32),
                ("dtype", C.c_int32)]


_lib = None
_p, _i32, _f32, _sz = C.c_void_p, C.c_int32, C.c_float, C.c_size_t


def load():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m top_sparse_kv_block_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = C.CDLL(LIB_PATH)
    S = C.POINTER(skv_shape)
    L.sparse_kv_score.argtypes = [S, _i32, _p, _i32, _p, _p, _f32, _p, _p]
    L.sparse_kv_topk.argtypes = [S, _p, _p, _i32, _i32, _i32, _p, _p, _p, _sz, _p]
    L.sparse_kv_cache_update.argtypes = [S, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p,
                                         _p]
    L.sparse_kv_cache_update_importance.argtypes = [S, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                                    _p, _i32, _p, _p, _p]
    L.sparse_kv_append.argtypes = [S, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _p]
    L.sparse_kv_select.argtypes = [S, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                   _i32, _p, _p, _p, _sz, _p]
    L.sparse_decode_attention.argtypes = [S, _p, _p, _p, _i32, _p, _p, _p, _p, _p, _i32, _f32, _i32, _p, _p, _i32, _p, _p,
                                          _p, _sz, _p]
    L.sparse_kv_select_attend.argtypes = [S, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                          _p, _p, _p, _p, _p, _i32, _f32, _i32, _p, _p, _p, _sz, _p]
    L.sparse_kv_select_attend_noalloc.argtypes = [S, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p,
                                                  _p, _p, _p, _p, _p, _p, _p, _i32, _f32, _i32, _p, _p, _p]
    L.sparse_kv_select_attend_splits.argtypes = [S, _i32]
    L.sparse_kv_select_attend_splits.restype = _i32
    L.sparse_decode_attention_splits.argtypes = [S, _i32]
    L.sparse_decode_attention_splits.restype = _i32
    L.sparse_decode_attention_workspace_bytes.argtypes = [S, _i32, _i32]
    L.sparse_decode_attention_workspace_bytes.restype = _sz
    L.sparse_kv_topk_workspace_bytes.argtypes = [S, _i32]
    L.sparse_kv_topk_workspace_bytes.restype = _sz
    L.sparse_kv_workspace_bytes.argtypes = [S, _i32, _i32]
    L.sparse_kv_workspace_bytes.restype = _sz
    L.sparse_kv_quest_meta.argtypes = [S, _p, _p, _p, _p]
    L.sparse_kv_stream_read.argtypes = [S, _p, _p, _p]
    L.sparse_kv_check_state.argtypes = [S, _i32, _p, _p, _p, _p, _p]
    L.sparse_kv_host_alloc.argtypes = [_sz, C.POINTER(_p), C.POINTER(_p)]
    L.sparse_kv_host_free.argtypes = [_p]
    L.sparse_kv_status_string.argtypes = [C.c_int]
    L.sparse_kv_status_string.restype = C.c_char_p
    for fn in ("sparse_kv_score", "sparse_kv_topk", "sparse_kv_cache_update", "sparse_decode_attention",
               "sparse_kv_quest_meta", "sparse_kv_host_alloc", "sparse_kv_host_free", "sparse_kv_select_attend",
               "sparse_kv_cache_update_importance", "sparse_kv_append", "sparse_kv_select",
               "sparse_kv_select_attend_noalloc", "sparse_kv_stream_read", "sparse_kv_check_state"):
        getattr(L, fn).restype = C.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().sparse_kv_status_string(int(status)).decode()


def make_shape(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, dtype, block_size=16) -> skv_shape:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return skv_shape(batch, n_q_heads, n_kv_heads, head_dim, block_size, max_ctx, code)


def dtype_code(dt) -> int:
    if dt in (torch.float32, "f32", "float32"):
        return SKV_F32
    if dt in (torch.bfloat16, "bf16", "bfloat16"):
        return SKV_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _torch_dtype(code: int):
    return torch.float32 if code == SKV_F32 else torch.bfloat16


def _ptr(t, dtype=None, name="tensor", allow_none=False, numel=None):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the shape needs {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn, rc):
    if rc != 0:
        raise SparseKVError(fn, rc)


def sparse_kv_score(shape, mode, q, n_queries, keys_or_meta, seq_lens, scale, scores, stream=None):
    dt = _torch_dtype(shape.dtype)
    b, hq, hkv, d, t = shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.max_ctx
    nb = t // 16
    kv_numel = b * hkv * t * d if mode == SKV_SCORE_BLOCKMAX else b * hkv * nb * 2 * d
    rc = load().sparse_kv_score(C.byref(shape), int(mode), _ptr(q, dt, "q", numel=b * n_queries * hq * d),
                                int(n_queries), _ptr(keys_or_meta, dt, "keys_or_meta", numel=kv_numel),
                                _ptr(seq_lens, torch.int32, "seq_lens", numel=b), float(scale),
                                _ptr(scores, torch.float32, "scores", numel=b * hkv * nb), _stream(stream))
    _check("sparse_kv_score", rc)


def _workspace(ws):
    # (pointer, bytes) of an optional workspace tensor (None: NULL, 0 bytes)
    if ws is None:
        return None, 0
    return _ptr(ws, None, "workspace"), ws.numel() * ws.element_size()


def sparse_kv_topk(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, sel_blocks, sel_count,
                   workspace=None, stream=None):
    """``workspace``: a device tensor of at least
    sparse_kv_topk_workspace_bytes(shape, k_blocks) bytes (None when that is 0)."""
    P = shape.batch * shape.n_kv_heads
    rc = load().sparse_kv_topk(C.byref(shape), _ptr(scores, torch.float32, "scores", numel=P * (shape.max_ctx // 16)),
                               _ptr(seq_lens, torch.int32, "seq_lens", numel=shape.batch), int(k_blocks),
                               int(sink_tokens), int(recent_tokens),
                               _ptr(sel_blocks, torch.int32, "sel_blocks", numel=P * k_blocks),
                               _ptr(sel_count, torch.int32, "sel_count", numel=P), *_workspace(workspace),
                               _stream(stream))
    _check("sparse_kv_topk", rc)


def sparse_kv_cache_update(shape, k_blocks, capacity, sel_blocks, sel_count, slot_block, slot_stamp, clock, sel_slot,
                           sel_hit, miss_block, miss_slot, miss_count, src_k=None, src_v=None,
                           src_kind=SKV_SRC_DEVICE, pool_k=None, pool_v=None, stream=None):
    """``src_k``/``src_v`` may be device tensors, or integer device addresses of
    mapped host memory (with ``src_kind=SKV_SRC_HOST_MAPPED``), or None (lists only)."""
    dt = _torch_dtype(shape.dtype)
    P, d, t = shape.batch * shape.n_kv_heads, shape.head_dim, shape.max_ctx
    pk, pc = P * k_blocks, P * capacity

    def src(x, name):
        if x is None or isinstance(x, int):
            return x
        return _ptr(x, dt, name, numel=P * t * d)

    rc = load().sparse_kv_cache_update(
        C.byref(shape), int(k_blocks), int(capacity), _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P), _ptr(slot_block, torch.int32, "slot_block", numel=pc),
        _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc), _ptr(clock, torch.int32, "clock", numel=P),
        _ptr(sel_slot, torch.int32, "sel_slot", numel=pk), _ptr(sel_hit, torch.uint8, "sel_hit", numel=pk),
        _ptr(miss_block, torch.int32, "miss_block", numel=pk), _ptr(miss_slot, torch.int32, "miss_slot", numel=pk),
        _ptr(miss_count, torch.int32, "miss_count", numel=P), src(src_k, "src_k"), src(src_v, "src_v"),
        int(src_kind), _ptr(pool_k, dt, "pool_k", allow_none=True, numel=pc * 16 * d),
        _ptr(pool_v, dt, "pool_v", allow_none=True, numel=pc * 16 * d), _stream(stream))
    _check("sparse_kv_cache_update", rc)


def sparse_kv_cache_update_importance(shape, k_blocks, capacity, sel_blocks, sel_count, scores, slot_block,
                                      slot_stamp, clock, sel_slot, sel_hit, miss_block, miss_slot, miss_count,
                                      src_k=None, src_v=None, src_kind=SKV_SRC_DEVICE, pool_k=None, pool_v=None,
                                      stream=None):
    """As sparse_kv_cache_update, evicting the least important unselected
    block (by this step's scores) instead of the least recently used."""
    dt = _torch_dtype(shape.dtype)
    P, d, t = shape.batch * shape.n_kv_heads, shape.head_dim, shape.max_ctx
    pk, pc = P * k_blocks, P * capacity

    def src(x, name):
        if x is None or isinstance(x, int):
            return x
        return _ptr(x, dt, name, numel=P * t * d)

    rc = load().sparse_kv_cache_update_importance(
        C.byref(shape), int(k_blocks), int(capacity), _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P),
        _ptr(scores, torch.float32, "scores", numel=P * (t // 16)),
        _ptr(slot_block, torch.int32, "slot_block", numel=pc),
        _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc), _ptr(clock, torch.int32, "clock", numel=P),
        _ptr(sel_slot, torch.int32, "sel_slot", numel=pk), _ptr(sel_hit, torch.uint8, "sel_hit", numel=pk),
        _ptr(miss_block, torch.int32, "miss_block", numel=pk), _ptr(miss_slot, torch.int32, "miss_slot", numel=pk),
        _ptr(miss_count, torch.int32, "miss_count", numel=P), src(src_k, "src_k"), src(src_v, "src_v"),
        int(src_kind), _ptr(pool_k, dt, "pool_k", allow_none=True, numel=pc * 16 * d),
        _ptr(pool_v, dt, "pool_v", allow_none=True, numel=pc * 16 * d), _stream(stream))
    _check("sparse_kv_cache_update_importance", rc)


def sparse_kv_select(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity, sel_blocks, sel_count,
                     slot_block, slot_stamp, clock, sel_slot, sel_hit, miss_block, miss_slot, miss_count, src_k=None,
                     src_v=None, src_kind=SKV_SRC_DEVICE, pool_k=None, pool_v=None, workspace=None, stream=None):
    """sparse_kv_topk then sparse_kv_cache_update (LRU) in one launch (two for
    rows over 16384 blocks), same results; ``workspace`` as for sparse_kv_topk."""
    dt = _torch_dtype(shape.dtype)
    P, d, t = shape.batch * shape.n_kv_heads, shape.head_dim, shape.max_ctx
    pk, pc = P * k_blocks, P * capacity

    def src(x, name):
        if x is None or isinstance(x, int):
            return x
        return _ptr(x, dt, name, numel=P * t * d)

    rc = load().sparse_kv_select(
        C.byref(shape), _ptr(scores, torch.float32, "scores", numel=P * (t // 16)),
        _ptr(seq_lens, torch.int32, "seq_lens", numel=shape.batch), int(k_blocks), int(sink_tokens),
        int(recent_tokens), int(capacity), _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P), _ptr(slot_block, torch.int32, "slot_block", numel=pc),
        _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc), _ptr(clock, torch.int32, "clock", numel=P),
        _ptr(sel_slot, torch.int32, "sel_slot", numel=pk), _ptr(sel_hit, torch.uint8, "sel_hit", numel=pk),
        _ptr(miss_block, torch.int32, "miss_block", numel=pk), _ptr(miss_slot, torch.int32, "miss_slot", numel=pk),
        _ptr(miss_count, torch.int32, "miss_count", numel=P), src(src_k, "src_k"), src(src_v, "src_v"),
        int(src_kind), _ptr(pool_k, dt, "pool_k", allow_none=True, numel=pc * 16 * d),
        _ptr(pool_v, dt, "pool_v", allow_none=True, numel=pc * 16 * d), *_workspace(workspace), _stream(stream))
    _check("sparse_kv_select", rc)


def sparse_kv_append(shape, new_k, new_v, seq_lens, keys, values, meta=None, slot_block=None, capacity=0,
                     pool_k=None, pool_v=None, stream=None):
    """Store one new token per sequence at seq_lens[b] (which grows by one on
    the device), keep the Quest boxes exact and refresh resident pool slots."""
    dt = _torch_dtype(shape.dtype)
    b, hkv, d, t = shape.batch, shape.n_kv_heads, shape.head_dim, shape.max_ctx
    P = b * hkv
    rc = load().sparse_kv_append(
        C.byref(shape), _ptr(new_k, dt, "new_k", numel=P * d), _ptr(new_v, dt, "new_v", numel=P * d),
        _ptr(seq_lens, torch.int32, "seq_lens", numel=b), _ptr(keys, dt, "keys", numel=P * t * d),
        _ptr(values, dt, "values", numel=P * t * d),
        _ptr(meta, dt, "meta", allow_none=True, numel=P * (t // 16) * 2 * d),
        _ptr(slot_block, torch.int32, "slot_block", allow_none=True, numel=P * int(capacity)), int(capacity),
        _ptr(pool_k, dt, "pool_k", allow_none=True, numel=P * int(capacity) * 16 * d),
        _ptr(pool_v, dt, "pool_v", allow_none=True, numel=P * int(capacity) * 16 * d), _stream(stream))
    _check("sparse_kv_append", rc)


def sparse_decode_attention(shape, q, pool_k, pool_v, capacity, sel_blocks, sel_slot, sel_hit, sel_count, seq_lens,
                            k_blocks, scale, num_splits, src_k, src_v, src_kind, out, lse, workspace, stream=None):
    """``src_k``/``src_v`` (device tensors, integer addresses of mapped host
    memory, or None) turn on fetch-on-attend for the blocks with sel_hit == 0."""
    dt = _torch_dtype(shape.dtype)
    b, hq, d, t = shape.batch, shape.n_q_heads, shape.head_dim, shape.max_ctx
    P = b * shape.n_kv_heads
    pk, pc = P * k_blocks, P * capacity

    def src(x, name):
        if x is None or isinstance(x, int):
            return x
        return _ptr(x, dt, name, numel=P * t * d)

    rc = load().sparse_decode_attention(
        C.byref(shape), _ptr(q, dt, "q", numel=b * hq * d), _ptr(pool_k, dt, "pool_k", numel=pc * 16 * d),
        _ptr(pool_v, dt, "pool_v", numel=pc * 16 * d), int(capacity),
        _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk), _ptr(sel_slot, torch.int32, "sel_slot", numel=pk),
        _ptr(sel_hit, torch.uint8, "sel_hit", allow_none=True, numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P), _ptr(seq_lens, torch.int32, "seq_lens", numel=b),
        int(k_blocks), float(scale), int(num_splits), src(src_k, "src_k"), src(src_v, "src_v"), int(src_kind),
        _ptr(out, torch.float32, "out", numel=b * hq * d), _ptr(lse, torch.float32, "lse", allow_none=True, numel=b * hq),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("sparse_decode_attention", rc)


def sparse_kv_select_attend(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity, sel_blocks,
                            sel_count, slot_block, slot_stamp, clock, sel_slot, sel_hit, miss_block, miss_slot,
                            miss_count, q, pool_k, pool_v, src_k, src_v, src_kind, scale, num_splits, out, lse,
                            workspace, stream=None):
    """Top-k + working-set update + attention with fetch-on-attend in one call."""
    dt = _torch_dtype(shape.dtype)
    b, hq, d, t = shape.batch, shape.n_q_heads, shape.head_dim, shape.max_ctx
    P = b * shape.n_kv_heads
    pk, pc = P * k_blocks, P * capacity

    def src(x, name):
        if isinstance(x, int):
            return x
        return _ptr(x, dt, name, numel=P * t * d)

    rc = load().sparse_kv_select_attend(
        C.byref(shape), _ptr(scores, torch.float32, "scores", numel=P * (t // 16)),
        _ptr(seq_lens, torch.int32, "seq_lens", numel=b), int(k_blocks), int(sink_tokens), int(recent_tokens),
        int(capacity), _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P), _ptr(slot_block, torch.int32, "slot_block", numel=pc),
        _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc), _ptr(clock, torch.int32, "clock", numel=P),
        _ptr(sel_slot, torch.int32, "sel_slot", numel=pk), _ptr(sel_hit, torch.uint8, "sel_hit", numel=pk),
        _ptr(miss_block, torch.int32, "miss_block", numel=pk), _ptr(miss_slot, torch.int32, "miss_slot", numel=pk),
        _ptr(miss_count, torch.int32, "miss_count", numel=P), _ptr(q, dt, "q", numel=b * hq * d),
        _ptr(pool_k, dt, "pool_k", numel=pc * 16 * d), _ptr(pool_v, dt, "pool_v", numel=pc * 16 * d),
        src(src_k, "src_k"), src(src_v, "src_v"), int(src_kind), float(scale), int(num_splits),
        _ptr(out, torch.float32, "out", numel=b * hq * d), _ptr(lse, torch.float32, "lse", allow_none=True, numel=b * hq),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("sparse_kv_select_attend", rc)


def sparse_kv_select_attend_noalloc(shape, scores, seq_lens, k_blocks, sink_tokens, recent_tokens, capacity,
                                    sel_blocks, sel_count, slot_block, slot_stamp, clock, sel_slot, sel_hit,
                                    miss_block, miss_slot, miss_count, q, pool_k, pool_v, src_k, src_v, src_kind,
                                    scale, num_splits, out, lse, stream=None):
    """sparse_kv_select_attend with the partials in the library's static
    device scratch: no workspace argument and no allocation."""
    dt = _torch_dtype(shape.dtype)
    b, hq, d, t = shape.batch, shape.n_q_heads, shape.head_dim, shape.max_ctx
    P = b * shape.n_kv_heads
    pk, pc = P * k_blocks, P * capacity
    rc = load().sparse_kv_select_attend_noalloc(
        C.byref(shape), _ptr(scores, torch.float32, "scores", numel=P * (t // 16)),
        _ptr(seq_lens, torch.int32, "seq_lens", numel=b), int(k_blocks), int(sink_tokens), int(recent_tokens),
        int(capacity), _ptr(sel_blocks, torch.int32, "sel_blocks", numel=pk),
        _ptr(sel_count, torch.int32, "sel_count", numel=P), _ptr(slot_block, torch.int32, "slot_block", numel=pc),
        _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc), _ptr(clock, torch.int32, "clock", numel=P),
        _ptr(sel_slot, torch.int32, "sel_slot", numel=pk), _ptr(sel_hit, torch.uint8, "sel_hit", numel=pk),
        _ptr(miss_block, torch.int32, "miss_block", numel=pk), _ptr(miss_slot, torch.int32, "miss_slot", numel=pk),
        _ptr(miss_count, torch.int32, "miss_count", numel=P), _ptr(q, dt, "q", numel=b * hq * d),
        _ptr(pool_k, dt, "pool_k", numel=pc * 16 * d), _ptr(pool_v, dt, "pool_v", numel=pc * 16 * d),
        _ptr(src_k, dt, "src_k", numel=P * t * d), _ptr(src_v, dt, "src_v", numel=P * t * d), int(src_kind),
        float(scale), int(num_splits), _ptr(out, torch.float32, "out", numel=b * hq * d),
        _ptr(lse, torch.float32, "lse", allow_none=True, numel=b * hq), _stream(stream))
    _check("sparse_kv_select_attend_noalloc", rc)


def sparse_decode_attention_splits(shape, k_blocks) -> int:
    return int(load().sparse_decode_attention_splits(C.byref(shape), int(k_blocks)))


def sparse_kv_select_attend_splits(shape, k_blocks) -> int:
    return int(load().sparse_kv_select_attend_splits(C.byref(shape), int(k_blocks)))


def sparse_decode_attention_workspace_bytes(shape, k_blocks, num_splits) -> int:
    return int(load().sparse_decode_attention_workspace_bytes(C.byref(shape), int(k_blocks), int(num_splits)))


def sparse_kv_topk_workspace_bytes(shape, k_blocks) -> int:
    return int(load().sparse_kv_topk_workspace_bytes(C.byref(shape), int(k_blocks)))


def sparse_kv_workspace_bytes(shape, k_blocks, num_splits=0) -> int:
    return int(load().sparse_kv_workspace_bytes(C.byref(shape), int(k_blocks), int(num_splits)))


def sparse_kv_quest_meta(shape, keys, seq_lens, meta, stream=None):
    dt = _torch_dtype(shape.dtype)
    P, d, t = shape.batch * shape.n_kv_heads, shape.head_dim, shape.max_ctx
    rc = load().sparse_kv_quest_meta(C.byref(shape), _ptr(keys, dt, "keys", numel=P * t * d),
                                     _ptr(seq_lens, torch.int32, "seq_lens", numel=shape.batch),
                                     _ptr(meta, dt, "meta", numel=P * (t // 16) * 2 * d), _stream(stream))
    _check("sparse_kv_quest_meta", rc)


def sparse_kv_check_state(shape, capacity, slot_block, slot_stamp, clock, flags, stream=None):
    """Per-row consistency flags of a working-set state into ``flags``
    [B, Hkv] int32 (1 id out of range, 2 block in two slots, 4 stamp ahead of
    the clock)."""
    P, pc = shape.batch * shape.n_kv_heads, shape.batch * shape.n_kv_heads * int(capacity)
    rc = load().sparse_kv_check_state(C.byref(shape), int(capacity),
                                      _ptr(slot_block, torch.int32, "slot_block", numel=pc),
                                      _ptr(slot_stamp, torch.int32, "slot_stamp", numel=pc),
                                      _ptr(clock, torch.int32, "clock", numel=P),
                                      _ptr(flags, torch.int32, "flags", numel=P), _stream(stream))
    _check("sparse_kv_check_state", rc)


def sparse_kv_stream_read(shape, keys, sink, stream=None):
    """Measurement helper: one read of ``keys`` in the block scan's load form."""
    dt = _torch_dtype(shape.dtype)
    P, d, t = shape.batch * shape.n_kv_heads, shape.head_dim, shape.max_ctx
    rc = load().sparse_kv_stream_read(C.byref(shape), _ptr(keys, dt, "keys", numel=P * t * d),
                                      _ptr(sink, torch.int32, "sink", numel=1), _stream(stream))
    _check("sparse_kv_stream_read", rc)


class HostBuffer:
    """Pinned, device-mapped host memory from ``sparse_kv_host_alloc``."""

    def __init__(self, nbytes: int):
        h, d = C.c_void_p(), C.c_void_p()
        rc = load().sparse_kv_host_alloc(int(nbytes), C.byref(h), C.byref(d))
        _check("sparse_kv_host_alloc", rc)
        self.nbytes, self.host_ptr, self.device_ptr = int(nbytes), h.value, d.value

    def numpy(self, dtype, shape):
        import numpy as np
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        assert n <= self.nbytes
        buf = (C.c_char * n).from_address(self.host_ptr)
        return np.frombuffer(buf, dtype=dtype).reshape(shape)

    def free(self):
        if self.host_ptr:
            _check("sparse_kv_host_free", load().sparse_kv_host_free(self.host_ptr))
            self.host_ptr = self.device_ptr = None
