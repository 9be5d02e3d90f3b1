"""Host-side argument validation of every C entry point (CPU only).

Each call below is invalid in exactly one way and must return the status the
header documents for it before anything is launched; the pointers are
non-NULL placeholders that are never dereferenced.  Without a GPU a call that
got past validation reports SKV_ERR_HIP instead, so a wrong status here means
a check is missing or misordered.
"""
import ctypes as C

import pytest
import torch

from top_sparse_kv_block_amd import binding as B

# placeholder pointers must never reach a launch: where a GPU is visible a
# missing check would turn into a memory fault, so these run on the CPU only
pytestmark = pytest.mark.skipif(torch.cuda.is_available(), reason="host-side checks with placeholder pointers")

P = C.c_void_p(0x1000)  # placeholder device pointer
NUL = None
OK, NULL, SHAPE, DTYPE, CAPACITY, WORKSPACE, UNSUPPORTED = 0, 1, 2, 3, 4, 5, 6


def shape(batch=2, hq=8, hkv=2, d=64, ctx=1024, dtype="f32", block=16):
    return C.byref(B.make_shape(batch, hq, hkv, d, ctx, dtype, block_size=block))


@pytest.fixture(scope="module")
def L():
    return B.load()


def score(L, s=None, mode=0, q=P, nq=1, keys=P, lens=P, out=P):
    return L.sparse_kv_score(s if s is not None else shape(), mode, q, nq, keys, lens, 0.1, out, NUL)


def test_shape_checks(L):
    assert L.sparse_kv_score(None, 0, P, 1, P, P, 0.1, P, NUL) == NULL
    bad_dtype = B.make_shape(2, 8, 2, 64, 1024, "f32")
    bad_dtype.dtype = 7
    assert score(L, C.byref(bad_dtype)) == DTYPE
    assert score(L, shape(hq=8, hkv=3)) == SHAPE      # Hq % Hkv != 0
    assert score(L, shape(d=96)) == SHAPE             # head_dim 64 or 128
    assert score(L, shape(block=32)) == SHAPE         # 16-token blocks only
    assert score(L, shape(ctx=1000)) == SHAPE         # T a multiple of 16
    assert score(L, shape(batch=0)) == SHAPE


def test_score(L):
    assert score(L, q=NUL) == NULL
    assert score(L, out=NUL) == NULL
    assert score(L, nq=0) == SHAPE
    assert score(L, nq=5) == SHAPE
    assert score(L, shape(hq=32, hkv=2), nq=4) == SHAPE  # 64 query rows per kv head > 32
    assert score(L, mode=9) == UNSUPPORTED


def topk(L, s=None, scores=P, k=8, sink=0, recent=0, ws=NUL, ws_bytes=0):
    return L.sparse_kv_topk(s if s is not None else shape(), scores, P, k, sink, recent, P, P, ws, ws_bytes, NUL)


def test_topk(L):
    assert topk(L, scores=NUL) == NULL
    assert topk(L, k=0) == SHAPE
    assert topk(L, k=65) == SHAPE                    # k > NB (64 blocks)
    assert topk(L, shape(ctx=16 * 4096), k=1025) == SHAPE  # k > 1024
    assert topk(L, sink=-1) == SHAPE
    assert topk(L, k=8, sink=64, recent=64) == CAPACITY  # 4 + 4 + 1 forced blocks > 8
    assert topk(L, shape(ctx=16 * 65537)) == UNSUPPORTED  # rows over 65536 blocks
    # rows over 16384 blocks need the workspace: missing, short, misaligned
    long = shape(ctx=16 * 16385)
    need = B.sparse_kv_topk_workspace_bytes(B.make_shape(2, 8, 2, 64, 16 * 16385, "f32"), 8)
    assert need == 4 * 17 * 8 * 8  # 4 rows, 17 chunks of 1024 blocks, 8 (score, id) pairs each
    assert topk(L, long) == WORKSPACE
    assert topk(L, long, ws=P, ws_bytes=need - 1) == WORKSPACE
    assert topk(L, long, ws=C.c_void_p(0x1010), ws_bytes=need) == WORKSPACE


def update(L, k=8, cap=16, src=(NUL, NUL), kind=0, pool=(P, P), sel=P, fn="sparse_kv_cache_update", s=None):
    args = [s if s is not None else shape(), k, cap, sel, P]
    if fn == "sparse_kv_cache_update_importance":
        args.append(P)
    args += [P, P, P, P, P, P, P, P, src[0], src[1], kind, pool[0], pool[1], NUL]
    return getattr(L, fn)(*args)


@pytest.mark.parametrize("fn", ["sparse_kv_cache_update", "sparse_kv_cache_update_importance"])
def test_cache_update(L, fn):
    assert update(L, sel=NUL, fn=fn) == NULL
    assert update(L, k=0, fn=fn) == SHAPE
    assert update(L, k=16, cap=8, fn=fn) == CAPACITY
    assert update(L, cap=1025, fn=fn) == UNSUPPORTED
    assert update(L, kind=3, fn=fn) == SHAPE
    assert update(L, src=(P, NUL), fn=fn) == NULL      # K without V
    assert update(L, src=(P, P), pool=(NUL, P), fn=fn) == NULL  # fetch needs the pool
    assert update(L, fn=fn, s=shape(ctx=16 * (2 ** 21 + 1))) == UNSUPPORTED  # block ids past 21 bits


def test_importance_needs_scores(L):
    args = [shape(), 8, 16, P, P, NUL] + [P] * 8 + [NUL, NUL, 0, P, P, NUL]
    assert L.sparse_kv_cache_update_importance(*args) == NULL


def select(L, s=None, k=8, cap=16, sink=0, recent=0, kind=0, src=(NUL, NUL), scores=P, ws=NUL, ws_bytes=0):
    return L.sparse_kv_select(s if s is not None else shape(), scores, P, k, sink, recent, cap, P, P, P, P, P, P, P,
                              P, P, P, src[0], src[1], kind, P, P, ws, ws_bytes, NUL)


def test_select(L):
    assert select(L, scores=NUL) == NULL
    assert select(L, k=0) == SHAPE
    assert select(L, k=16, cap=8) == CAPACITY
    assert select(L, cap=1025) == UNSUPPORTED
    assert select(L, sink=64, recent=64) == CAPACITY
    assert select(L, kind=2) == SHAPE
    assert select(L, src=(NUL, P)) == NULL
    assert select(L, shape(ctx=16 * 65537)) == UNSUPPORTED
    assert select(L, shape(ctx=16 * 40000)) == WORKSPACE
    assert select(L, shape(ctx=16 * 40000), ws=P, ws_bytes=8) == WORKSPACE


def attention(L, s=None, k=8, cap=16, splits=0, src=(NUL, NUL), hit=P, ws=P, ws_bytes=1 << 20, kind=0):
    return L.sparse_decode_attention(s if s is not None else shape(), P, P, P, cap, P, P, hit, P, P, k, 0.1, splits,
                                     src[0], src[1], kind, P, P, ws, ws_bytes, NUL)


def test_attention(L):
    assert attention(L, k=0) == SHAPE
    assert attention(L, splits=9) == SHAPE            # more splits than blocks
    assert attention(L, k=200, splits=129) == SHAPE   # more than 128 splits
    assert attention(L, kind=5) == SHAPE
    assert attention(L, src=(P, P), hit=NUL) == NULL  # fetch on attend needs the hit flags
    assert attention(L, shape(hq=34, hkv=2)) == UNSUPPORTED  # group of 17 heads
    assert attention(L, ws=NUL) == WORKSPACE
    assert attention(L, ws=C.c_void_p(0x1004)) == WORKSPACE  # not 256-byte aligned
    assert attention(L, splits=4, ws_bytes=16) == WORKSPACE


def test_select_attend(L):
    def call(s=None, k=8, cap=16, src=(P, P), splits=0, ws_bytes=1 << 20):
        return L.sparse_kv_select_attend(s if s is not None else shape(), P, P, k, 0, 0, cap, P, P, P, P, P, P, P,
                                         P, P, P, P, P, P, src[0], src[1], 0, 0.1, splits, P, P, P, ws_bytes, NUL)
    assert call(src=(NUL, NUL)) == NULL                # the fused call always fetches on attend
    assert call(shape(ctx=16 * 65537)) == UNSUPPORTED  # rows over 65536 blocks
    # past 16384 blocks the workspace also holds the top-k's chunk candidates
    long = B.make_shape(2, 8, 2, 64, 16 * 20000, "f32")
    att = B.sparse_decode_attention_workspace_bytes(long, 8, 4)
    tk = B.sparse_kv_topk_workspace_bytes(long, 8)
    assert tk > 0
    assert call(C.byref(long), splits=4, ws_bytes=att) == WORKSPACE
    assert call(C.byref(long), splits=4, ws_bytes=att + tk - 1) == WORKSPACE
    assert call(k=16, cap=8) == CAPACITY
    assert call(splits=9) == SHAPE
    assert call(splits=4, ws_bytes=16) == WORKSPACE


def test_append(L):
    def call(new_k=P, sb=NUL, cap=0, pool=(NUL, NUL)):
        return L.sparse_kv_append(shape(), new_k, P, P, P, P, NUL, sb, cap, pool[0], pool[1], NUL)
    assert call(new_k=NUL) == NULL
    assert call(sb=P, cap=4) == NULL                   # a slot table needs the pool
    assert call(sb=P, cap=0, pool=(P, P)) == SHAPE
    assert call(sb=P, cap=1025, pool=(P, P)) == UNSUPPORTED


def test_helpers(L):
    assert L.sparse_kv_quest_meta(shape(), P, P, NUL, NUL) == NULL
    assert L.sparse_kv_host_free(NUL) == NULL
    h, d = C.c_void_p(), C.c_void_p()
    assert L.sparse_kv_host_alloc(0, C.byref(h), C.byref(d)) == SHAPE
    assert L.sparse_kv_host_alloc(16, None, C.byref(d)) == NULL
    assert L.sparse_decode_attention_workspace_bytes(shape(), 8, 9) == 0
    assert L.sparse_decode_attention_splits(shape(hq=8, hkv=3), 8) == 0
    assert L.sparse_kv_select_attend_splits(shape(), 0) == 0


def test_workspace_sizes():
    s = B.make_shape(1, 64, 8, 128, 1 << 20, "bf16")  # 8 rows of 65536 blocks
    # chunks of 1024, 2048 or 4096 blocks: the smallest giving at most 4096
    # candidates (chunks x k rounded up to 4), else at most 16384
    assert B.sparse_kv_topk_workspace_bytes(s, 128) == 8 * 32 * 128 * 8   # 2048-block chunks
    assert B.sparse_kv_topk_workspace_bytes(s, 1024) == 8 * 16 * 1024 * 8  # 4096: 16384 candidates
    assert B.sparse_kv_topk_workspace_bytes(s, 256) == 8 * 16 * 256 * 8   # 4096: exactly 4096
    assert B.sparse_kv_topk_workspace_bytes(s, 257) == 8 * 32 * 260 * 8  # 2048: stride 260, 8320 candidates
    short = B.make_shape(8, 32, 8, 128, 32768, "bf16")
    assert B.sparse_kv_topk_workspace_bytes(short, 128) == 0
    assert B.sparse_kv_topk_workspace_bytes(short, 0) == 0  # invalid
    # one size for every call of the step: the largest of the three
    for sh, k in ((s, 128), (short, 128), (s, 1024)):
        one = B.sparse_kv_workspace_bytes(sh, k, 0)
        assert one >= B.sparse_kv_topk_workspace_bytes(sh, k)
        assert one >= B.sparse_decode_attention_workspace_bytes(sh, k, B.sparse_decode_attention_splits(sh, k))
        assert one >= B.sparse_decode_attention_workspace_bytes(sh, k, B.sparse_kv_select_attend_splits(sh, k))
    assert B.sparse_kv_workspace_bytes(short, 128, 0) == max(
        B.sparse_decode_attention_workspace_bytes(short, 128, 0),
        B.sparse_decode_attention_workspace_bytes(short, 128, B.sparse_kv_select_attend_splits(short, 128)))
    assert B.sparse_kv_workspace_bytes(short, 128, 200) == 0  # more splits than blocks


def test_check_state(L):
    def call(s=None, cap=16, sb=P, flags=P):
        return L.sparse_kv_check_state(s if s is not None else shape(), cap, sb, P, P, flags, NUL)
    assert call(sb=NUL) == NULL
    assert call(flags=NUL) == NULL
    assert call(cap=0) == SHAPE
    assert call(cap=1025) == UNSUPPORTED
