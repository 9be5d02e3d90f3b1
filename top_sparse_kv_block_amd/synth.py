"""Seeded synthetic workloads for the sparse KV-cache decode step.

This module only draws inputs: keys, values, queries, draft queries, sequence
lengths and (for the host-tier workload) block selections.  It holds none of
the step's arithmetic (no scoring, no selection, no cache policy, no
attention), so both the HIP path and the CPU oracle can be fed from it.

Every tensor is drawn from its own NumPy ``PCG64`` stream whose seed sequence
is keyed by ``(workload seed, tensor id, layer, b, j-or-h)``, so any single row
can be regenerated on its own (the parity tests at full size rely on this).

Shapes of the workloads follow the pages' examples: a Llama-3.1-8B-shaped
layer (32 q-heads / 8 kv-heads, head_dim 128, 32K context; "KV Cache 塞不进 HBM 了",
intro), a 2048-token KV budget (OasisKV summary, experiments), a 512-token
budget (same), 16-token blocks (KV-Cache 压缩技术的工程原理, §5.2) and
adjacent-step selection overlap above 80% ("KV Cache 塞不进 HBM 了", §2.1).

Readings of what the pages leave open (all documented alongside the design):

* Heavy keys: a key at a heavy position gets ``3*sqrt(D)*(1+0.1*xi)`` times the
  unit direction of the group-mean step-0 query added to it, so heavy keys
  are about three typical key norms long, aligned to the query, and not tied.
* Query evolution: ``q_t = rho*q_{t-1} + sigma*eps_t``; the tiny workload uses
  rho=0.9, sigma=0.1 literally, the others the stationary AR(1) form
  rho=0.95, sigma=sqrt(1-rho^2).
* Drafts: ``draft_{t,i} = q_t + 0.2*i*eps_{t,i}`` for i = 1..n_drafts; only the
  drafts score, attention uses q_t.
* bf16 values are produced by round-to-nearest-even from float32.
"""

from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, replace

import numpy as np

# tensor ids used in seed-sequence spawn keys
_T_K, _T_V, _T_Q, _T_HEAVY, _T_DRAFT, _T_LEN, _T_SEL = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class Workload:
    """One synthetic workload (shape + input recipe)."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str  # "f32" | "bf16"
    ctx: int  # tokens per sequence
    budget: int  # KV budget in tokens per (sequence, kv-head) per step
    capacity: int  # working-set slots per (sequence, kv-head)
    steps: int
    scoring: str  # "blockmax" | "quest" | "given"
    n_drafts: int = 0  # 0: the current query scores; >0: that many drafts score
    draft_sigma: float = 0.2
    sink: int = 0  # tokens always kept at the start
    recent: int = 0  # tokens always kept at the end
    rho: float = 0.95
    sigma: float | None = None  # None -> sqrt(1 - rho^2)
    heavy: int = 0  # heavy keys per row (absolute count)
    heavy_frac: float = 0.0  # or a fraction of ctx (floor)
    seed: int = 0
    layers: int = 1
    block: int = 16
    ragged: bool = False  # draw seq_lens in [ctx/2, ctx] instead of all = ctx

    # derived -----------------------------------------------------------
    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def k_blocks(self) -> int:
        return self.budget // self.block

    @property
    def nb_max(self) -> int:
        return (self.ctx + self.block - 1) // self.block

    @property
    def rows(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def n_score_queries(self) -> int:
        return self.n_drafts if self.n_drafts > 0 else 1

    @property
    def q_sigma(self) -> float:
        return self.sigma if self.sigma is not None else math.sqrt(1.0 - self.rho * self.rho)

    @property
    def heavy_count(self) -> int:
        if self.heavy_frac > 0:
            return int(math.floor(self.heavy_frac * self.ctx))
        return min(self.heavy, self.ctx)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  "tiny" is the small case the oracle finishes in
# seconds; "llama8b_32k" is the throughput workload.
WORKLOADS = {
    "tiny": Workload(
        name="tiny", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, dtype="f32",
        ctx=1024, budget=128, capacity=16, steps=4, scoring="blockmax",
        rho=0.9, sigma=0.1, heavy=8, seed=1),
    "llama8b_32k": Workload(
        name="llama8b_32k", batch=8, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        ctx=32768, budget=2048, capacity=128, steps=32, scoring="blockmax",
        rho=0.95, heavy_frac=0.01, seed=2),
    "quest_128k": Workload(
        name="quest_128k", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        ctx=131072, budget=512, capacity=32, steps=16, scoring="quest",
        sink=4, recent=128, rho=0.95, heavy_frac=0.01, seed=3),
    "host_tier_32l": Workload(
        name="host_tier_32l", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
        ctx=131072, budget=2048, capacity=256, steps=8, scoring="given",
        rho=0.95, seed=4, layers=32),
    "lookahead_1m": Workload(
        name="lookahead_1m", batch=1, n_q_heads=64, n_kv_heads=8, head_dim=128, dtype="bf16",
        ctx=1048576, budget=2048, capacity=128, steps=8, scoring="blockmax",
        n_drafts=4, rho=0.95, heavy_frac=0.01, seed=5),
}


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key))))


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------- queries
def gen_queries(w: Workload, layer: int = 0):
    """Query chains.

    Returns ``(q, score_q)`` in the workload dtype (uint16 bits for bf16):
    ``q[steps, B, Hq, D]`` the attention queries, and
    ``score_q[steps, B, NQ, Hq, D]`` the vectors that score (q itself when
    there are no drafts, else the drafts).  Also returns the float64 step-0
    queries through ``gen_queries.q0`` semantics via :func:`_q_chain`.
    """
    q64, drafts64 = _q_chain(w, layer)
    q = _cast(q64, w.dtype)
    if w.n_drafts > 0:
        sq = _cast(drafts64, w.dtype)
    else:
        sq = q.reshape(w.steps, w.batch, 1, w.n_q_heads, w.head_dim).copy()
    return q, sq


def _q_chain(w: Workload, layer: int):
    S, B, H, D = w.steps, w.batch, w.n_q_heads, w.head_dim
    q = np.empty((S, B, H, D), dtype=np.float64)
    drafts = np.empty((S, B, max(w.n_drafts, 1), H, D), dtype=np.float64) if w.n_drafts else None
    for b in range(B):
        for h in range(H):
            r = _rng(w.seed, _T_Q, layer, b, h)
            q[0, b, h] = r.standard_normal(D)
            for t in range(1, S):
                q[t, b, h] = w.rho * q[t - 1, b, h] + w.q_sigma * r.standard_normal(D)
            if w.n_drafts:
                rd = _rng(w.seed, _T_DRAFT, layer, b, h)
                for t in range(S):
                    for i in range(1, w.n_drafts + 1):
                        drafts[t, b, i - 1, h] = q[t, b, h] + w.draft_sigma * i * rd.standard_normal(D)
    return q, drafts


# ---------------------------------------------------------------- keys/values
def _heavy_dir(w: Workload, q0: np.ndarray, b: int, j: int) -> np.ndarray:
    g = w.group
    m = q0[b, j * g:(j + 1) * g].mean(axis=0)
    n = np.linalg.norm(m)
    return m / n if n > 0 else m


def gen_kv_row(w: Workload, b: int, j: int, layer: int = 0, q0: np.ndarray | None = None):
    """K and V of one (sequence, kv-head) row, shape [ctx, D], workload dtype."""
    T, D = w.ctx, w.head_dim
    k = _rng(w.seed, _T_K, layer, b, j).standard_normal((T, D), dtype=np.float32)
    v = _rng(w.seed, _T_V, layer, b, j).standard_normal((T, D), dtype=np.float32)
    nh = w.heavy_count
    if nh > 0:
        if q0 is None:
            q0 = _q_chain(w.scaled(steps=1, n_drafts=0), layer)[0][0]
        u = _heavy_dir(w, q0, b, j).astype(np.float64)
        rh = _rng(w.seed, _T_HEAVY, layer, b, j)
        pos = rh.choice(T, size=nh, replace=False)
        xi = rh.standard_normal(nh)
        amp = 3.0 * math.sqrt(D) * (1.0 + 0.1 * xi)
        k[pos] = (k[pos].astype(np.float64) + amp[:, None] * u[None, :]).astype(np.float32)
    return _cast(k, w.dtype), _cast(v, w.dtype)


def gen_kv(w: Workload, layer: int = 0, out_k: np.ndarray | None = None, out_v: np.ndarray | None = None):
    """Full K and V, ``[B, Hkv, ctx, D]`` (float32, or uint16 bf16 bits)."""
    q0 = _q_chain(w.scaled(steps=1, n_drafts=0), layer)[0][0]
    npdt = np.float32 if w.dtype == "f32" else np.uint16
    shape = (w.batch, w.n_kv_heads, w.ctx, w.head_dim)
    K = out_k if out_k is not None else np.empty(shape, dtype=npdt)
    V = out_v if out_v is not None else np.empty(shape, dtype=npdt)

    def one(bj):
        b, j = bj
        K[b, j], V[b, j] = gen_kv_row(w, b, j, layer, q0)

    jobs = [(b, j) for b in range(w.batch) for j in range(w.n_kv_heads)]
    with _cf.ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, jobs))
    return K, V


def gen_seq_lens(w: Workload) -> np.ndarray:
    if not w.ragged:
        return np.full(w.batch, w.ctx, dtype=np.int32)
    r = _rng(w.seed, _T_LEN, 0, 0, 0)
    lo = max(1, w.ctx // 2)
    lens = r.integers(lo, w.ctx + 1, size=w.batch).astype(np.int32)
    lens[0] = w.ctx  # keep one full-length sequence
    return lens


# ---------------------------------------------------------------- selections
def gen_layer_selections(w: Workload, retain: float = 0.8):
    """Block selections for the host-tier workload (the indexer is not run).

    Per row: a shared chain X_s of k/2 blocks and, per layer, an own chain
    Y_{l,s} of k/2 blocks disjoint from X_s; each chain keeps ``retain`` of
    its blocks from one step to the next and refills uniformly from the
    blocks it does not hold.  Adjacent layers therefore share about half of
    their blocks and adjacent steps about ``retain`` of them.

    Returns int32 ``sel[steps, layers, B, Hkv, k]`` ascending per row.
    """
    k = w.k_blocks
    half = k // 2
    nb = w.nb_max
    out = np.empty((w.steps, w.layers, w.batch, w.n_kv_heads, k), dtype=np.int32)
    for b in range(w.batch):
        for j in range(w.n_kv_heads):
            r = _rng(w.seed, _T_SEL, 0, b, j)
            X = set(r.choice(nb, size=half, replace=False).tolist())
            Y = []
            for l in range(w.layers):
                pool = np.setdiff1d(np.arange(nb), np.fromiter(X, dtype=np.int64))
                Y.append(set(r.choice(pool, size=k - half, replace=False).tolist()))
            for s in range(w.steps):
                if s > 0:
                    X = _evolve(r, X, half, nb, set(), retain)
                for l in range(w.layers):
                    if s > 0:
                        Y[l] = _evolve(r, Y[l] - X, k - half, nb, X, retain)
                    else:
                        Y[l] = Y[l] - X
                        Y[l] = _refill(r, Y[l], k - half, nb, X)
                    sel = sorted(X | Y[l])
                    out[s, l, b, j] = np.asarray(sel, dtype=np.int32)
    return out


def _refill(r, keep: set, size: int, nb: int, avoid: set) -> set:
    keep = set(keep)
    while len(keep) < size:
        c = int(r.integers(0, nb))
        if c not in keep and c not in avoid:
            keep.add(c)
    return keep


def _evolve(r, cur: set, size: int, nb: int, avoid: set, retain: float) -> set:
    cur = sorted(cur)
    n_keep = min(len(cur), int(round(retain * size)))
    keep = set(r.choice(np.asarray(cur, dtype=np.int64), size=n_keep, replace=False).tolist()) if n_keep else set()
    return _refill(r, keep, size, nb, avoid)


def gen_workload(w: Workload, layer: int = 0):
    """Everything one layer of a workload needs, as NumPy arrays."""
    q, sq = gen_queries(w, layer)
    K, V = gen_kv(w, layer)
    return dict(q=q, score_q=sq, K=K, V=V, seq_lens=gen_seq_lens(w))
