#!/usr/bin/env python3
"""Benchmark of the sparse KV-cache decode step on one MI355X.

A step is one pass of the whole path for one attention layer over one batch:
block scoring -> top-k under the budget -> working-set update -> split-K GQA
attention that also fetches the step's misses into the pool.  By default
stages 2-4 run as the library's fused select-attend call (same results as
the three separate calls; --four-calls runs those instead).  The default
workload is the Llama-3.1-8B-shaped layer: batch 8, 32 q-heads / 8 kv-heads,
head_dim 128, bf16 K/V, 32768-token context in 16-token blocks, a
2048-token budget (128 blocks) and a 128-slot working set per (sequence,
kv-head).  Inputs are seeded synthetic tensors of that shape, resident in
HBM before timing starts; queries follow an AR(1) chain so consecutive
steps overlap (>80%) the way the method expects.

Output: one JSON line with steps/s (value), ms per step, achieved
algorithmic HBM GB/s for the whole step, the roofline of the dominant
kernel (the block-scoring scan) and a per-call breakdown, both timed with
HIP events on the stream the kernels run on during a second pass of the
same steps right after the timed region (event markers inside the timed
region would add queue gaps to it), the host-tier miss fetch over PCIe
(``host_fetch``: full K/V in pinned host memory, host->device GB/s of the
misses beside a plain pinned copy; never part of ``value``), and the
oracle's throughput on the host cores on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
METRIC = "sparse decode steps/s + achieved HBM GB/s (32K ctx, 2048-token budget)"
KERNEL_SOURCES = {
    "score": ("top_sparse_kv_block_amd/csrc/score.hip", "top_sparse_kv_block_amd/csrc/skv_device.h"),
    "select_attend": ("top_sparse_kv_block_amd/csrc/attention.hip", "top_sparse_kv_block_amd/csrc/skv_rowops.h",
                      "top_sparse_kv_block_amd/csrc/skv_device.h"),
    "merge_commit": ("top_sparse_kv_block_amd/csrc/attention.hip", "top_sparse_kv_block_amd/csrc/skv_device.h"),
    "topk_chunk": ("top_sparse_kv_block_amd/csrc/topk.hip", "top_sparse_kv_block_amd/csrc/skv_rowops.h",
                   "top_sparse_kv_block_amd/csrc/skv_device.h"),
}
KERNEL_NAMES = {"score": "score_blockmax", "select_attend": "select_attend_kernel",
                "merge_commit": "merge_commit_kernel"}
LONG_ROW_BLOCKS = 16384  # rows past this run the top-k's chunk launch before the fused kernel


def traffic_file(workload: str) -> str:
    """The counter-traffic summary of a workload's step (JSON; a markdown twin beside it)."""
    return os.path.join(ROOT, "profiles", f"{workload}_step_traffic.json")


# ---------------------------------------------------------------- byte model
def kv_cache_bytes(seq_len, layers, kv_heads, head_dim, bytes_per_elem):
    """KV-cache size: 2 (K and V) * L * layers * kv_heads * head_dim * bytes."""
    return 2 * seq_len * layers * kv_heads * head_dim * bytes_per_elem


def step_bytes(w, misses: float) -> dict:
    """Algorithmic HBM bytes of one step (what the method must move).

    score scan: every key of every row once (P*T*D*e); Quest reads the
    per-block min/max instead (P*NB*2*D*e); scoring queries; scores written.
    top-k: scores read, selection written.  attention: every selected
    block's K and V read once per kv group (from the pool for hits, from the
    source for misses), q read, output and lse written.  fetch: each miss's
    K and V block written into its pool slot.  Small state arrays (slot
    tables, lists) are left out (<0.1%).
    """
    P, e, D, T = w.rows, w.elem_bytes, w.head_dim, w.ctx
    nb, k = w.nb_max, w.k_blocks
    blk = 16 * D * e
    scan = P * nb * 2 * D * e if w.scoring == "quest" else P * T * D * e
    score_q = w.batch * w.n_score_queries * w.n_q_heads * D * e
    scores = P * nb * 4
    topk = P * nb * 4 + P * k * 4
    fetch = misses * blk * 2
    attn = P * k * blk * 2 + w.batch * w.n_q_heads * D * e + w.batch * w.n_q_heads * (D + 1) * 4
    return dict(score=scan + score_q + scores, topk=topk, fetch=fetch, attention=attn,
                total=scan + score_q + scores + topk + fetch + attn)


def score_launch_bytes(w) -> int:
    """Bytes one scoring launch must move: per block 16*D*e of keys (the
    Quest bound: its 2*D*e min/max box) plus its 4-byte score, times P*NB
    blocks, plus the scoring queries."""
    per_block = (2 if w.scoring == "quest" else 16) * w.head_dim * w.elem_bytes + 4
    return w.rows * w.nb_max * per_block + w.batch * w.n_score_queries * w.n_q_heads * w.head_dim * w.elem_bytes


def _score_kernel_name(w) -> str:
    """The scoring kernel the library runs for this workload's scoring mode and dtype."""
    if w.scoring == "quest":
        return "score_quest_mfma_kernel" if w.dtype == "bf16" else "score_quest_kernel"
    return "score_blockmax_mfma_kernel" if w.dtype == "bf16" else "score_blockmax_kernel"


def chunk_candidate_bytes(w) -> int:
    """Bytes of the chunk candidates of rows past LONG_ROW_BLOCKS blocks
    ((score, id) pairs; the library's top-k workspace size), else 0."""
    if w.nb_max <= LONG_ROW_BLOCKS:
        return 0
    from top_sparse_kv_block_amd import binding as B
    shape = B.make_shape(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype)
    return int(B.sparse_kv_topk_workspace_bytes(shape, w.k_blocks))


def fused_launch_bytes(w, misses: float, splits: int) -> int:
    """Algorithmic bytes of one select-attend launch: the row's scores (past
    LONG_ROW_BLOCKS blocks: its chunk candidates) and slot table (with
    stamps) read once, every selected block's K and V read once (hits from
    the pool, misses from the source), each miss written into its pool
    slot, q read, the split partials and the step's lists written."""
    P, e, D, G = w.rows, w.elem_bytes, w.head_dim, w.group
    blk = 16 * D * e
    sel_in = chunk_candidate_bytes(w) or P * w.nb_max * 4
    return int(sel_in + P * w.capacity * 8 + P * w.k_blocks * blk * 2 + misses * blk * 2
               + w.batch * w.n_q_heads * D * e + P * splits * G * (D + 2) * 4 + P * w.k_blocks * 17 + P * 8)


def chunk_launch_bytes(w) -> int:
    """Algorithmic bytes of the top-k's chunk launch: every score read once,
    the chunk candidates written."""
    return int(w.rows * w.nb_max * 4 + chunk_candidate_bytes(w))


def merge_launch_bytes(w, splits: int) -> int:
    """Algorithmic bytes of one merge-commit launch: the partials read, the
    output and lse written, the selection and its slots read, the selected
    slots' blocks and stamps and the clock written."""
    P, D, G = w.rows, w.head_dim, w.group
    return int(P * splits * G * (D + 2) * 4 + w.batch * w.n_q_heads * (D + 1) * 4 + P * w.k_blocks * 16
               + P * 12)


def _sources_sha(kernel: str = "score") -> str:
    """Hash of the kernel's source files without their // comments and blank
    lines, so that counters taken on a kernel stay valid across edits of its
    comments (no counted code changes) and expire with any code change."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def _kernel_names(w) -> dict:
    """Kernel-name patterns of the step's counted kernels: the scan of this
    workload's scoring mode, the fused select-attend, the merge, and (rows
    past LONG_ROW_BLOCKS blocks) the top-k's chunk launch."""
    names = dict(KERNEL_NAMES, score="score_quest" if w.scoring == "quest" else "score_blockmax")
    if w.nb_max > LONG_ROW_BLOCKS:
        names["topk_chunk"] = "topk_chunk_kernel"
    return names


def _traffic(w):
    """Counter-derived HBM bytes per scoring launch, if the counters were
    taken on the current kernel source; else None."""
    try:
        with open(traffic_file(w.name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    k = t.get("kernels", {}).get("score", {})
    if k.get("source_sha") != _sources_sha("score") or t.get("workload") != w.name:
        return None
    return k.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (as lscpu shows it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def input_sha256(data) -> dict:
    """SHA-256 of every generated input tensor (its raw bytes, C order)."""
    return {name: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
            for name, a in sorted(data.items()) if isinstance(a, np.ndarray)}


# ---------------------------------------------------------------- oracle leg
def cpu_baseline(w, data, seconds: float):
    """The oracle, as it stands, on the host cores: whole steps (fp64 scores
    for every row, top-k, linked-list LRU, block copies, attention) until
    `seconds` of wall time have passed."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    q, sq, K, V, lens = data["q"], data["score_q"], data["K"], data["V"], data["seq_lens"]
    scale = 1.0 / math.sqrt(w.head_dim)
    lru = oracle.LRU(w.rows, w.capacity)
    npdt = np.float32 if w.dtype == "f32" else np.uint16
    pool_k = np.zeros((w.batch, w.n_kv_heads, w.capacity, 16, w.head_dim), dtype=npdt)
    pool_v = np.zeros_like(pool_k)
    # Quest boxes: set-up, outside the timed steps (as on the GPU)
    meta = oracle.quest_meta(K, lens) if w.scoring == "quest" else None
    t0 = time.perf_counter()
    steps, misses = 0, 0
    while True:
        t = steps % q.shape[0]
        if meta is not None:
            s = oracle.score_quest(sq[t], meta, lens, scale, T=w.ctx)
        else:
            s = oracle.score_blockmax(sq[t], K, lens, scale)
        sel, cnt = oracle.topk(s, lens, w.k_blocks, w.ctx, sink=w.sink, recent=w.recent)
        out = lru.step(sel.reshape(w.rows, -1), cnt.reshape(-1), w.nb_max)
        oracle.gather(out["miss_block"], out["miss_slot"], out["miss_count"], K, V, pool_k, pool_v)
        oracle.attention(q[t], K, V, sel, cnt, lens, scale)
        misses += int(out["miss_count"].sum())
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=round(steps / el, 4), unit="steps/s", cores=threads, kind="oracle",
                sample=f"{steps} whole steps (all {w.rows} rows, fp64) of the {w.name} workload, "
                       f"{el:.1f} s wall on {threads} OpenMP threads",
                gbps=round(step_bytes(w, misses / steps)["total"] * steps / el / 1e9, 3),
                cpu_model=cpu_model(),
                note="the oracle is a plain fp64 correctness reference, not a tuned CPU implementation")


# ---------------------------------------------------------------- counters
COPY_MIB = 512  # calibration copy: 512 MiB read + 512 MiB written


def pmc_pass(args):
    """Run under ``rocprofv3 --pmc <counter>``: one plain device copy of
    COPY_MIB MiB (the calibration kernel, known bytes), `steps` launches of
    the scoring kernel on the benchmark workload, then warmup + steps fused
    steps (scoring + select-attend + merge) from a cold working set.  The
    miss counts of the last `steps` fused steps go to ``--pmc-out`` (JSON)
    for the algorithmic bytes of those launches.  Prints one line."""
    import torch

    from top_sparse_kv_block_amd import binding as B
    from top_sparse_kv_block_amd import synth
    from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig

    w = synth.WORKLOADS[args.workload]
    n_fused = args.warmup + args.steps
    data = synth.gen_workload(w.scaled(steps=max(n_fused, 1)))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda() \
        if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, sq, dK, dV, dlens = dev(data["q"]), dev(data["score_q"]), dev(data["K"]), dev(data["V"]), dev(data["seq_lens"])
    mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity,
                     mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent)
    buf = LayerBuffers(cfg)
    keys_or_meta = dK
    if mode == B.SKV_SCORE_QUEST:  # the Quest scan reads the per-block boxes
        keys_or_meta = torch.empty(w.batch, w.n_kv_heads, cfg.nb, 2, w.head_dim, dtype=cfg.torch_dtype,
                                   device="cuda")
        B.sparse_kv_quest_meta(cfg.shape, dK, dlens, keys_or_meta)
    n = COPY_MIB << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    for t in range(args.steps):
        B.sparse_kv_score(cfg.shape, mode, sq[t], cfg.n_queries, keys_or_meta, dlens, cfg.softmax_scale,
                          buf.scores)
    buf.reset()
    misses = torch.zeros(n_fused, dtype=torch.int64, device="cuda")
    for t in range(n_fused):
        buf.score(sq[t], keys_or_meta, dlens)
        buf.select_attend(q[t], dlens, dK, dV)
        misses[t] = buf.miss_count.sum()
    torch.cuda.synchronize()
    if args.pmc_out:
        with open(args.pmc_out, "w") as f:
            json.dump({"workload": w.name, "warmup": args.warmup, "steps": args.steps,
                       "splits": buf.fused_splits, "misses": misses[args.warmup:].tolist()}, f)
    print(f"pmc pass done: copy {COPY_MIB} MiB, {args.steps} scoring launches, {n_fused} fused steps on {w.name}",
          flush=True)


def _counter_rows(path):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _dispatch_order(r):
    for key in ("Dispatch_Id", "Correlation_Id", "Index"):
        if r.get(key, "").strip().isdigit():
            return int(r[key])
    return 0


XCHECK_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_MISS_sum")


def _xcheck(path, steps, names):
    """Raw counters of a third --pmc run (XCHECK_COUNTERS): L2-to-memory
    read requests, their 32-byte and 128-byte ('bubble') parts, and L2
    misses (reads and writes), per kernel (`names`: kernel-name patterns)."""
    rows = _counter_rows(path)
    out = {}
    for counter in XCHECK_COUNTERS:
        rs = [r for r in rows if r.get("Counter_Name") == counter]
        copy = [float(r["Counter_Value"]) for r in rs if "copybuffer" in r["Kernel_Name"].lower()]
        per = {}
        for kname, pat in names.items():
            ks = sorted((r for r in rs if pat in r["Kernel_Name"]), key=_dispatch_order)
            vals = [float(r["Counter_Value"]) for r in ks][-steps:]
            per[kname] = float(np.mean(vals)) if vals else None
        out[counter] = dict(copy=max(copy) if copy else None, kernels=per)
    return out


def traffic_summary(fetch_dir, write_dir, misses_file, workload, xcheck_dir=None):
    """Counter-derived HBM traffic of the step's kernels (the scan, the fused
    select-attend, the merge-commit) from two rocprofv3 --pmc runs of
    ``--pmc-pass`` (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
    scaled by the factor that makes the calibration copy read (write)
    exactly COPY_MIB MiB, against each launch's algorithmic bytes.  Writes
    the JSON the benchmark reads and a short markdown summary under
    profiles/."""
    from top_sparse_kv_block_amd import synth

    w = synth.WORKLOADS[workload]
    names = _kernel_names(w)
    with open(misses_file) as f:
        mf = json.load(f)
    steps, splits, miss = mf["steps"], mf["splits"], mf["misses"]
    algo = {"score": [score_launch_bytes(w)] * steps,
            "select_attend": [fused_launch_bytes(w, m, splits) for m in miss],
            "merge_commit": [merge_launch_bytes(w, splits)] * steps,
            "topk_chunk": [chunk_launch_bytes(w)] * steps}
    counters = {}
    for counter, path in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(path) if r.get("Counter_Name") == counter]
        copy = [float(r["Counter_Value"]) for r in rows if "copybuffer" in r["Kernel_Name"].lower()]
        if not copy:
            raise SystemExit(f"{counter}: no calibration copy dispatch")
        factor = (COPY_MIB << 20) / (max(copy) * 1024.0)
        per = {}
        for kname, pat in names.items():
            ks = sorted((r for r in rows if pat in r["Kernel_Name"]), key=_dispatch_order)
            vals = [float(r["Counter_Value"]) for r in ks][-steps:]
            if not vals:
                raise SystemExit(f"{counter}: no {pat} dispatches")
            per[kname] = dict(kib_avg=float(np.mean(vals)), bytes=float(np.mean(vals)) * 1024.0 * factor,
                              dispatches=len(vals))
        counters[counter] = dict(copy_kib=max(copy), factor=factor, kernels=per)
    kernels = {}
    for kname in names:
        fetch = counters["FETCH_SIZE"]["kernels"][kname]["bytes"]
        write = counters["WRITE_SIZE"]["kernels"][kname]["bytes"]
        a = float(np.mean(algo[kname]))
        kernels[kname] = dict(kernel=names[kname], source_sha=_sources_sha(kname),
                              bytes_per_launch=int(round(fetch + write)), fetch_bytes=int(round(fetch)),
                              write_bytes=int(round(write)), algorithmic_bytes_per_launch=int(round(a)),
                              ratio=round((fetch + write) / a, 4))
    xc = None
    if xcheck_dir:
        xc = _xcheck(xcheck_dir, steps, names)
        # read requests against the copy's reads; L2 misses against the
        # copy's reads and writes (a write also misses once per line)
        for counter, copy_bytes in (("TCC_EA0_RDREQ_sum", float(COPY_MIB << 20)),
                                    ("TCC_MISS_sum", float(2 * (COPY_MIB << 20)))):
            c = xc[counter]
            if not c["copy"]:
                continue
            unit = copy_bytes / c["copy"]  # bytes per request / per miss of the calibration copy
            c["bytes_per_unit"] = unit
            for kname in names:
                v = c["kernels"][kname]
                kernels[kname][f"bytes_from_{counter}"] = int(round(v * unit)) if v is not None else None
    res = dict(workload=w.name, steps=steps, splits=splits, miss_blocks_per_step=float(np.mean(miss)),
               kernels=kernels, counters=counters, xcheck=xc)
    out_json = traffic_file(w.name)
    pdir = "pmc" if w.name == "llama8b_32k" else f"pmc_{w.name}"  # the counter runs' output folders
    os.makedirs(os.path.dirname(out_json), exist_ok=True)
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    md = out_json.replace(".json", ".md")
    with open(md, "w") as f:
        f.write(f"# HBM traffic of the step's kernels, {w.name} workload\n\n"
                "Counter runs (one MI355X; `$REPO` is the repository root), then the summary:\n\n```\n"
                f"cd /tmp && rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/{pdir}_fetch -o f -- "
                f"python3 $REPO/bench.py --pmc-pass --steps {steps} --warmup {mf['warmup']} --workload {w.name} "
                f"--pmc-out $REPO/gpurun_out/{pdir}_misses.json\n"
                f"cd /tmp && rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/{pdir}_write -o w -- "
                f"python3 $REPO/bench.py --pmc-pass --steps {steps} --warmup {mf['warmup']} --workload {w.name}\n"
                "cd /tmp && rocprofv3 --pmc " + " ".join(XCHECK_COUNTERS) + " --output-format csv -d "
                f"$REPO/gpurun_out/{pdir}_xcheck -o x -- "
                f"python3 $REPO/bench.py --pmc-pass --steps {steps} --warmup {mf['warmup']} --workload {w.name}\n"
                f"python3 bench.py --workload {w.name} --traffic-summary gpurun_out/{pdir}_fetch "
                f"gpurun_out/{pdir}_write gpurun_out/{pdir}_misses.json gpurun_out/{pdir}_xcheck\n```\n\n"
                f"Calibration: a plain device copy of {COPY_MIB} MiB; each counter is scaled so that the copy "
                f"reads (writes) exactly {COPY_MIB} MiB.  Scale factors: FETCH_SIZE "
                f"{counters['FETCH_SIZE']['factor']:.4f}, WRITE_SIZE {counters['WRITE_SIZE']['factor']:.4f}.  The "
                f"fused and merge launches are the last {steps} of {steps + mf['warmup']} steps from a cold working "
                f"set ({np.mean(miss):.1f} missed blocks per step, {splits} splits).\n\n"
                "| kernel | FETCH_SIZE KiB / launch | WRITE_SIZE KiB / launch | scaled bytes / launch | "
                "algorithmic bytes / launch | ratio |\n|---|---:|---:|---:|---:|---:|\n")
        for kname, v in kernels.items():
            f.write(f"| {v['kernel']} | {counters['FETCH_SIZE']['kernels'][kname]['kib_avg']:.0f} | "
                    f"{counters['WRITE_SIZE']['kernels'][kname]['kib_avg']:.0f} | {v['bytes_per_launch']} | "
                    f"{v['algorithmic_bytes_per_launch']} | {v['ratio']:.4f} |\n")
        if xc is not None:
            f.write("\nCross-check with raw counters (a third run, `--pmc " + " ".join(XCHECK_COUNTERS) + "`): "
                    "each counter per dispatch; the read bytes from the L2-to-memory read requests (unit: the "
                    "copy's read bytes per request) beside the scaled FETCH_SIZE, and the read + write bytes from "
                    "the L2 misses (unit: the copy's read + write bytes per miss) beside scaled FETCH_SIZE + "
                    "WRITE_SIZE.\n\n"
                    "| kernel | " + " | ".join(XCHECK_COUNTERS) + " | read bytes from RDREQ | FETCH_SIZE bytes "
                    "| bytes from TCC_MISS | FETCH + WRITE bytes |\n|---|" + "---:|" * (len(XCHECK_COUNTERS) + 4)
                    + "\n")
            f.write("| copy (calibration) | " + " | ".join(f"{xc[c]['copy']:.0f}" for c in XCHECK_COUNTERS)
                    + f" | {COPY_MIB << 20} | {COPY_MIB << 20} | {2 * (COPY_MIB << 20)} | {2 * (COPY_MIB << 20)} |\n")
            for kname, v in kernels.items():
                f.write(f"| {v['kernel']} | " + " | ".join(f"{xc[c]['kernels'][kname]:.0f}" for c in XCHECK_COUNTERS)
                        + f" | {v.get('bytes_from_TCC_EA0_RDREQ_sum')} | {v['fetch_bytes']} | "
                        f"{v.get('bytes_from_TCC_MISS_sum')} | {v['bytes_per_launch']} |\n")
            f.write("\nUnits implied by the copy: "
                    + ", ".join(f"{c} {xc[c].get('bytes_per_unit', 0):.1f} B" for c in ("TCC_EA0_RDREQ_sum",
                                                                                        "TCC_MISS_sum"))
                    + ".  Every L2-to-memory read is a 128-byte request and TCC_BUBBLE_sum stays 0, while the "
                      "FETCH_SIZE expression counts a request that is neither a bubble nor 32 bytes as 64 bytes: "
                      "that is the factor 2 of its scale.\n")
        f.write("\nKernel source sha: " + ", ".join(f"{k} {v['source_sha']}" for k, v in kernels.items()) + ".\n")
    return res


# ---------------------------------------------------------------- host tier
def host_fetch_leg(layers: int = 4, steps: int = 3, seed: int = 4):
    """Miss fetch over PCIe at the host-tier row shape (16 x 8 rows, 131072
    tokens, k = 128 of 256 slots, given selections with ~50% cross-layer and
    ~80% cross-step overlap).  One layer's full K and V (2 x 4 GiB) sit in
    pinned, device-mapped host memory and every layer reads it (each layer
    has its own working set and selections, so the transfers are the same
    as with distinct host layers).  Step 0 (cold) is not timed.  Reports the
    host->device rate of the misses for the separate gather and for fetch on
    attend, beside a plain pinned hipMemcpyAsync of 256 MiB, and the layer
    loop with the cross-layer prefetch (layer l+1's working set takes layer
    l's picks on a second stream while layer l attends): the misses left on
    each layer's critical path, the blocks prefetched, and the time of each
    layer's own update (the stall once its selection is known) with and
    without it.  Layer 0 of each step has no earlier layer and is left out
    of these per-layer figures."""
    import torch

    from top_sparse_kv_block_amd import binding as B
    from top_sparse_kv_block_amd import synth
    from top_sparse_kv_block_amd.step import LayerBuffers, StepConfig, layer_sweep

    w = synth.WORKLOADS["host_tier_32l"].scaled(layers=layers, steps=steps)
    t0 = time.time()
    sels = torch.from_numpy(synth.gen_layer_selections(w)).cuda()
    n_elem = w.rows * w.ctx * w.head_dim
    nbytes = n_elem * w.elem_bytes
    hk, hv = B.HostBuffer(nbytes), B.HostBuffer(nbytes)
    try:
        g = torch.Generator(device="cuda").manual_seed(seed)
        chunk = torch.randn(1 << 25, generator=g, device="cuda").to(torch.bfloat16)  # 64 MiB
        for hb in (hk, hv):
            ht = torch.from_numpy(hb.numpy(np.int16, (n_elem,))).view(torch.bfloat16)
            for off in range(0, n_elem, chunk.numel()):
                n = min(chunk.numel(), n_elem - off)
                ht[off:off + n].copy_(chunk[:n])
        lens = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
        q = torch.randn(w.batch, w.n_q_heads, w.head_dim, generator=g, device="cuda").to(torch.bfloat16)
        cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ctx, w.dtype, w.k_blocks, w.capacity)
        bufs = [LayerBuffers(cfg) for _ in range(layers)]
        for b in bufs:
            b.sel_count.fill_(w.k_blocks)
        torch.cuda.synchronize()
        setup_s = time.time() - t0
        blk2 = 2 * 16 * w.head_dim * w.elem_bytes  # K + V bytes of one block

        srcs = [(hk.device_ptr, hv.device_ptr)] * layers
        side = torch.cuda.Stream()

        def run_sweep(prefetch):
            # the layer loop of one decode step (layer_sweep); with prefetch,
            # layer l+1's working set takes layer l's picks on a second stream
            for b in bufs:
                b.reset()
            evs, walls = [], []
            misses = torch.zeros(steps, layers, 2, dtype=torch.int64, device="cuda")
            for s in range(steps):
                for l, b in enumerate(bufs):
                    b.sel_blocks.copy_(sels[s, l])
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                rec = []
                layer_sweep(bufs, q, lens, srcs, B.SKV_SRC_HOST_MAPPED, prefetch=prefetch, side_stream=side,
                            events=rec)
                e[1].record()
                for l, b in enumerate(bufs):
                    misses[s, l, 0] = b.miss_count.sum()
                    if prefetch and l > 0:
                        misses[s, l, 1] = b.pf_miss_count.sum()
                evs.append(rec)
                walls.append(e)
            torch.cuda.synchronize()
            # steps after the cold one; layers after the first (the first has no earlier layer)
            upd = sum(r[l]["update"][0].elapsed_time(r[l]["update"][1]) for r in evs[1:] for l in range(1, layers))
            pf = sum(r[l]["prefetch"][0].elapsed_time(r[l]["prefetch"][1]) for r in evs[1:]
                     for l in range(layers - 1)) if prefetch else 0.0
            wall = sum(a.elapsed_time(b) for a, b in walls[1:])
            m = misses[1:, 1:].sum(dim=(0, 1)).tolist()
            n = (steps - 1) * (layers - 1)
            return dict(crit=m[0] / n, pf=m[1] / n, update_us=upd * 1e3 / n, prefetch_us=pf * 1e3 / n,
                        wall_us_per_layer=wall * 1e3 / ((steps - 1) * layers), m_total=m[0], upd_ms=upd)

        def run_fetch_on_attend():
            # list-only updates (the no-IO control: NULL sources) followed by
            # attention that fetches the misses over PCIe itself
            for b in bufs:
                b.reset()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(layers * steps)]
            misses = torch.zeros(steps, layers, dtype=torch.int64, device="cuda")
            for s in range(steps):
                for l, b in enumerate(bufs):
                    b.sel_blocks.copy_(sels[s, l])
                    e = ev[s * layers + l]
                    e[2].record()
                    b.cache_update(None, None)
                    e[3].record()
                    e[0].record()
                    b.attention(q, lens, hk.device_ptr, hv.device_ptr, B.SKV_SRC_HOST_MAPPED)
                    e[1].record()
                    misses[s, l] = b.miss_count.sum()
            torch.cuda.synchronize()
            us = sum(e[0].elapsed_time(e[1]) for e in ev[layers:]) * 1e3
            # per layer, the same layers as gather_us_per_layer (steps after the cold one, layers after the first)
            no_io = [ev[s * layers + l][2].elapsed_time(ev[s * layers + l][3]) * 1e3
                     for s in range(1, steps) for l in range(1, layers)]
            m = int(misses[1:].sum().item())
            m_crit = int(misses[1:, 1:].sum().item())
            return m, us, float(np.mean(no_io)), m_crit

        plain = run_sweep(False)
        cross = run_sweep(True)
        m_f, us_f, no_io_us, m_crit = run_fetch_on_attend()
        # plain pinned copy, 256 MiB, for scale
        n_c = 128 << 20
        src = torch.from_numpy(hk.numpy(np.int16, (n_c,)))
        dst = torch.empty(n_c, dtype=torch.int16, device="cuda")
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(4):
            dst.copy_(src, non_blocking=True)
        c1.record()
        torch.cuda.synchronize()
        memcpy_gbps = 4 * n_c * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        timed = (steps - 1) * layers
        n_l = (steps - 1) * (layers - 1)
        return {
            "workload": w.name,
            "rows": w.rows, "ctx": w.ctx, "k_blocks": w.k_blocks, "capacity_slots": w.capacity,
            "layers_run": layers, "timed_layer_steps": timed,
            "host_source": "one layer's K and V (8 GiB) in pinned mapped host memory, read by every layer",
            "miss_blocks_per_layer": round(plain["crit"], 1),
            "gather_h2d_gbps": round(plain["m_total"] * blk2 / (plain["upd_ms"] * 1e-3) / 1e9, 2),
            "gather_us_per_layer": round(plain["update_us"], 1),
            "no_io_update_us_per_layer": round(no_io_us, 1),
            "no_io_same_misses": bool(m_crit == plain["m_total"]),
            "cross_layer_prefetch": {
                "critical_miss_blocks_per_layer": round(cross["crit"], 1),
                "prefetched_blocks_per_layer": round(cross["pf"], 1),
                "critical_update_us_per_layer": round(cross["update_us"], 1),
                "prefetch_us_per_layer": round(cross["prefetch_us"], 1),
                "miss_stall_hidden": round(1.0 - cross["update_us"] / plain["update_us"], 3),
                "sweep_us_per_layer": round(cross["wall_us_per_layer"], 1),
                "sweep_us_per_layer_without": round(plain["wall_us_per_layer"], 1),
                "layers_counted": n_l,
            },
            "fetch_on_attend_h2d_gbps": round(m_f * blk2 / (us_f * 1e-6) / 1e9, 2),
            "attention_with_fetch_us_per_layer": round(us_f / timed, 1),
            "pinned_memcpy_h2d_gbps": round(memcpy_gbps, 2),
            "setup_s": round(setup_s, 1),
        }
    finally:
        torch.cuda.synchronize()
        hk.free()
        hv.free()


# ---------------------------------------------------------------- GPU leg
def run(args):
    import torch

    from top_sparse_kv_block_amd import binding as B
    from top_sparse_kv_block_amd import synth
    from top_sparse_kv_block_amd.step import Lag1Pipeline, LayerBuffers, StepConfig

    w = synth.WORKLOADS[args.workload]
    if args.lag1:
        # lag-1 keeps the previous selection resident while the next update runs: 2k slots
        w = w.scaled(capacity=max(w.capacity, 2 * w.k_blocks))
    if w.scoring == "given":
        raise SystemExit("the host-tier workload has no scoring stage; its PCIe fetch is the host_fetch leg")
    nsteps = args.warmup + args.steps
    wq = w.scaled(steps=max(nsteps, 1))
    t_gen = time.time()
    data = synth.gen_workload(wq)
    print(f"[bench] generated {w.name} inputs in {time.time() - t_gen:.1f}s", file=sys.stderr, flush=True)

    torch.cuda.set_device(0)
    dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
                     if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a))).cuda()
    q_all, sq_all = dev(data["q"]), dev(data["score_q"])
    T = w.ctx
    if args.grow:
        # room for one appended token per step (warm-up, timed steps and the
        # per-call timing pass); the appended rows are seeded random values
        T = w.ctx + 16 * ((args.warmup + 2 * args.steps + 15) // 16)
        kv_shape = (w.batch, w.n_kv_heads, T, w.head_dim)
        dK = torch.zeros(kv_shape, dtype=q_all.dtype, device="cuda")
        dV = torch.zeros_like(dK)
        dK[:, :, :w.ctx] = dev(data["K"])
        dV[:, :, :w.ctx] = dev(data["V"])
        g = torch.Generator(device="cuda").manual_seed(w.seed + 100)
        new_rows = torch.randn(2, nsteps + args.steps, w.batch, w.n_kv_heads, w.head_dim, generator=g,
                               device="cuda").to(q_all.dtype)
    else:
        dK, dV = dev(data["K"]), dev(data["V"])
    dlens = dev(data["seq_lens"])
    mode = B.SKV_SCORE_QUEST if w.scoring == "quest" else B.SKV_SCORE_BLOCKMAX
    cfg = StepConfig(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, T, w.dtype, w.k_blocks, w.capacity,
                     mode=mode, n_queries=w.n_score_queries, sink=w.sink, recent=w.recent, num_splits=args.splits)
    buf = LayerBuffers(cfg)
    select = False
    keys_or_meta = dK
    if mode == B.SKV_SCORE_QUEST:
        keys_or_meta = torch.empty(w.batch, w.n_kv_heads, cfg.nb, 2, w.head_dim, dtype=cfg.torch_dtype,
                                   device="cuda")
        B.sparse_kv_quest_meta(cfg.shape, dK, dlens, keys_or_meta)
    miss_log = torch.zeros(nsteps, w.batch, w.n_kv_heads, dtype=torch.int32, device="cuda")
    shape, st = cfg.shape, None
    scale = cfg.softmax_scale

    pipe = Lag1Pipeline(buf) if args.lag1 else None

    def step(t, ev=None):
        if pipe is not None:
            return step_lag1(t, ev)
        if args.fused:
            return step_fused(t, ev)
        # ev: optional list of 5 events bracketing the four calls (profiling pass only)
        if args.grow:
            grow()
        if ev is not None:
            ev[0].record()
        B.sparse_kv_score(shape, mode, sq_all[t], cfg.n_queries, keys_or_meta, dlens, scale, buf.scores, st)
        if ev is not None:
            ev[1].record()
        if select:
            B.sparse_kv_select(shape, buf.scores, dlens, cfg.k_blocks, cfg.sink, cfg.recent, cfg.capacity,
                               buf.sel_blocks, buf.sel_count, buf.slot_block, buf.slot_stamp, buf.clock, buf.sel_slot,
                               buf.sel_hit, buf.miss_block, buf.miss_slot, miss_log[t], None, None, B.SKV_SRC_DEVICE,
                               buf.pool_k, buf.pool_v, buf.topk_workspace, st)
            if ev is not None:
                ev[2].record()
                ev[3].record()
            B.sparse_decode_attention(shape, q_all[t], buf.pool_k, buf.pool_v, cfg.capacity, buf.sel_blocks,
                                      buf.sel_slot, buf.sel_hit, buf.sel_count, dlens, cfg.k_blocks, scale,
                                      buf.splits, dK, dV, B.SKV_SRC_DEVICE, buf.out, buf.lse, buf.workspace, st)
            if ev is not None:
                ev[4].record()
            return
        B.sparse_kv_topk(shape, buf.scores, dlens, cfg.k_blocks, cfg.sink, cfg.recent, buf.sel_blocks,
                         buf.sel_count, buf.topk_workspace, st)
        if ev is not None:
            ev[2].record()
        # list-only cache update; the attention kernel fetches the misses
        if args.eviction == "importance":
            B.sparse_kv_cache_update_importance(shape, cfg.k_blocks, cfg.capacity, buf.sel_blocks, buf.sel_count,
                                                buf.scores, buf.slot_block, buf.slot_stamp, buf.clock, buf.sel_slot,
                                                buf.sel_hit, buf.miss_block, buf.miss_slot, miss_log[t], None, None,
                                                B.SKV_SRC_DEVICE, buf.pool_k, buf.pool_v, st)
        else:
            B.sparse_kv_cache_update(shape, cfg.k_blocks, cfg.capacity, buf.sel_blocks, buf.sel_count,
                                     buf.slot_block, buf.slot_stamp, buf.clock, buf.sel_slot, buf.sel_hit,
                                     buf.miss_block, buf.miss_slot, miss_log[t], None, None, B.SKV_SRC_DEVICE,
                                     buf.pool_k, buf.pool_v, st)
        if ev is not None:
            ev[3].record()
        B.sparse_decode_attention(shape, q_all[t], buf.pool_k, buf.pool_v, cfg.capacity, buf.sel_blocks,
                                  buf.sel_slot, buf.sel_hit, buf.sel_count, dlens, cfg.k_blocks, scale, buf.splits,
                                  dK, dV, B.SKV_SRC_DEVICE, buf.out, buf.lse, buf.workspace, st)
        if ev is not None:
            ev[4].record()

    def step_lag1(t, ev=None):
        # attention over the previous step's selection on this stream; score,
        # top-k and the working-set update of this step on the side stream.
        # ev brackets the whole step (the two streams overlap)
        if ev is not None:
            ev[0].record()
        pipe.step(q_all[t], sq_all[t], keys_or_meta, dlens, dK, dV, B.SKV_SRC_DEVICE, miss_count=miss_log[t])
        if ev is not None:
            pipe.join()
            for e in ev[1:]:
                e.record()

    appended = [0]

    def grow():
        # one new token per sequence before the step (lengths grow on the device)
        i = appended[0]
        appended[0] += 1
        B.sparse_kv_append(shape, new_rows[0, i], new_rows[1, i], dlens, dK, dV,
                           keys_or_meta if mode == B.SKV_SCORE_QUEST else None, buf.slot_block, cfg.capacity,
                           buf.pool_k, buf.pool_v, st)

    def step_fused(t, ev=None):
        # score, then top-k + working-set update + attention (fetching the
        # misses) as the single fused call; ev brackets the two calls
        if args.grow:
            grow()
        if ev is not None:
            ev[0].record()
        B.sparse_kv_score(shape, mode, sq_all[t], cfg.n_queries, keys_or_meta, dlens, scale, buf.scores, st)
        if ev is not None:
            ev[1].record()
        B.sparse_kv_select_attend(shape, buf.scores, dlens, cfg.k_blocks, cfg.sink, cfg.recent, cfg.capacity,
                                  buf.sel_blocks, buf.sel_count, buf.slot_block, buf.slot_stamp, buf.clock,
                                  buf.sel_slot, buf.sel_hit, buf.miss_block, buf.miss_slot, miss_log[t], q_all[t],
                                  buf.pool_k, buf.pool_v, dK, dV, B.SKV_SRC_DEVICE, scale, buf.fused_splits,
                                  buf.out, buf.lse, buf.workspace, st)
        if ev is not None:
            for e in ev[2:]:
                e.record()

    # cold start, warm-up (not timed)
    if pipe is not None:
        pipe.reset()
    else:
        buf.reset()
    for t in range(args.warmup):
        step(t)
    if pipe is not None:
        pipe.join()
    torch.cuda.synchronize()

    # the state after the warm-up, restored before every repetition (and
    # before the per-call passes below) so each one runs the same steps from
    # the same working sets: slot tables, stamps, clocks, pools, lengths
    # (they grow with --grow, as do the Quest boxes), the lag-1 list sets
    def state_tensors():
        ts = [buf.slot_block, buf.slot_stamp, buf.clock, buf.pool_k, buf.pool_v, dlens]
        if pipe is not None:
            for lst in pipe.lists:
                ts += [lst.sel_blocks, lst.sel_count, lst.sel_slot, lst.sel_hit, lst.miss_block, lst.miss_slot,
                       lst.miss_count]
        if args.grow and mode == B.SKV_SCORE_QUEST:
            ts.append(keys_or_meta)
        return ts

    saved = [t.clone() for t in state_tensors()]
    pipe_t = pipe.t if pipe is not None else 0
    appended_t = appended[0]

    def restore():
        for t, v in zip(state_tensors(), saved):
            t.copy_(v)
        appended[0] = appended_t
        if pipe is not None:
            pipe.t, pipe._upd_prev = pipe_t, None
        torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides, run
    # `reps` times from the restored state; the median is reported.  By
    # default the steps are captured once into a HIP graph and the graph is
    # replayed (the host then only submits one launch); --eager enqueues the
    # calls per step from Python instead.
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
            if pipe is not None:
                pipe.join()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rep_s, enq_s = [], []
    for _ in range(max(args.reps, 1)):
        restore()
        t0 = time.perf_counter()
        e0.record()
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(args.warmup + i)
            if pipe is not None:
                pipe.join()
        enq_s.append(time.perf_counter() - t0)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        rep_s.append(max(wall, e0.elapsed_time(e1) / 1e3))
    elapsed = float(np.median(rep_s))
    t_enq = float(np.median(enq_s))
    misses = miss_log[args.warmup:].sum().item()

    # profiling passes right after the timed region, on the same stream:
    # (a) the scoring kernel alone, `steps` launches back to back between two
    #     events -> its average launch duration (the roofline point);
    # (b) the same steps again with each call bracketed by events -> a
    #     per-call breakdown (each bracket also holds one event marker).
    def score_pass():
        for i in range(args.steps):
            B.sparse_kv_score(shape, mode, sq_all[args.warmup + i], cfg.n_queries, keys_or_meta, dlens, scale,
                              buf.scores, st)

    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph is not None:  # replayed as a graph too, so launch gaps stay small
        sgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sgraph):
            score_pass()
        torch.cuda.synchronize()
        s0.record()
        sgraph.replay()
    else:
        s0.record()
        score_pass()
    s1.record()
    torch.cuda.synchronize()
    score_avg_s = s0.elapsed_time(s1) / 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    restore()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    stage = np.array([[ev[c].elapsed_time(ev[c + 1]) for c in range(4)] for ev in evs]) * 1e3  # us

    # achievable-read anchor: the scan's bytes read by a kernel with the
    # scan's launch shape and load form and no arithmetic, timed like it
    read_gbps = None
    if mode == B.SKV_SCORE_BLOCKMAX:
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")

        def read_pass():
            for _ in range(args.steps):
                B.sparse_kv_stream_read(shape, dK, sink, st)

        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if graph is not None:
            rgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(rgraph):
                read_pass()
            torch.cuda.synchronize()
            r0.record()
            rgraph.replay()
        else:
            r0.record()
            read_pass()
        r1.record()
        torch.cuda.synchronize()
        read_avg_s = r0.elapsed_time(r1) / 1e3 / args.steps
        read_gbps = w.rows * T * w.head_dim * w.elem_bytes / read_avg_s / 1e9

    # no-IO control: the same steps' working-set updates timed with NULL
    # sources (lists only) and with the HBM source (lists, then the copy of
    # every miss into the pool), from the same restored state, so both see
    # the same selections and misses
    no_io = None
    if pipe is None and not args.grow and not select and args.eviction == "lru":
        def update_pass(with_src):
            restore()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for i in range(args.steps):
                t = args.warmup + i
                B.sparse_kv_score(shape, mode, sq_all[t], cfg.n_queries, keys_or_meta, dlens, scale, buf.scores, st)
                B.sparse_kv_topk(shape, buf.scores, dlens, cfg.k_blocks, cfg.sink, cfg.recent, buf.sel_blocks,
                                 buf.sel_count, buf.topk_workspace, st)
                ev[i][0].record()
                src = (dK, dV) if with_src else (None, None)
                B.sparse_kv_cache_update(shape, cfg.k_blocks, cfg.capacity, buf.sel_blocks, buf.sel_count,
                                         buf.slot_block, buf.slot_stamp, buf.clock, buf.sel_slot, buf.sel_hit,
                                         buf.miss_block, buf.miss_slot, miss_log[t], *src, B.SKV_SRC_DEVICE,
                                         buf.pool_k, buf.pool_v, st)
                ev[i][1].record()
                B.sparse_decode_attention(shape, q_all[t], buf.pool_k, buf.pool_v, cfg.capacity, buf.sel_blocks,
                                          buf.sel_slot, buf.sel_hit, buf.sel_count, dlens, cfg.k_blocks, scale,
                                          buf.splits, *((None, None) if with_src else (dK, dV)), B.SKV_SRC_DEVICE,
                                          buf.out, buf.lse, buf.workspace, st)
            torch.cuda.synchronize()
            us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
            return us, miss_log[args.warmup:].sum().item() / args.steps

        update_pass(False)  # untimed: the update and gather kernels' first launches (code load)
        update_pass(True)
        us_none, m_none = update_pass(False)
        us_hbm, m_hbm = update_pass(True)
        blk2 = 2 * 16 * w.head_dim * w.elem_bytes
        no_io = {"no_io_update_us": round(us_none, 2), "update_with_hbm_gather_us": round(us_hbm, 2),
                 "io_us": round(us_hbm - us_none, 2), "miss_blocks_per_step": round(m_hbm, 1),
                 "same_misses": bool(m_none == m_hbm),
                 "gather_gbps": round(m_hbm * blk2 * 2 / max(us_hbm - us_none, 1e-3) / 1e3, 1),
                 "what": "working-set update of the same steps with NULL sources (lists only: the mechanism) "
                         "against the HBM source (lists + copy of every miss into the pool: read + write)"}

    bytes_total = step_bytes(w, misses / args.steps)["total"] * args.steps
    sbytes = score_launch_bytes(w)
    achieved = sbytes / score_avg_s / 1e9
    traffic = _traffic(w)
    steps_per_s = args.steps / elapsed
    res = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * elapsed / args.steps, 4),
        "reps": len(rep_s),
        "ms_per_step_median": round(1e3 * elapsed / args.steps, 4),
        "ms_per_step_min": round(1e3 * min(rep_s) / args.steps, 4),
        "ms_per_step_max": round(1e3 * max(rep_s) / args.steps, 4),
        "spread": round((max(rep_s) - min(rep_s)) / elapsed, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "ctx": w.ctx, "block": 16, "budget_tokens": w.budget,
                   "k_blocks": w.k_blocks, "capacity_slots": w.capacity, "scoring": w.scoring,
                   "n_score_queries": w.n_score_queries,
                   "attn_splits": buf.fused_splits if args.fused else buf.splits,
                   "parallelism": "single-gpu"},
        "hbm_gbps": round(bytes_total / elapsed / 1e9, 1),
        "hbm_frac": round(bytes_total / elapsed / 1e9 / HBM_PEAK_GBPS, 4),
        "bytes_per_step": int(bytes_total / args.steps),
        "miss_blocks_per_step": round(misses / args.steps, 1),
        "mode": "hip-graph replay" if graph is not None else "eager",
        "host_enqueue_us_per_step": round(1e6 * t_enq / args.steps, 2),
        "path": ("lag-1 pipeline: attention over the previous selection || score, top-k, update on a second stream"
                 if pipe is not None else "score + fused select/update/attend" if args.fused else
                 "score + one-launch select (top-k, update) + attention" if select else "four calls"),
        "eviction": args.eviction,
        "grow": bool(args.grow),
        "stage_us": ({"step": round(float(stage.sum(axis=1).mean()), 2)} if pipe is not None else
                     {"score": round(float(stage[:, 0].mean()), 2),
                      "select_update_attend": round(float(stage[:, 1].mean()), 2)} if args.fused else
                     {"score": round(float(stage[:, 0].mean()), 2), "select": round(float(stage[:, 1].mean()), 2),
                      "attention": round(float(stage[:, 3].mean()), 2)} if select else
                     {name: round(float(v), 2) for name, v in
                      zip(("score", "topk", "cache_update", "attention"), stage.mean(axis=0))}),
        "roofline": {"bound": "hbm", "kernel": _score_kernel_name(w),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "avg_launch_us": round(score_avg_s * 1e6, 2),
                     "bytes_per_launch": sbytes,
                     "achievable_read_gbps": round(read_gbps, 1) if read_gbps else None,
                     "frac_of_achievable": round(achieved / read_gbps, 4) if read_gbps else None,
                     "read_anchor": "sparse_kv_stream_read: the scan's launch shape and 16-byte load form, no "
                                    "arithmetic, over the same keys" if read_gbps else None},
        "input_sha256": input_sha256(data),
    }
    if no_io is not None:
        res["no_io"] = no_io
    if not args.no_host_fetch:
        res["host_fetch"] = host_fetch_leg()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, data, args.cpu_seconds)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--reps", type=int, default=10,
                    help="repetitions of the timed steps, each from the restored post-warm-up state; the median "
                         "is reported")
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--splits", type=int, default=0, help="attention splits (0 = library default)")
    ap.add_argument("--eager", action="store_true", help="enqueue every call from Python instead of a graph")
    ap.add_argument("--four-calls", dest="fused", action="store_false",
                    help="run stages 2-4 as three calls instead of the fused select-attend call")
    ap.add_argument("--eviction", choices=("lru", "importance"), default="lru",
                    help="working-set eviction; importance (by this step's scores) runs the four calls")
    ap.add_argument("--grow", action="store_true",
                    help="append one token per sequence before every step (decode-time growth; Quest boxes kept)")
    ap.add_argument("--lag1", action="store_true",
                    help="lag-1 pipeline: each step attends over the previous step's selection while its own "
                         "score, top-k and update run on a second stream (capacity raised to 2k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-host-fetch", action="store_true", help="skip the host-tier PCIe fetch measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="calibration copy + scoring launches only, to run under rocprofv3 --pmc")
    ap.add_argument("--pmc-out", default=None, help="with --pmc-pass: JSON file for the fused steps' miss counts")
    ap.add_argument("--traffic-summary", nargs="+", metavar="DIR",
                    help="FETCH_DIR WRITE_DIR MISSES_JSON [XCHECK_DIR]: turn the rocprofv3 --pmc outputs of "
                         "--pmc-pass into the traffic file under profiles/")
    args = ap.parse_args(argv)
    if args.eviction == "importance":
        args.fused = False  # the fused call evicts LRU only
    if args.lag1:
        if args.grow or args.eviction != "lru":
            raise SystemExit("--lag1 runs on a fixed-length cache with LRU eviction")
        args.fused = False
        args.no_cpu_baseline = True  # the oracle leg replays the synchronous step
    if args.grow:
        args.no_cpu_baseline = True  # the oracle leg replays the fixed-length workload
    if args.traffic_summary:
        ts = args.traffic_summary
        if len(ts) not in (3, 4):
            raise SystemExit("--traffic-summary takes FETCH_DIR WRITE_DIR MISSES_JSON [XCHECK_DIR]")
        print(json.dumps(traffic_summary(ts[0], ts[1], ts[2], args.workload, ts[3] if len(ts) == 4 else None)))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the step runs on a single MI355X and has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        return 2
    if args.pmc_pass:
        pmc_pass(args)
        return 0
    res = run(args)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
