"""The benchmark's byte model, pinned to the pages' KV-size formula (CPU only)."""
import json
import os

import bench
from top_sparse_kv_block_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_size_formula_example():
    # 2 * L * layers * kv_heads * head_dim * bytes; Llama-3.1-8B at 32K is about 4 GB
    with open(os.path.join(GOLD, "kv_bytes.json")) as f:
        g = json.load(f)
    e = g["example"]
    b = bench.kv_cache_bytes(e["seq_len"], e["layers"], e["kv_heads"], e["head_dim"], e["bytes_per_elem"])
    assert b == g["bytes"]
    assert round(b / 2**30) == g["approx_gb"]


def test_score_scan_is_the_k_half_of_one_layers_cache():
    w = synth.WORKLOADS["llama8b_32k"]
    by = bench.step_bytes(w, 0)
    k_half = w.batch * bench.kv_cache_bytes(w.ctx, 1, w.n_kv_heads, w.head_dim, 2) // 2
    scan_extra = w.batch * w.n_q_heads * w.head_dim * 2 + w.rows * w.nb_max * 4
    assert by["score"] == k_half + scan_extra
    # the selected K and V: 128 blocks of 16 tokens per row
    assert by["attention"] >= w.rows * w.k_blocks * 16 * w.head_dim * 2 * 2
    # a miss's K and V are read once (counted with attention's reads) and
    # written once into the pool
    assert bench.step_bytes(w, 10)["fetch"] == 10 * 2 * 16 * w.head_dim * 2


def test_multi_gpu_request_exits_with_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_scoring_launch_bytes_per_block():
    # exact block max reads the block's 16 keys; the Quest bound reads its
    # min/max box (2 vectors); both write one 4-byte score per block
    for name, per_block in (("llama8b_32k", 16 * 128 * 2 + 4), ("quest_128k", 2 * 128 * 2 + 4)):
        w = synth.WORKLOADS[name]
        q = w.batch * w.n_score_queries * w.n_q_heads * w.head_dim * w.elem_bytes
        assert bench.score_launch_bytes(w) == w.rows * w.nb_max * per_block + q
    # the 32K figure quoted with the roofline
    assert bench.score_launch_bytes(synth.WORKLOADS["llama8b_32k"]) == 537460736
