"""Seeded input generators and the traffic model, pinned to the pages' printed figures."""
import json

import numpy as np
import torch

import workloads as W


def test_generation_is_deterministic_and_seed_dependent():
    w = W.WORKLOADS["batched"].replace(batch=3, seq_len=2048, seq_len_min=700)
    a = W.make_inputs(w, seed=4)
    b = W.make_inputs(w, seed=4)
    c = W.make_inputs(w, seed=5)
    for key in ("q", "k", "v", "seq_lens"):
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["k"], c["k"])
    assert a["k"].dtype == torch.bfloat16 and a["k"].shape == (3, 2048, 8, 128)
    assert int(a["seq_lens"].min()) >= 700 and int(a["seq_lens"].max()) <= 2048


def test_sinks_needles_outliers_and_paging_are_present():
    w = W.WORKLOADS["llama32k"].replace(seq_len=512)
    x = W.make_inputs(w, seed=0)
    norms = x["k"].float().norm(dim=-1)            # [B, n, Hkv]
    assert float(norms[:, :4].mean()) > 6 * float(norms[:, 4:].mean())

    w = W.WORKLOADS["batched"].replace(batch=2, seq_len=1024, seq_len_min=1024)
    x = W.make_inputs(w, seed=1)
    q, k = x["q"].float(), x["k"].float()
    for b in range(2):
        for h in range(w.q_heads):
            s = (k[b, :, h // w.group] @ q[b, h]) / 128 ** 0.5
            assert int((s > 3.5).sum()) >= 12           # needles stand out of N(0, 1) scores

    w = W.WORKLOADS["qwen128k"].replace(batch=1, seq_len=2048)
    x = W.make_inputs(w, seed=2)
    std = x["v"].float().std(dim=(0, 1))               # [Hkv, d]
    assert int((std > 3).sum()) == 8 * w.kv_heads

    w = W.WORKLOADS["paged"].replace(batch=4, seq_len=160)
    x = W.make_inputs(w, seed=3)
    bt = x["block_table"]
    assert bt.shape == (4, 10) and sorted(bt.flatten().tolist()) == list(range(40))
    rows = W.sequence_rows(x, "k", 2)
    assert torch.equal(rows[17], x["k"][int(bt[2, 1]), 1])


def test_traffic_model_matches_pages_figures(golden_dir):
    with open(f"{golden_dir}/traffic_model.json") as f:
        g = json.load(f)
    kv = g["kv_bytes_per_layer_token"]
    w = W.Workload("l", batch=1, q_heads=32, kv_heads=kv["kv_heads"], head_dim=kv["head_dim"],
                   seq_len=kv["seq_len"])
    dense = W.dense_read_bytes(w, [kv["seq_len"]])
    assert abs(dense / kv["approx_bytes"] - 1) < kv["rel_tol"]
    assert dense == 128 * 2 ** 20
    for key in ("gqa_worst_case_union_32k", "per_head_fraction_8k", "gqa_worst_case_union_8k"):
        c = g[key]
        worst_rows = min(c["group"] * c["samples"], c["seq_len"])
        assert abs(100.0 * worst_rows / c["seq_len"] - c["percent"]) <= c["abs_tol"]


def test_traffic_bytes_counts_k_and_distinct_v_rows():
    w = W.WORKLOADS["llama32k"]
    t = W.traffic_bytes(w, [32768], unique_v_rows=1000)
    assert t == (32768 * 8 + 1000) * 256
