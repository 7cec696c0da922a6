"""Benchmark of one SANTA decode step on one MI355X.

A step is one ``santa_decode`` call over one batch of synthetic input: the
fused kernel (scores, global partition function, sampling and gather in one
launch), plus the target sort for multinomial sampling.  The default workload is
the Llama-3.1-8B-shaped layer: batch 1, 32 query / 8 KV heads, d = 128, 32768
bf16 keys, S = 256 systematic samples.  ``--kv-copies`` independent caches
(default 8, 1 GiB) are cycled through, one per step like the layers of a model,
so that K is read from HBM and not from the 256 MB Infinity Cache.

Timing: exactly ``--steps`` calls are timed with HIP events on the launch stream,
replayed from HIP graphs of a few calls each, in ``min(20, steps)`` rounds of
equal length; ``value`` comes from the whole timed interval, and the line also
gives the median of the per-round times with a 95 % bootstrap interval.

The JSON line also carries: the roofline of the dominant kernel (the fused
decode kernel, bound by HBM bandwidth: all of K plus the distinct sampled V rows
per launch), the HBM bandwidth of a plain device copy measured in the same run,
the two-kernel path, S^2ANTA-flash and the top-k comparator on the same inputs,
the Qwen2.5-7B-shaped long-context step (all three sampling rules), Bernoulli
qK^T (B = 8 draws, with the fraction of key features read) beside the exact step
on the same inputs, SANTA++ on the Qwen-shaped 32K layer (31 teams per query
head, with its logical KV access) beside the exact step on the same caches, a
parity sample of the timed
configuration against the oracle (boundary cases, largest CDF difference), and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "decode attention steps/sec (heads×batch) at 32k ctx; achieved HBM GB/s vs peak"
KERNEL_SOURCES = ["santa_fused.hip", "santa_score.hip", "santa_sample.hip", "santa_split.h", "santa_device.h",
                  "santa_internal.h"]
ROUNDS = 20                    # timed rounds (fewer only if fewer calls are timed)
MAX_GRAPH_CALLS = 32           # calls captured per HIP graph
BOUNDARY_WINDOW = 1e-6


def strip_comments(text: str) -> str:
    """C/C++ source without its comments and blank lines (string literals in these
    sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(read=None) -> str:
    """Hash of the decode kernels' sources (fused, score and sample passes),
    comments left out (a comment edit does not change the kernels the counters
    were taken on)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, "sampling_sparse_attention_amd", "csrc", name)) as f:
                text = f.read()
        else:
            text = read(name)
        h.update(strip_comments(text).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per decode step (the dominant kernel, or the score and sample
    passes together) from the committed rocprofv3 counter summary of the
    workload, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama32k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--samples", type=int, default=None)
    ap.add_argument("--mode", type=int, default=None)
    ap.add_argument("--split", type=int, default=0, help="keys per split (0: library default)")
    ap.add_argument("--kv-copies", type=int, default=8)
    ap.add_argument("--eager", action="store_true", help="launch every call from Python, no HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the headline step (no two-kernel, flash, Qwen or copy lines)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run plain device-to-device copies of BYTES bytes (the reference kernel "
                         "for scaling HBM byte counters) and print their bandwidth")
    return ap.parse_args(argv)


def copy_bandwidth(nbytes: int, reps: int = 10):
    """Device-to-device copies of `nbytes`: seconds per copy and (read + write) GB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    t = start.elapsed_time(end) / reps * 1e-3
    del src, dst
    torch.cuda.empty_cache()
    return t, 2 * nbytes / t / 1e9


def make_copies(w, n, device):
    return [W.make_inputs(w, seed=c, device=device) for c in range(n)]


class Runner:
    """Pre-bound calls of one workload over its KV copies."""

    def __init__(self, santa, copies, S, mode, split):
        self.santa = santa
        self.copies = copies
        x = copies[0]
        self.S, self.mode = S, mode
        self.shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len,
                                      split_size=split)
        B, Hq, d = x["q"].shape
        dev = x["q"].device
        self.o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B, Hq, S), dtype=torch.int32, device=dev)
        self.ws = santa.allocate_workspace(self.shape, S, mode, dev)
        self.seed = x["workload"].sample_seed

    def args(self, c):
        x = self.copies[c % len(self.copies)]
        return (self.shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], self.S, self.mode,
                self.seed, self.o, self.idx, self.ws)

    def step(self, c):
        self.santa.santa_decode(*self.args(c))

    def two_kernel(self, c):
        self.santa.santa_score_pass(*self.args(c))
        self.santa.santa_sample_pass(*self.args(c))

    def flash(self, c):
        self.santa.santa_decode_flash(*self.args(c))

    def topk(self, c):
        a = self.args(c)
        self.santa.santa_decode_topk(*a[:6], self.S, *a[9:])


def graph_plan(steps: int, ncopies: int, rounds: int = ROUNDS):
    """How `steps` timed calls are replayed: (calls per graph L, graphs P, replays,
    rounds).  L is the largest divisor of `steps` that leaves at least `rounds`
    replays (at most MAX_GRAPH_CALLS), so exactly `steps` calls run; graph j holds
    calls j*L .. j*L + L - 1, whose KV copies continue where graph j - 1 stopped,
    and the pattern repeats after P graphs."""
    # at least 10 rounds when there are 10 calls, up to `rounds` while graphs stay full
    nr = max(1, min(10, steps), min(rounds, steps // MAX_GRAPH_CALLS))
    cap = max(1, min(MAX_GRAPH_CALLS, steps // nr))
    L = max(d for d in range(1, cap + 1) if steps % d == 0)
    P = ncopies // math.gcd(L, ncopies)
    return L, P, steps // L, nr


def timed(fn, steps, eager, ncopies):
    """Times exactly `steps` calls fn(i) (call i on KV copy i mod ncopies) with events
    on the launch stream.  Returns (seconds per call over the whole interval, seconds
    per call of each round, calls timed)."""
    stream = torch.cuda.current_stream()
    if eager:
        nr = max(1, min(ROUNDS, steps))
        marks = [round(r * steps / nr) for r in range(nr + 1)]
        events = [torch.cuda.Event(enable_timing=True) for _ in range(nr + 1)]
        torch.cuda.synchronize()
        events[0].record(stream)
        for r in range(nr):
            for i in range(marks[r], marks[r + 1]):
                fn(i)
            events[r + 1].record(stream)
        torch.cuda.synchronize()
        per_round = [events[r].elapsed_time(events[r + 1]) * 1e-3 / (marks[r + 1] - marks[r]) for r in range(nr)]
        return events[0].elapsed_time(events[-1]) * 1e-3 / steps, per_round, steps
    L, P, replays, nr = graph_plan(steps, ncopies)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(P * L):
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for j in range(P):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(L):
                fn(j * L + i)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    marks = [round(r * replays / nr) for r in range(nr + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nr + 1)]
    events[0].record(stream)
    for r in range(nr):
        for k in range(marks[r], marks[r + 1]):
            graphs[k % P].replay()
        events[r + 1].record(stream)
    torch.cuda.synchronize()
    per_round = [events[r].elapsed_time(events[r + 1]) * 1e-3 / ((marks[r + 1] - marks[r]) * L) for r in range(nr)]
    calls = replays * L
    del graphs
    return events[0].elapsed_time(events[-1]) * 1e-3 / calls, per_round, calls


def round_stats(rounds, seed=0, n_boot=2000):
    """Median of the per-round times and a 95 % bootstrap interval of it (seconds in,
    microseconds out)."""
    import numpy as np
    x = np.asarray(rounds, dtype=np.float64)
    if x.size == 0:
        return None
    rng = np.random.default_rng(seed)
    boot = np.median(x[rng.integers(0, x.size, size=(n_boot, x.size))], axis=1)
    return {"rounds": int(x.size), "median_us": float(np.median(x)) * 1e6,
            "ci95_us": [float(np.percentile(boot, 2.5)) * 1e6, float(np.percentile(boot, 97.5)) * 1e6],
            "min_us": float(x.min()) * 1e6, "max_us": float(x.max()) * 1e6}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_arrays(x):
    q = x["q"].double().cpu().numpy()
    k = x["k"].cpu().float().numpy()
    v = x["v"].cpu().float().numpy()
    lens = x["seq_lens"].cpu().numpy()
    bt = None if x["block_table"] is None else x["block_table"].cpu().numpy()
    return q, k, v, lens, bt


def parity_sample(santa, run, w, S, mode, heads):
    """The timed configuration (KV copy 0, the timed launch) against the oracle on
    `heads`: idx exact outside the 1e-6 boundary window, boundary cases counted, o
    against the oracle's fp64 gather of the GPU's own idx.  The largest CDF
    difference compares the oracle's CDF with the one built (in fp64) from the
    GPU's own fp32 scores, read from the score pass's stash; the sample pass that
    follows consumes and clears the stash again."""
    import numpy as np
    from oracle import santa as O
    run.step(0)
    torch.cuda.synchronize()
    idx_gpu = run.idx.cpu().numpy().astype(np.int64)
    o_gpu = run.o.cpu().double().numpy()
    lay = santa.santa_workspace_layout_query(run.shape, S, mode)
    santa.santa_score_pass(*run.args(0))
    torch.cuda.synchronize()
    B, Hq = w.batch, w.q_heads
    row = lay.stash_row_bytes // 4
    stash = run.ws[lay.stash_offset:lay.stash_offset + B * Hq * lay.stash_row_bytes].view(torch.float32)
    stash = stash.view(B, Hq, row)
    s_gpu = {bh: stash[bh[0], bh[1]].double().cpu().numpy() for bh in heads}
    santa.santa_sample_pass(*run.args(0))
    torch.cuda.synchronize()
    q, k, v, lens, bt = _oracle_arrays(run.copies[0])
    res = O.decode(q, k, v, lens, bt, w.page_size, S, mode, w.sample_seed, heads=heads)
    rep = dict(heads=0, targets=0, boundary_cases=0, boundary_mismatches=0, far_mismatches=0,
               worst_rel_l2=0.0, max_abs_cdf_diff=0.0)
    for (b, h), r in res.items():
        n = int(r["n"])
        if n == 0:
            continue
        rep["heads"] += 1
        rep["targets"] += S
        near = r["delta"] < BOUNDARY_WINDOW
        bad = idx_gpu[b, h] != r["idx"]
        rep["boundary_cases"] += int(near.sum())
        rep["boundary_mismatches"] += int((bad & near).sum())
        rep["far_mismatches"] += int((bad & ~near).sum())
        g = h // w.group
        vals = O.sequence_keys(v, n, b, bt, w.page_size)[:, g, :].astype(np.float64)
        own = O.estimate(vals, idx_gpu[b, h])
        rep["worst_rel_l2"] = max(rep["worst_rel_l2"], float(np.linalg.norm(o_gpu[b, h] - own) /
                                                             max(np.linalg.norm(own), 1e-30)))
        F_gpu = O.cdf(O.softmax(s_gpu[(b, h)][:n]))
        rep["max_abs_cdf_diff"] = max(rep["max_abs_cdf_diff"], float(np.abs(F_gpu - r["F"]).max()))
    return rep


def cpu_baseline(w, x, S, mode, seconds):
    """The oracle on the host, one BLAS thread: full decode steps of the same
    workload (all heads), repeated until about `seconds` of CPU time."""
    from threadpoolctl import threadpool_limits
    from oracle import santa as O
    q, k, v, lens, bt = _oracle_arrays(x)
    heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)]
    done_heads = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 <= seconds:
            for i in range(0, len(heads), w.group):
                O.decode(q, k, v, lens, bt, w.page_size, S, mode, w.sample_seed, heads=heads[i:i + w.group])
                done_heads += w.group
                if time.perf_counter() - t0 > seconds:
                    break
        elapsed = time.perf_counter() - t0
    return {"value": done_heads / elapsed, "unit": "heads×batch/s", "cores": 1, "kind": "oracle",
            "sample": f"{done_heads} query heads of the {w.name} workload (NumPy fp64 oracle, one BLAS "
                      f"thread, {w.group} heads of one KV head per call) in {elapsed:.1f} s",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def step_record(santa, w, run, S, mode, t_step, rounds, calls):
    """Algorithmic traffic of `run`'s step: all K plus the distinct sampled V rows of
    each KV copy's call (their mean over the copies)."""
    uniq = []
    for c in range(len(run.copies)):
        run.step(c)
        torch.cuda.synchronize()
        uniq.append(W.unique_v_rows(run.idx.cpu(), w.group))
    lens = run.copies[0]["seq_lens"].cpu().tolist()
    u = sum(uniq) / len(uniq)
    alg = W.traffic_bytes(w, lens, int(round(u)))
    return {"step_us": t_step * 1e6, "calls_timed": calls, "rounds": round_stats(rounds),
            "algorithmic_bytes": alg, "unique_v_rows": u, "achieved_GBs": alg / t_step / 1e9,
            "frac_of_peak": alg / t_step / 1e9 / PEAK_HBM_GBS,
            "path": santa.santa_decode_path(run.shape, S, mode)}


def qwen_line(santa, steps, eager, dev):
    """The Qwen2.5-7B-shaped long-context step (one KV copy of 1 GiB: K alone is
    twice the Infinity Cache) for every sampling rule of the workload."""
    w = W.WORKLOADS["qwen128k"]
    S = w.samples[0]
    copies = make_copies(w, 1, dev)
    torch.cuda.synchronize()
    out = {"config": {"batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                      "seq_len": w.seq_len, "samples": S, "kv_copies": 1}}
    for mode in w.modes:
        run = Runner(santa, copies, S, mode, 0)
        for i in range(20):
            run.step(i)
        t, rounds, calls = timed(run.step, steps, eager, 1)
        rec = step_record(santa, w, run, S, mode, t, rounds, calls)
        rec["heads_x_batch_per_s"] = w.batch * w.q_heads / t
        out[W.MODE_NAMES[mode]] = rec
        del run
    lens = copies[0]["seq_lens"].cpu().tolist()
    out["dense_read_bytes"] = W.dense_read_bytes(w, lens)
    out["dense_read_us_at_peak"] = out["dense_read_bytes"] / (PEAK_HBM_GBS * 1e9) * 1e6
    del copies
    torch.cuda.empty_cache()
    return out


def bern_line(santa, steps, eager, dev, ncopies):
    """Bernoulli qK^T with the mean group query (B = 8 draws) on the Llama-shaped step
    with log-normal query channel scales, beside the exact step on the same inputs.
    Algorithmic bytes: the kept feature rows of K^T (count > 0) plus the distinct
    sampled V rows."""
    w = W.WORKLOADS["bern32k"]
    S, mode, B = w.samples[0], w.modes[0], w.bernoulli
    copies = make_copies(w, ncopies, dev)
    for x in copies:
        x["kt"] = W.keys_transposed(x)
    run = Runner(santa, copies, S, mode, 0)
    counts = torch.empty((w.batch, w.kv_heads, w.head_dim), dtype=torch.uint8, device=dev)

    def bern(c):
        x = copies[c % len(copies)]
        santa.santa_decode_bernoulli(run.shape, x["q"], x["kt"], x["v"], x["seq_lens"], S, mode, run.seed, B,
                                     run.o, run.idx, counts, run.ws)

    for i in range(20):
        bern(i)
    t_b, r_b, c_b = timed(bern, steps, eager, ncopies)
    t_e, r_e, c_e = timed(run.step, steps, eager, ncopies)
    lens = copies[0]["seq_lens"].cpu().tolist()
    k_read, feats, uniq = [], [], []
    for c in range(ncopies):
        bern(c)
        torch.cuda.synchronize()
        cnt = counts.cpu()
        kept = (cnt > 0).sum(dim=2)                       # [B, Hkv]
        k_read.append(sum(int(kept[b].sum()) * int(lens[b]) for b in range(w.batch)) * w.elem_bytes)
        feats.append(float((cnt > 0).double().mean()))
        uniq.append(W.unique_v_rows(run.idx.cpu(), w.group))
    kb = sum(k_read) / ncopies
    u = sum(uniq) / ncopies
    alg = kb + u * w.head_dim * w.elem_bytes
    out = {"config": {"batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                      "seq_len": w.seq_len, "samples": S, "mode": W.MODE_NAMES[mode], "draws": B,
                      "q_channel_sigma": w.q_channel_sigma, "kv_copies": ncopies},
           "step_us": t_b * 1e6, "calls_timed": c_b, "rounds": round_stats(r_b),
           "key_feature_access": sum(feats) / ncopies, "k_bytes_read": kb, "unique_v_rows": u,
           "algorithmic_bytes": alg, "achieved_GBs": alg / t_b / 1e9, "frac_of_peak": alg / t_b / 1e9 / PEAK_HBM_GBS,
           "exact_step_us": t_e * 1e6, "exact_rounds": round_stats(r_e)}
    del run, copies
    torch.cuda.empty_cache()
    return out


def pp_line(santa, steps, eager, dev, ncopies):
    """SANTA++ on the Qwen-shaped 32K layer (K = 31 teams per query head from S = 124,
    P = 16, R = 4; the team tables are built before timing), beside the exact SANTA
    step on the same caches.  Logical KV access counts, per KV head, the M
    representative keys plus the K and V rows of the union of the group's selected
    teams, over the 2 N rows of a dense read; the algorithmic bytes are those rows."""
    w = W.WORKLOADS["qwen32k"]
    P, R = 16, 4
    N = w.seq_len
    copies = make_copies(w, ncopies, dev)
    shape = santa.make_shape(copies[0]["q"], copies[0]["k"], None, max_seq_len=w.seq_len)
    tables = []
    for x in copies:
        t = santa.allocate_pp_table(shape, N, P, R, x["k"].dtype, dev)
        santa.santa_pp_build(shape, x["k"], x["v"], t)
        tables.append(t)
    M = tables[0]["M"]
    K = min(M, w.samples[0] // (P // R))
    B, Hq, d = copies[0]["q"].shape
    o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    teams = torch.empty((B, Hq, K + 1), dtype=torch.int32, device=dev)
    corr = torch.empty((B, Hq, K), dtype=torch.float32, device=dev)
    ws = torch.empty(santa.santa_pp_workspace_size(shape, N, P, R, K), dtype=torch.uint8, device=dev)

    def pp(c):
        x = copies[c % len(copies)]
        santa.santa_pp_decode(shape, x["q"], x["k"], x["v"], x["seq_lens"], tables[c % len(copies)], K,
                              w.sample_seed, o, teams, corr, ws)

    for i in range(20):
        pp(i)
    t_p, r_p, c_p = timed(pp, steps, eager, ncopies)
    run = Runner(santa, copies, w.samples[0], w.modes[0], 0)
    t_e, r_e, c_e = timed(run.step, steps, eager, ncopies)
    rows_read = []
    for c in range(ncopies):
        pp(c)
        torch.cuda.synchronize()
        ts = tables[c]["team_start"].cpu()
        sel = teams.cpu()[:, :, :K]
        total = 0
        for b in range(B):
            for g in range(w.kv_heads):
                u = torch.unique(sel[b, g * w.group:(g + 1) * w.group].reshape(-1)).long()
                total += int((ts[b, g, u + 1] - ts[b, g, u]).sum())
        rows_read.append(total)
    union_rows = sum(rows_read) / ncopies
    groups = B * w.kv_heads
    row = d * w.elem_bytes
    alg = groups * M * row + 2 * union_rows * row
    out = {"config": {"batch": B, "q_heads": Hq, "kv_heads": w.kv_heads, "head_dim": d, "prompt_tokens": N,
                      "parents": "contiguous", "P": P, "R": R, "S": w.samples[0], "teams_per_head": K,
                      "teams": M, "suffix_rows": 0, "kv_copies": ncopies},
           "step_us": t_p * 1e6, "calls_timed": c_p, "rounds": round_stats(r_p),
           "union_rows": union_rows, "logical_kv_access": (groups * M + 2 * union_rows) / (2 * groups * N),
           "algorithmic_bytes": alg, "achieved_GBs": alg / t_p / 1e9, "frac_of_peak": alg / t_p / 1e9 / PEAK_HBM_GBS,
           "exact_santa_step_us": t_e * 1e6, "exact_santa_rounds": round_stats(r_e)}
    del run, copies, tables
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import sampling_sparse_attention_amd as santa
    if not os.path.exists(santa.library_path):
        from sampling_sparse_attention_amd import build
        build.build()
    santa.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        t, gbs = copy_bandwidth(args.calibrate_copy)
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "copy_us": t * 1e6,
                          "read_plus_write_gbs": gbs}))
        return
    w = W.WORKLOADS[args.workload]
    S = args.samples or w.samples[0]
    mode = w.modes[-1] if args.mode is None else args.mode
    ncopies = max(1, args.kv_copies)
    print(f"[bench] generating {ncopies} copies of {w.name} "
          f"({2 * w.kv_cache_bytes() * ncopies / 2**30:.2f} GiB)", file=sys.stderr, flush=True)
    copies = make_copies(w, ncopies, dev)
    torch.cuda.synchronize()
    run = Runner(santa, copies, S, mode, args.split)
    lay = santa.santa_workspace_layout_query(run.shape, S, mode)

    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()
    print("[bench] timing steps", file=sys.stderr, flush=True)
    t_step, rounds, calls = timed(run.step, args.steps, args.eager, ncopies)
    head = step_record(santa, w, run, S, mode, t_step, rounds, calls)
    lens = copies[0]["seq_lens"].cpu().tolist()
    dense = W.dense_read_bytes(w, lens)
    achieved = head["achieved_GBs"]
    path = head["path"]

    extras = {}
    if not args.no_extras:
        print("[bench] timing the two-kernel path, flash, the Qwen step and a plain copy", file=sys.stderr,
              flush=True)
        side_steps = min(args.steps, 400)
        t_two, r_two, c_two = timed(run.two_kernel, side_steps, args.eager, ncopies)
        extras["two_kernel"] = {"step_us": t_two * 1e6, "calls_timed": c_two, "rounds": round_stats(r_two)}
        flash = {}
        if mode != W.MODE_MULTINOMIAL:
            # S^2ANTA-flash on the same inputs, at this S and at the page's flash
            # operating point S = 2048
            for S_f in sorted({S, 2048}):
                if S_f < lay.num_splits:
                    continue
                run_f = Runner(santa, copies, S_f, mode, args.split)
                t_f, r_f, c_f = timed(run_f.flash, side_steps, args.eager, ncopies)
                run_f.flash(0)
                torch.cuda.synchronize()
                u_f = W.unique_v_rows(run_f.idx.cpu(), w.group)
                b_f = W.traffic_bytes(w, lens, u_f)
                flash[f"S{S_f}"] = {"step_us": t_f * 1e6, "calls_timed": c_f, "unique_v_rows": u_f,
                                    "algorithmic_bytes": b_f, "achieved_GBs": b_f / t_f / 1e9}
                del run_f
        extras["flash"] = flash
        # the deterministic top-k comparator at the matched budget k = S
        run_k = Runner(santa, copies, S, W.MODE_SYSTEMATIC, args.split)
        t_k, r_k, c_k = timed(run_k.topk, side_steps, args.eager, ncopies)
        run_k.topk(0)
        torch.cuda.synchronize()
        u_k = W.unique_v_rows(run_k.idx.cpu(), w.group)
        b_k = W.traffic_bytes(w, lens, u_k)
        extras["topk"] = {"k": S, "step_us": t_k * 1e6, "calls_timed": c_k, "unique_v_rows": u_k,
                          "algorithmic_bytes": b_k, "achieved_GBs": b_k / t_k / 1e9}
        del run_k
        t_copy, copy_gbs = copy_bandwidth(1 << 30)
        extras["copy"] = {"bytes": 1 << 30, "copy_us": t_copy * 1e6, "read_plus_write_GBs": copy_gbs,
                          "frac_of_peak": copy_gbs / PEAK_HBM_GBS}

    rec = {
        "metric": METRIC,
        "value": w.batch * w.q_heads / t_step,
        "unit": "heads×batch/s",
        "n_gpus": 1,
        "steps": calls,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "seq_len": w.seq_len, "samples": S,
                   "mode": W.MODE_NAMES[mode], "split_size": lay.split_size,
                   "kv_copies": ncopies, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": {"bound": "hbm",
                     "kernel": "score_kernel+sample_kernel" if path == santa.PATH_TWO_KERNELS else "fused_kernel",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": counter_traffic(w.name),
                     "bytes_per_launch": head["algorithmic_bytes"], "avg_launch_us": t_step * 1e6},
        "step": {"decode_us": t_step * 1e6, "decode_rounds": head["rounds"], "decode_path": path,
                 "algorithmic_bytes": head["algorithmic_bytes"],
                 "k_bytes": int(sum(lens)) * w.kv_heads * w.head_dim * w.elem_bytes,
                 "unique_v_rows": head["unique_v_rows"], "dense_read_bytes": dense,
                 "dense_read_us_at_peak": dense / (PEAK_HBM_GBS * 1e9) * 1e6, **extras},
        "parity": None,
        "cpu_baseline": None,
    }
    if "copy" in extras:
        c = extras["copy"]["read_plus_write_GBs"]
        rec["roofline"]["measured_copy_GBs"] = c
        rec["roofline"]["frac_of_measured_copy"] = achieved / c
        rec["step"]["dense_read_us_at_measured_copy"] = dense / (c * 1e9) * 1e6
    if not args.no_extras and args.workload == "llama32k":
        print("[bench] timing the Qwen-shaped step and Bernoulli qK^T", file=sys.stderr, flush=True)
        del copies, run
        torch.cuda.empty_cache()
        rec["qwen128k"] = qwen_line(santa, min(args.steps, 400), args.eager, dev)
        rec["bernoulli"] = bern_line(santa, min(args.steps, 400), args.eager, dev, ncopies)
        rec["santa_pp"] = pp_line(santa, min(args.steps, 400), args.eager, dev, ncopies)
        copies = make_copies(w, 1, dev)
        run = Runner(santa, copies, S, mode, args.split)
    if not args.no_cpu_baseline:
        print("[bench] oracle: parity sample and CPU timing", file=sys.stderr, flush=True)
        heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)][:64]
        rec["parity"] = parity_sample(santa, run, w, S, mode, heads)
        rec["cpu_baseline"] = cpu_baseline(w, copies[0], S, mode, args.cpu_seconds)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
