"""Benchmark of one SANTA decode step on one MI355X.

A step is one ``santa_decode`` call over one batch of synthetic input: the
fused kernel (scores, global partition function, sampling and gather in one
launch), plus the target sort for multinomial sampling.  The default workload is the Llama-3.1-8B-shaped layer:
batch 1, 32 query / 8 KV heads, d = 128, 32768 bf16 keys, S = 256 systematic
samples.  ``--kv-copies`` independent caches (default 8, 1 GiB) are cycled
through, one per step like the layers of a model, so that K is read from HBM
and not from the 256 MB Infinity Cache.

The timed steps are graph replays split into 10 rounds; the line reports the mean
over all of them as the value and, beside it, the median of the round means with
a 95 % bootstrap interval.

Prints one JSON line: throughput in heads x batch per second, the roofline of
the dominant kernel (the fused decode kernel, bound by HBM bandwidth: all of K
plus the distinct sampled V rows per launch), the two-kernel path's stage
times for comparison, and the CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
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
KERNEL_SOURCES = ["santa_fused.hip", "santa_split.h", "santa_device.h", "santa_internal.h"]


def strip_comments(text: str) -> str:
    """C/C++ source without its comments and blank lines (string literals in these
    sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(read=None) -> str:
    """Hash of the fused kernel's sources, comments left out (a comment edit
    does not change the kernel the counters were taken on)."""
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
    """HBM bytes per fused-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"fused_kernel_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="llama32k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--samples", type=int, default=None)
    ap.add_argument("--mode", type=int, default=None)
    ap.add_argument("--split", type=int, default=0, help="keys per split (0: library default)")
    ap.add_argument("--kv-copies", type=int, default=8)
    ap.add_argument("--eager", action="store_true", help="launch every call from Python, no HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run plain device-to-device copies of BYTES bytes (the reference kernel "
                         "for scaling HBM byte counters) and print their bandwidth")
    return ap.parse_args()


def calibrate_copy(nbytes: int, reps: int = 10):
    """Plain copies of a known size: what FETCH_SIZE / WRITE_SIZE read for them
    converts the counters of the SANTA kernels into bytes."""
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
    print(json.dumps({"calibrate_copy_bytes": nbytes, "reps": reps, "copy_us": t * 1e6,
                      "read_plus_write_gbs": 2 * nbytes / t / 1e9}))


def make_copies(w, n, device):
    copies = []
    for c in range(n):
        copies.append(W.make_inputs(w, seed=c, device=device))
    return copies


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

    def _args(self, c):
        x = self.copies[c % len(self.copies)]
        return (self.shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], self.S, self.mode,
                self.seed, self.o, self.idx, self.ws)

    def step(self, c):
        self.santa.santa_decode(*self._args(c))

    def score(self, c):
        self.santa.santa_score_pass(*self._args(c))

    def sample(self, c):
        self.santa.santa_sample_pass(*self._args(c))


def timed(fn, reps, eager, ncopies):
    """Average GPU time per call of fn(c), measured with events on the launch
    stream: replays of a captured graph of `ncopies` calls, or eager calls."""
    stream = torch.cuda.current_stream()
    if eager:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(reps):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps * 1e-3
    per_graph = ncopies * max(1, 32 // ncopies)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for i in range(per_graph):
            fn(i)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            fn(i)
    torch.cuda.synchronize()
    replays = max(1, reps // per_graph)
    graph.replay()
    torch.cuda.synchronize()
    # events at round boundaries (ROUNDS rounds of about equal length) on the
    # launch stream; the whole interval gives the mean, the rounds its spread
    nr = min(ROUNDS, replays)
    marks = [round(i * replays / nr) for i in range(nr + 1)]
    events = [torch.cuda.Event(enable_timing=True) for _ in range(nr + 1)]
    events[0].record(stream)
    for r in range(nr):
        for _ in range(marks[r + 1] - marks[r]):
            graph.replay()
        events[r + 1].record(stream)
    torch.cuda.synchronize()
    LAST_ROUNDS[:] = [events[r].elapsed_time(events[r + 1]) / ((marks[r + 1] - marks[r]) * per_graph) * 1e-3
                      for r in range(nr)]
    return events[0].elapsed_time(events[-1]) / (replays * per_graph) * 1e-3


ROUNDS = 10
LAST_ROUNDS = []        # seconds per call in each round of the last graph-timed call of timed()


def round_stats(rounds, seed=0, n_boot=2000):
    """Median of the per-round times and a 95 % bootstrap interval of it (seconds)."""
    import numpy as np
    x = np.asarray(rounds, dtype=np.float64)
    if x.size == 0:
        return None
    rng = np.random.default_rng(seed)
    boot = np.median(x[rng.integers(0, x.size, size=(n_boot, x.size))], axis=1)
    return {"rounds": int(x.size), "median_us": float(np.median(x)) * 1e6,
            "ci95_us": [float(np.percentile(boot, 2.5)) * 1e6, float(np.percentile(boot, 97.5)) * 1e6],
            "min_us": float(x.min()) * 1e6, "max_us": float(x.max()) * 1e6}


def cpu_baseline(w, x_gpu, S, mode, seconds):
    """The oracle on the host: full decode steps of the same workload (all heads),
    repeated until about `seconds` of CPU time."""
    import numpy as np
    from oracle import santa as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    q = x_gpu["q"].double().cpu().numpy()
    k = x_gpu["k"].cpu().float().numpy()
    v = x_gpu["v"].cpu().float().numpy()
    lens = x_gpu["seq_lens"].cpu().numpy()
    bt = None if x_gpu["block_table"] is None else x_gpu["block_table"].cpu().numpy()
    heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)]
    # bounded sample: whole steps if they fit in the budget, else a prefix of heads
    done_heads = 0
    t0 = time.perf_counter()
    while True:
        for i in range(0, len(heads), w.group):
            O.decode(q, k, v, lens, bt, w.page_size, S, mode, w.sample_seed, heads=heads[i:i + w.group])
            done_heads += w.group
            if time.perf_counter() - t0 > seconds and done_heads >= w.group:
                break
        if time.perf_counter() - t0 > seconds:
            break
    elapsed = time.perf_counter() - t0
    return {"value": done_heads / elapsed, "unit": "heads×batch/s", "cores": int(blas),
            "kind": "oracle",
            "sample": f"{done_heads} query heads of the {w.name} workload (NumPy fp64 oracle, "
                      f"{w.group} heads of one KV head per call) in {elapsed:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
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
        calibrate_copy(args.calibrate_copy)
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
    t_step = timed(run.step, args.steps, args.eager, ncopies)
    step_rounds = None if args.eager else round_stats(LAST_ROUNDS)
    # the two-kernel path (score pass + sample pass), for comparison
    t_two = timed(lambda c: (run.score(c), run.sample(c)), args.steps, args.eager, ncopies)
    # S^2ANTA-flash (santa_decode_flash) on the same inputs, at this S and at the
    # page's flash operating point S = 2048: reported beside the headline
    flash = {}
    if mode != W.MODE_MULTINOMIAL:
        for S_f in sorted({S, 2048}):
            if S_f < lay.num_splits:
                continue
            run_f = Runner(santa, copies, S_f, mode, args.split)
            call = lambda c, r=run_f: santa.santa_decode_flash(*r._args(c))
            t_f = timed(call, args.steps, args.eager, ncopies)
            call(0)
            torch.cuda.synchronize()
            u_f = W.unique_v_rows(run_f.idx.cpu(), w.group)
            b_f = W.traffic_bytes(w, copies[0]["seq_lens"].cpu().tolist(), u_f)
            flash[f"S{S_f}"] = {"step_us": t_f * 1e6, "unique_v_rows": u_f, "algorithmic_bytes": b_f,
                                "achieved_GBs": b_f / t_f / 1e9}
            del run_f

    # algorithmic traffic of one step: all K rows + distinct sampled V rows
    lens = copies[0]["seq_lens"].cpu()
    uniq = []
    for c in range(ncopies):
        run.step(c)
        torch.cuda.synchronize()
        uniq.append(W.unique_v_rows(run.idx.cpu(), w.group))
    uniq_mean = sum(uniq) / len(uniq)
    alg_bytes = W.traffic_bytes(w, lens.tolist(), int(round(uniq_mean)))
    dense = W.dense_read_bytes(w, lens.tolist())
    achieved = alg_bytes / t_step / 1e9
    traffic = counter_traffic(w.name)
    path = santa.santa_decode_path(run.shape, S, mode)

    rec = {
        "metric": METRIC,
        "value": w.batch * w.q_heads / t_step,
        "unit": "heads×batch/s",
        "n_gpus": 1,
        "steps": args.steps,
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
                     "kernel": "fused_kernel" if path == santa.PATH_FUSED else "score+sample",
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "bytes_per_launch": alg_bytes, "avg_launch_us": t_step * 1e6},
        "step": {"decode_us": t_step * 1e6, "decode_rounds": step_rounds, "decode_path": path,
                 "two_kernel_step_us": t_two * 1e6, "flash": flash,
                 "algorithmic_bytes": alg_bytes, "k_bytes": int(lens.sum()) * w.kv_heads * w.head_dim * w.elem_bytes,
                 "unique_v_rows": uniq_mean, "dense_read_bytes": dense,
                 "dense_read_us_at_peak": dense / (PEAK_HBM_GBS * 1e9) * 1e6},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, copies[0], S, mode, args.cpu_seconds)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
