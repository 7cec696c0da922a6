"""santa_decode_bernoulli (Bernoulli qK^T with the mean group query, then SANTA)
against oracle/bernoulli.py through the C ABI.

* The feature counts of every (sequence, KV head) are bit-exact: both sides take
  the stratified keep decisions in fp64 from the same Philox4x64-10 draws.
* The sampled indices equal the oracle's, which samples from its fp64
  estimated scores, except for targets within a CDF window of an interval
  edge.  The window is 1e-6 (the exact path's) plus twice the p-weighted bound
  on the GPU's fp32 score error.  The library states its summation: the
  weights are rounded once to fp32, the kept features (ascending) are dealt
  round-robin to F groups, each group sums its terms by fused multiply-adds in
  order and the group sums are added pairwise.  The bound below covers every
  such split (F a power of two up to 32; F = 1 is the sequential sum): to
  first order the error of key j's score is at most 2^-24 times (the sum of
  |w_f k_jf| for the weights' rounding, plus the magnitudes of every group's
  running sums, plus log2(F) times the sum of |w_f k_jf| for the pairwise
  additions); the test takes the largest of these over every F, divides by
  sqrt(d) and adds the rounding of the 1/sqrt(d) scale.  A CDF moves by at
  most twice the p-weighted mean of the scores' errors.
* o lies within 1e-3 relative L2 of the fp64 gather-mean of the GPU's own
  indices.

Inputs: the seeded workloads with log-normal query channel scales (sigma 0.8),
small ones spanning several splits and a ragged tail, every built shape, a
zero query and one-channel queries (exact estimated scores), and the
Llama-shaped step, the batched step (fused kernel with tickets) and the
Qwen-shaped step (two kernels) at full size on sampled heads."""
import math

import numpy as np
import pytest
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from oracle import bernoulli as BQ
from oracle import santa as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    santa.library()


def _inputs(G=4, d=128, dtype="bf16", lens=(1000, 1537, 64, 17), seed=3, sigma=0.8, B=8):
    w = W.Workload("bern_small", batch=len(lens), q_heads=2 * G, kv_heads=2, head_dim=d, seq_len=max(lens),
                   dtype=dtype, sinks=2, sink_scale=6.0, q_channel_sigma=sigma, bernoulli=B)
    x = W.make_inputs(w, seed=seed)
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    print(f"[case] bernoulli G={G} d={d} {dtype} lens={lens} B={B}", flush=True)
    x = H.to_device(x)
    x["kt"] = W.keys_transposed(x)
    return x


def run_bern(x, S, mode, seed, B, split=0, workspace=None):
    w = x["workload"]
    shape = santa.make_shape(x["q"], x["v"], None, max_seq_len=w.seq_len, split_size=split)
    Bs, Hq, d = x["q"].shape
    dev = x["q"].device
    o = torch.full((Bs, Hq, d), float("nan"), dtype=torch.float32, device=dev)
    idx = torch.full((Bs, Hq, S), -7, dtype=torch.int32, device=dev)
    counts = torch.full((Bs, w.kv_heads, d), 255, dtype=torch.uint8, device=dev)
    ws = workspace if workspace is not None else santa.allocate_workspace(shape, S, mode, dev)
    santa.santa_decode_bernoulli(shape, x["q"], x["kt"], x["v"], x["seq_lens"], S, mode, seed, B, o, idx,
                                 counts, ws)
    torch.cuda.synchronize()
    return o.cpu(), idx.cpu(), counts.cpu(), ws


def score_window(q_group, k, counts, B, h, s):
    """CDF window of head h of the group: 1e-6 + 2 * sum_j p_j e_j, e_j the bound on the
    fp32 error of the scaled score s_j (see the module docstring)."""
    d = q_group.shape[1]
    m = BQ.mean_group_query(q_group)
    top = m.max()
    if top == 0:
        return H.BOUNDARY_WINDOW
    ratio = np.divide((top / B) * counts, m, out=np.zeros_like(m), where=m > 0)
    feats = np.nonzero(counts)[0]
    terms = k[:, feats] * (q_group[h] * ratio)[feats]
    mag = np.abs(terms).sum(1)
    worst = np.zeros(len(k))
    for lg in range(6):                      # F = 1, 2, 4, ..., 32 lane groups
        F = 1 << lg
        run = sum(np.abs(np.cumsum(terms[:, r::F], axis=1)).sum(1) for r in range(F))
        worst = np.maximum(worst, run + lg * mag)
    e = 2.0 ** -24 * (worst + mag) / math.sqrt(d) + 2.0 ** -23 * np.abs(s)
    p = np.exp(s - s.max())
    p /= p.sum()
    return H.BOUNDARY_WINDOW + 2.0 * float((p * e).sum())


def check_bern(x, S, mode, seed, B, o, idx, counts, heads=None, label=None):
    """Counts of every group bit-exact; the heads ``heads`` (default: all) against the oracle."""
    w = x["workload"]
    G, d = w.group, w.head_dim
    lens = x["seq_lens"].cpu()
    q = x["q"].double().cpu().numpy()
    rep = H.ParityReport()
    if heads is None:
        heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)]
    by_group = {}
    for b, h in heads:
        by_group.setdefault((b, h // G), []).append(h % G)
    for b in range(w.batch):
        for g in range(w.kv_heads):
            qg = q[b, g * G:(g + 1) * G]
            want = BQ.feature_counts(BQ.mean_group_query(qg), B, seed, b, g)
            got = counts[b, g].numpy().astype(np.int64)
            assert np.array_equal(got, want), (f"counts (b={b}, g={g}): {int((got != want).sum())} features "
                                               f"differ, first {np.nonzero(got != want)[0][:4]}")
    for (b, g), hs in by_group.items():
        n = int(lens[b])
        if n == 0:
            for hh in hs:
                assert torch.all(idx[b, g * G + hh] == -1) and torch.all(o[b, g * G + hh] == 0), \
                    f"empty sequence {b}"
            continue
        qg = q[b, g * G:(g + 1) * G]
        k, v = H.head_rows(x, b, g)
        s_hat, c = BQ.estimated_scores(qg, k, B, seed, b, g)
        for hh in hs:
            s = s_hat[hh] / math.sqrt(d)
            hq = g * G + hh
            ridx, t, F, p = O.sample_head(s, S, mode, seed, b, hq)
            ref = dict(idx=ridx, t=t, F=F, p=p, v=v, delta=O.boundary_distance(F, ridx, t))
            win = score_window(qg, k, c, B, hh, s)
            H.check_head(rep, ref, idx[b, hq].numpy().astype(np.int64), o[b, hq].double().numpy(),
                         f"bernoulli (b={b}, h={hq}, mode={mode}, S={S}, B={B})", window=win)
    H.record(label or f"bernoulli {w.name} B{w.batch} {w.q_heads}/{w.kv_heads} d{w.head_dim} n{w.seq_len} "
                      f"{w.dtype} S{S} {W.MODE_NAMES[mode]} draws{B}", rep)
    return rep


@pytest.mark.parametrize("B", [1, 8, 12, 64])          # 12: a B that is not a power of two
def test_bernoulli_small_bf16_gqa4(B):
    x = _inputs(B=B)
    o, idx, counts, ws = run_bern(x, 256, W.MODE_SYSTEMATIC, 11, B)
    print(check_bern(x, 256, W.MODE_SYSTEMATIC, 11, B, o, idx, counts))
    assert santa.santa_workspace_status(ws) == 0
    assert torch.count_nonzero(ws) == 0          # the workspace is returned to zero


@pytest.mark.parametrize("mode", [W.MODE_MULTINOMIAL, W.MODE_STRATIFIED])
def test_bernoulli_sampling_modes(mode):
    x = _inputs(lens=(2500, 333), seed=5)
    o, idx, counts, _ = run_bern(x, 64, mode, 7, 8)
    print(check_bern(x, 64, mode, 7, 8, o, idx, counts))


@pytest.mark.parametrize("G,d,dtype", [(1, 64, "f32"), (7, 128, "bf16"), (8, 64, "bf16"), (2, 128, "f32")])
def test_bernoulli_shapes(G, d, dtype):
    x = _inputs(G=G, d=d, dtype=dtype, lens=(3001, 700, 1, 0), seed=G)
    # 64: a quarter of a row per wave; 256 .. 1024: whole feature rows per wave
    # (bf16 512 / 1024 and fp32 256 / 512 / 1024 are one, two and four key blocks)
    for split in (0, 64, 256, 512, 1024):
        o, idx, counts, _ = run_bern(x, 128, W.MODE_SYSTEMATIC, 2, 8, split=split)
        print(split, check_bern(x, 128, W.MODE_SYSTEMATIC, 2, 8, o, idx, counts))


def test_bernoulli_zero_and_one_channel_queries():
    """A zero query keeps no feature (every score 0: uniform sampling); a group whose
    queries share one nonzero channel keeps it B times and its scores are exact."""
    x = _inputs(lens=(1500, 900), seed=9)
    q = torch.zeros_like(x["q"])
    q[1, 4:8, 17] = torch.tensor([1.5, -2.0, 0.25, 3.0], dtype=q.dtype)
    x["q"] = q
    o, idx, counts, _ = run_bern(x, 256, W.MODE_SYSTEMATIC, 4, 8)
    assert int(counts[0].sum()) == 0 and int(counts[1, 0].sum()) == 0
    assert counts[1, 1, 17] == 8 and int(counts[1, 1].sum()) == 8
    print(check_bern(x, 256, W.MODE_SYSTEMATIC, 4, 8, o, idx, counts))


def test_bernoulli_workspace_reuse_across_shapes():
    """One workspace serves a large then a small problem, then the exact path."""
    x1 = _inputs(lens=(4000, 2000), seed=12)
    x2 = _inputs(G=8, d=64, lens=(300,), seed=13)
    shape1 = santa.make_shape(x1["q"], x1["v"], None, max_seq_len=x1["workload"].seq_len)
    ws = santa.allocate_workspace(shape1, 256, W.MODE_MULTINOMIAL, x1["q"].device)
    for x, mode in ((x1, W.MODE_MULTINOMIAL), (x2, W.MODE_SYSTEMATIC), (x1, W.MODE_STRATIFIED)):
        o, idx, counts, _ = run_bern(x, 256, mode, 3, 8, workspace=ws)
        check_bern(x, 256, mode, 3, 8, o, idx, counts)
        assert santa.santa_workspace_status(ws) == 0
    o, idx, ws2, _ = H.run_hip(x1, 256, W.MODE_SYSTEMATIC, 3)
    H.check_all(x1, 256, W.MODE_SYSTEMATIC, 3, o, idx)


def _full(name, base, **kw):
    w = W.WORKLOADS[base].replace(name=name, q_channel_sigma=0.8, bernoulli=8, **kw)
    x = W.make_inputs(w, seed=0, device="cuda")
    x["kt"] = W.keys_transposed(x)
    return x


def test_bernoulli_llama32k_full():
    x = _full("bern32k", "llama32k")
    print("[case] bernoulli llama32k B=8 S=256", flush=True)
    o, idx, counts, _ = run_bern(x, 256, W.MODE_SYSTEMATIC, 1, 8)
    frac = float((counts > 0).double().mean())
    print(check_bern(x, 256, W.MODE_SYSTEMATIC, 1, 8, o, idx, counts), f"features read {frac:.3f}")
    assert 0.5 < frac < 0.9


def test_bernoulli_batched_full_sampled_heads():
    x = _full("bern_batched", "batched")
    w = x["workload"]
    print("[case] bernoulli batched B=8 S=128", flush=True)
    o, idx, counts, _ = run_bern(x, 128, W.MODE_STRATIFIED, 1, 8)
    heads = [(b, g * w.group + (3 * b + g) % w.group) for b in range(w.batch) for g in range(w.kv_heads)
             if (b + g) % 4 == 0]
    print(check_bern(x, 128, W.MODE_STRATIFIED, 1, 8, o, idx, counts, heads=heads))


def test_bernoulli_qwen128k_full_sampled_heads():
    x = _full("bern_qwen128k", "qwen128k")
    w = x["workload"]
    print("[case] bernoulli qwen128k B=8 S=1024", flush=True)
    o, idx, counts, _ = run_bern(x, 1024, W.MODE_SYSTEMATIC, 1, 8)
    heads = [(b, g * w.group + (b + g) % w.group) for b in range(w.batch) for g in range(w.kv_heads)]
    print(check_bern(x, 1024, W.MODE_SYSTEMATIC, 1, 8, o, idx, counts, heads=heads))
