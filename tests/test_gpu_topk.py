"""santa_decode_topk (the top-k comparator) against oracle/topk.py through the
C ABI: small seeded inputs spanning several splits and a ragged tail, every
shape the kernels are built for, ties, sequences shorter than k, and the
Llama- and Qwen-shaped workloads at full size.

The kept set must equal the oracle's, except for keys whose fp64 score lies
within the fp32 rounding bound of the scores from the k-th largest score (on
either side of the selection edge): those are counted as boundary cases.  o
must lie within 1e-3 relative L2 of the oracle's renormalised attention over
the GPU's own kept set."""
import numpy as np
import pytest
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from oracle import topk as T
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    santa.library()


def _inputs(G=4, d=128, dtype="bf16", lens=(1000, 1537, 64, 17), page_size=0, seed=3, sinks=2):
    n_max = max(lens)
    if page_size:
        n_max = -(-n_max // page_size) * page_size
    w = W.Workload("small", batch=len(lens), q_heads=2 * G, kv_heads=2, head_dim=d, seq_len=n_max, dtype=dtype,
                   page_size=page_size, sinks=sinks, sink_scale=6.0)
    x = W.make_inputs(w, seed=seed)
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    print(f"[case] topk G={G} d={d} {dtype} lens={lens} page={page_size}", flush=True)
    return H.to_device(x)


def run_topk(x, k, split=0):
    shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len, split_size=split)
    B, Hq, d = x["q"].shape
    o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=x["q"].device)
    idx = torch.full((B, Hq, k), -7, dtype=torch.int32, device=x["q"].device)
    ws = santa.allocate_workspace(shape, k, W.MODE_SYSTEMATIC, x["q"].device)
    santa.santa_decode_topk(shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], k, o, idx, ws)
    torch.cuda.synchronize()
    return o.cpu(), idx.cpu(), ws


def check_topk(x, k, o, idx, heads=None, label=None):
    w = x["workload"]
    rep = H.ParityReport()
    lens = x["seq_lens"].cpu()
    if heads is None:
        heads = [(b, h) for b in range(w.batch) for h in range(w.q_heads)]
    rows = {}
    for b, h in heads:
        n = int(lens[b])
        ig = idx[b, h].numpy().astype(np.int64)
        where = f"topk (b={b}, h={h}, k={k})"
        if n == 0:
            assert np.all(ig == -1) and torch.all(o[b, h] == 0), where
            continue
        g = h // w.group
        if (b, g) not in rows:
            rows.clear()
            rows[(b, g)] = H.head_rows(x, b, g)
        kk, vv = rows[(b, g)]
        q = x["q"][b, h].double().cpu().numpy()
        s = T.scores(q, kk)
        kept = T.select(s, k)
        m = len(kept)
        assert np.all(ig[m:] == -1), f"{where}: padding"
        got = ig[:m]
        assert np.all(got[1:] > got[:-1]) and got.min() >= 0 and got.max() < n, f"{where}: idx not ascending/in range"
        # fp32 rounding bound of each score: the bf16 (or fp32) products summed in fp32
        bound = 2.0 * (w.head_dim + 2) * 2.0 ** -24 * (np.abs(kk) @ np.abs(q)) / np.sqrt(w.head_dim)
        thr = T.threshold(s, k)
        kth = kept[np.argmin(s[kept])]
        near = np.abs(s - thr) <= bound + bound[kth]
        diff = np.setxor1d(got, kept)
        rep.heads += 1
        rep.targets += m
        rep.boundary += int(near[kept].sum())
        assert np.all(near[diff]), f"{where}: {int((~near[diff]).sum())} keys differ away from the selection edge"
        rep.boundary_mismatch += len(diff) // 2
        own = T.estimate(s, vv, got)
        err = float(np.linalg.norm(o[b, h].double().numpy() - own) / max(np.linalg.norm(own), 1e-30))
        rep.worst_rel_l2 = max(rep.worst_rel_l2, err)
        assert err <= H.O_REL_L2, f"{where}: o relative L2 error {err:.3e}"
    H.record(label or f"topk {w.name} B{w.batch} {w.q_heads}/{w.kv_heads} d{w.head_dim} {w.dtype} k{k}", rep)
    return rep


@pytest.mark.parametrize("k", [1, 64, 300, 2000])
def test_topk_small_bf16_gqa4(k):
    x = _inputs()
    o, idx, ws = run_topk(x, k)
    print(check_topk(x, k, o, idx))
    assert santa.santa_workspace_status(ws) == 0
    assert torch.count_nonzero(ws) == 0          # the stash is returned to zero


@pytest.mark.parametrize("G,d,dtype,page", [(1, 64, "f32", 0), (7, 128, "bf16", 0), (8, 64, "bf16", 32),
                                            (2, 128, "f32", 16)])
def test_topk_shapes(G, d, dtype, page):
    x = _inputs(G=G, d=d, dtype=dtype, lens=(3001, 700, 1, 0), page_size=page)
    for k in (16, 777):
        o, idx, ws = run_topk(x, k)
        print(check_topk(x, k, o, idx))


def test_topk_equal_scores_keep_the_first_keys():
    x = _inputs(lens=(2048, 500))
    x["q"] = torch.zeros_like(x["q"])
    o, idx, _ = run_topk(x, 300)
    assert torch.equal(idx[0, 0], torch.arange(300, dtype=torch.int32))
    assert torch.equal(idx[1, 3], torch.arange(300, dtype=torch.int32))
    check_topk(x, 300, o, idx)


def test_topk_maximum_k_and_sequences_shorter_than_k():
    x = _inputs(lens=(9000, 8192, 100))
    o, idx, _ = run_topk(x, 8192)
    print(check_topk(x, 8192, o, idx))
    assert bool((idx[2, :, 100:] == -1).all())


def test_topk_llama32k_full():
    w = W.WORKLOADS["llama32k"]
    x = W.make_inputs(w, seed=0, device="cuda")
    print("[case] topk llama32k k=256", flush=True)
    o, idx, _ = run_topk(x, 256)
    print(check_topk(x, 256, o, idx))


def test_topk_qwen128k_sampled_heads():
    w = W.WORKLOADS["qwen128k"]
    x = W.make_inputs(w, seed=0, device="cuda")
    print("[case] topk qwen128k k=1024", flush=True)
    o, idx, _ = run_topk(x, 1024)
    heads = [(b, g * w.group + (b + g) % w.group) for b in range(w.batch) for g in range(w.kv_heads)]
    print(check_topk(x, 1024, o, idx, heads=heads))
