"""HIP path vs the oracle on small seeded inputs that span several splits and a
ragged tail (every call goes through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import sampling_sparse_attention_amd as santa
import workloads as W
from oracle import santa as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.ensure_built()
    santa.library()


def _inputs(G=4, d=128, dtype="bf16", lens=(1000, 1537, 64, 17), page_size=0, n_max=None, seed=3,
            q_scale=1.0, sinks=2):
    n_max = n_max or max(lens)
    if page_size:
        n_max = -(-n_max // page_size) * page_size
    w = W.Workload("small", batch=len(lens), q_heads=2 * G, kv_heads=2, head_dim=d, seq_len=n_max,
                   dtype=dtype, page_size=page_size, q_scale=q_scale, sinks=sinks, sink_scale=6.0)
    x = W.make_inputs(w, seed=seed)
    x["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    print(f"[case] G={G} d={d} {dtype} lens={lens} page={page_size}", flush=True)
    return H.to_device(x)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("S", [1, 64, 300])
def test_decode_small_bf16_gqa4(mode, S):
    x = _inputs()
    o, idx, _, _ = H.run_hip(x, S, mode, seed=11)
    rep = H.check_all(x, S, mode, 11, o, idx)
    print(rep)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_many_splits_per_sequence(mode):
    """64-key splits over sequences of 101 and 301 splits: the cross-split merge
    then holds two and eight split records per lane (one and four are covered by
    the 32k and 128k workloads)."""
    # two sequences: 1204 work items, more than the device holds at once (two-kernel path)
    x = _inputs(lens=(64 * 100 + 37, 64 * 300 + 5))
    o, idx, _, _ = H.run_hip(x, 300, mode, seed=17, split=64)
    print(H.check_all(x, 300, mode, 17, o, idx))
    # one sequence of 301 splits: 602 work items (fused kernel)
    x = _inputs(lens=(64 * 300 + 5,))
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len, split_size=64)
    assert santa.santa_decode_path(shape, 300, mode) == santa.PATH_FUSED
    o, idx, _, _ = H.run_hip(x, 300, mode, seed=17, split=64)
    print(H.check_all(x, 300, mode, 17, o, idx))


@pytest.mark.parametrize("mode,S", [(0, 8192), (1, 65535), (2, 65535)])
def test_maximum_sample_counts(mode, S):
    """The largest S each rule is built for (8192 sorted multinomial targets,
    65535 stratified or systematic ones): thousands of targets per split, placed
    in chunks of 256, and idx rows of S entries."""
    x = _inputs(lens=(3000, 1200))
    o, idx, _, _ = H.run_hip(x, S, mode, seed=13)
    print(H.check_all(x, S, mode, 13, o, idx))


@pytest.mark.parametrize("per_split", [31, 32, 33, 64])
@pytest.mark.parametrize("mode", [1, 2])
def test_sampler_paths_at_the_few_target_limit(per_split, mode):
    """q = 0 makes every score 0, so the 2048 keys have equal mass and the
    stratified or systematic targets fall evenly: S = 4 * per_split puts
    exactly per_split of them into each of the four 512-key splits.  Up to 32
    targets a split places one target per lane, above that it counts targets
    per key; both must reproduce the oracle's indices."""
    x = _inputs(lens=(2048,), q_scale=0.0, sinks=0)
    S = 4 * per_split
    o, idx, _, _ = H.run_hip(x, S, mode, seed=7, split=512)
    print(H.check_all(x, S, mode, 7, o, idx))


@pytest.mark.parametrize("split", [64, 128, 512, 1024])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decode_split_sizes(split, mode):
    x = _inputs(lens=(2049, 700, 1))
    o, idx, _, _ = H.run_hip(x, 96, mode, seed=5, split=split)
    print(H.check_all(x, 96, mode, 5, o, idx))


@pytest.mark.parametrize("G,d,dtype", [(1, 64, "f32"), (1, 128, "bf16"), (2, 64, "bf16"),
                                       (4, 64, "f32"), (7, 128, "bf16"), (8, 128, "bf16"),
                                       (8, 128, "f32"), (2, 128, "f32")])
@pytest.mark.parametrize("mode", [0, 2])
def test_decode_group_dim_dtype(G, d, dtype, mode):
    x = _inputs(G=G, d=d, dtype=dtype, lens=(777, 1300))
    o, idx, _, _ = H.run_hip(x, 128, mode, seed=2)
    print(H.check_all(x, 128, mode, 2, o, idx))


@pytest.mark.parametrize("page_size", [16, 32, 256])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_decode_paged(page_size, mode):
    x = _inputs(lens=(1000, 1537, 333), page_size=page_size)
    o, idx, _, _ = H.run_hip(x, 200, mode, seed=8)
    print(H.check_all(x, 200, mode, 8, o, idx))


def test_empty_sequences_and_samples_beyond_length():
    x = _inputs(lens=(0, 5, 17, 0, 64))
    for mode in (0, 1, 2):
        o, idx, _, _ = H.run_hip(x, 100, mode, seed=1)
        print(H.check_all(x, 100, mode, 1, o, idx))


def test_peaked_softmax_single_key():
    """A dominant sink takes (nearly) every sample; duplicates count with multiplicity."""
    x = _inputs(lens=(900, 1200), q_scale=4.0, sinks=1)
    for mode in (0, 1, 2):
        o, idx, _, _ = H.run_hip(x, 256, mode, seed=4)
        print(H.check_all(x, 256, mode, 4, o, idx))


def test_two_stage_calls_equal_decode():
    x = _inputs()
    for mode in (0, 1, 2):
        o1, i1, _, _ = H.run_hip(x, 64, mode, seed=9)
        o2, i2, _, _ = H.run_hip(x, 64, mode, seed=9, stages="split")
        assert torch.equal(i1, i2)
        assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("G,dtype,page", [(7, "bf16", 0), (8, "bf16", 0), (7, "bf16", 16), (8, "f32", 32)])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_two_stage_two_heads_per_wave(G, dtype, page, mode):
    """Groups of 7 and 8 heads on four waves, in the sample pass and in the fused
    kernel: a wave samples two heads and, when each has at most 32 targets in
    its split, gathers both heads' rows in one loop; a dominant sink gives
    splits where a head holds more than that (the one-head-at-a-time gather)
    and splits where a head holds none.  Both paths against the oracle, with
    the same indices."""
    x = _inputs(G=G, dtype=dtype, lens=(900, 1200), page_size=page, q_scale=4.0, sinks=1)
    o2, i2, _, _ = H.run_hip(x, 256, mode, seed=31, split=128, stages="split")
    print(H.check_all(x, 256, mode, 31, o2, i2))
    o1, i1, _, _ = H.run_hip(x, 256, mode, seed=31, split=128)
    print(H.check_all(x, 256, mode, 31, o1, i1))
    assert torch.equal(i1, i2)
    assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
    # the case mix this test is for: per (sequence, head, split) target counts
    lens = x["seq_lens"].tolist()
    counts = torch.cat([torch.bincount(i2[b, h].long() // 128, minlength=-(-lens[b] // 128))
                        for b in range(i2.shape[0]) for h in range(i2.shape[1])])
    assert int((counts > 32).sum()) > 0 and int(((counts > 0) & (counts <= 32)).sum()) > 0
    assert int((counts == 0).sum()) > 0


@pytest.mark.parametrize("G,lens,split", [(8, (40, 50), 64), (4, (3000, 2500), 64), (7, (900, 1200), 128)])
def test_two_stage_multinomial_target_sort(G, lens, split):
    """Multinomial targets on the two-kernel path: sorted by the score pass's
    first B * Hq workgroups when its grid has that many (many splits), by a
    launch of their own otherwise (one split per sequence, B * Hkv < B * Hq
    workgroups).  The indices equal the fused path's and the oracle's."""
    x = _inputs(G=G, lens=lens)
    o2, i2, ws, _ = H.run_hip(x, 200, 0, seed=13, split=split, stages="split")
    print(H.check_all(x, 200, 0, 13, o2, i2))
    assert santa.workspace_error(ws) == 0 and torch.count_nonzero(ws) == 0
    o1, i1, _, _ = H.run_hip(x, 200, 0, seed=13, split=split)
    assert torch.equal(i1, i2)
    assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)


def test_indices_deterministic_and_split_invariant():
    x = _inputs(lens=(3000, 2500))
    for mode in (0, 1, 2):
        _, a, _, _ = H.run_hip(x, 256, mode, seed=21)
        _, b, _, _ = H.run_hip(x, 256, mode, seed=21)
        assert torch.equal(a, b)
        _, c, _, _ = H.run_hip(x, 256, mode, seed=21, split=64)
        # different split sizes change only fp rounding of the CDF
        assert (a != c).float().mean() < 0.01
        _, d_, _, _ = H.run_hip(x, 256, mode, seed=22)
        assert not torch.equal(a, d_)


def test_score_pass_intermediates():
    """Stashed scores and split records (section 3.2, Pass 1) against the oracle."""
    for G, d, dtype, page in [(4, 128, "bf16", 0), (1, 64, "f32", 0), (7, 128, "bf16", 16)]:
        x = _inputs(G=G, d=d, dtype=dtype, lens=(1000, 1537), page_size=page)
        S, mode = 32, 2
        shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len)
        lay = santa.santa_workspace_layout_query(shape, S, mode)
        B, Hq, _ = x["q"].shape
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.empty((B, Hq, S), dtype=torch.int32, device="cuda")
        ws = santa.allocate_workspace(shape, S, mode, "cuda")
        santa.santa_score_pass(shape, x["q"], x["k"], x["v"], x["seq_lens"], x["block_table"], S,
                               mode, 0, o, idx, ws)
        torch.cuda.synchronize()
        wsc = ws.cpu()
        T, split = lay.num_splits, lay.split_size
        row = lay.stash_row_bytes // 4
        stash = wsc[lay.stash_offset: lay.stash_offset + B * Hq * row * 4].view(torch.float32)
        stash = stash.view(B, Hq, row).double().numpy()
        rec = wsc[lay.records_offset: lay.records_offset + B * Hq * T * 8].view(torch.int32)
        rec = rec.view(B, Hq, T, 2)
        m = rec[..., 0].contiguous().view(torch.float32).double().numpy()
        l = rec[..., 1].contiguous().view(torch.float32).double().numpy()
        assert torch.all(torch.isnan(o.cpu()))      # o is written by the sample pass alone
        # the group prefixes the score pass's last split leaves for the sample pass:
        # [B, Hq, T + 2] words after the records, W_t (2^-40 fixed point), Z, M | last << 32
        gp0 = lay.records_offset + B * Hq * T * 8
        gp = wsc[gp0: gp0 + B * Hq * (T + 2) * 8].view(torch.int64).view(B, Hq, T + 2).numpy()
        w = x["workload"]
        for b in range(B):
            n = int(x["seq_lens"][b])
            Tb = -(-n // split)
            assert np.all(l[b, :, :Tb] >= 1.0) and np.all(rec[b, :, Tb:].numpy() == 0)
            for h in range(Hq):
                M = m[b, h, :Tb].max()
                ml = int(gp[b, h, T + 1]) & 0xFFFFFFFFFFFFFFFF
                assert np.float32(M) == np.array([ml & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0]
                masses = l[b, h, :Tb] * np.exp(m[b, h, :Tb] - M)
                W = gp[b, h, :Tb + 1].astype(np.float64) * 2.0 ** -40
                assert W[0] == 0 and np.all(np.diff(W) >= 0)
                # fp32 exp of m_t - M: relative error up to about |m_t - M| * 2^-23
                rt = 2.0 ** -22 * (1.0 + np.abs(m[b, h, :Tb] - M))
                assert np.all(np.abs(np.diff(W) - masses) <= rt * masses + 2.0 ** -40)
                assert (ml >> 32) == int(np.nonzero(np.diff(W) > 0)[0].max())
            for h in range(Hq):
                kk, _ = H.head_rows(x, b, h // w.group)
                q = x["q"][b, h].double().cpu().numpy()
                s_ref = O.scores(q, kk)
                bound = np.abs(kk * q).sum(1) / math.sqrt(d) * 16 * 2.0 ** -24 + 1e-7
                err = np.abs(stash[b, h, :n] - s_ref)
                assert np.all(err <= bound), f"score error {err.max():.2e} (b={b}, h={h})"
                tiles = O.tile_partition(s_ref, split)
                assert np.allclose(m[b, h, :Tb], tiles[:, 0], rtol=0, atol=bound.max())
                assert np.allclose(l[b, h, :Tb], tiles[:, 1], rtol=2e-5, atol=0)
                # the statistics are those of the stashed scores themselves
                for t in range(Tb):
                    st = stash[b, h, t * split: min(n, (t + 1) * split)]
                    assert m[b, h, t] == st.max()
                    e = np.exp(st.astype(np.float32) - np.float32(st.max())).astype(np.float64)
                    assert abs(l[b, h, t] / e.sum() - 1) < 1e-6
        assert santa.workspace_error(ws) == 0


def test_fused_and_two_kernel_paths_agree():
    """santa_decode (one fused kernel here) and score pass + sample pass draw the same indices."""
    for mode in (0, 1, 2):
        for lens, page in [((1000, 1537, 64, 17), 0), ((1000, 1537, 333), 16)]:
            x = _inputs(lens=lens, page_size=page)
            shape = santa.make_shape(x["q"], x["k"], x["block_table"], max_seq_len=x["workload"].seq_len)
            assert santa.santa_decode_path(shape, 200, mode) == santa.PATH_FUSED
            o1, i1, ws1, _ = H.run_hip(x, 200, mode, seed=13)
            o2, i2, ws2, _ = H.run_hip(x, 200, mode, seed=13, stages="split")
            assert torch.equal(i1, i2)
            assert torch.allclose(o1, o2, rtol=1e-5, atol=1e-6)
            assert santa.workspace_error(ws1) == 0 and santa.workspace_error(ws2) == 0


def test_large_grid_repeated_calls_match_split_stages_and_oracle():
    """A step with more work items than the device holds at once (the fused kernel
    with tickets): the same indices as calling the score and sample passes directly,
    parity with the oracle, and a workspace left all zero (ticket counter included)
    after several calls in a row."""
    lens = (8192, 8000, 5000, 1, 0, 8191, 4096, 7777)
    x = _inputs(lens=lens, seed=9)
    S, split = 128, 64
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len, split_size=split)
    B, Hq, d = x["q"].shape
    for mode in (0, 1, 2):
        assert santa.santa_decode_path(shape, S, mode) == santa.PATH_FUSED_TICKETS
        ws = santa.allocate_workspace(shape, S, mode, "cuda")
        for seed in (5, 6, 7):
            o1 = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
            i1 = torch.empty((B, Hq, S), dtype=torch.int32, device="cuda")
            santa.santa_decode(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, seed, o1, i1, ws)
            torch.cuda.synchronize()
            assert santa.workspace_error(ws) == 0
            assert torch.count_nonzero(ws) == 0
            o2, i2, _, _ = H.run_hip(x, S, mode, seed=seed, split=split, stages="split")
            assert torch.equal(i1.cpu(), i2)
            assert torch.allclose(o1.cpu(), o2, rtol=1e-5, atol=1e-6)
        H.check_all(x, S, mode, 7, o1.cpu(), i1.cpu())


def test_workspace_reused_across_calls_and_shapes():
    """Calls leave the workspace zero, so one workspace serves many calls of different shapes in a row,
    mixing the fused kernel and the two halves; every call has its own q, K and V, so a record,
    count or slot left over from an earlier call would show in the indices or the output."""
    xs_a = [_inputs(lens=(2049, 700, 1), seed=30 + r) for r in range(3)]
    xs_b = [_inputs(G=1, d=64, dtype="f32", lens=(300, 0, 1500), seed=40 + r) for r in range(3)]
    big = max(santa.santa_workspace_size(santa.make_shape(x["q"], x["k"], None,
                                                          max_seq_len=x["workload"].seq_len), 128, 0)
              for x in (xs_a[0], xs_b[0]))
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    santa.santa_workspace_init(ws)
    for rep in range(3):
        xa, xb, xa2, xb2 = xs_a[rep], xs_b[rep], xs_a[(rep + 1) % 3], xs_b[(rep + 1) % 3]
        for x, mode in ((xa, 2), (xb, 0), (xa2, 1), (xb2, 2)):
            shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
            B, Hq, d = x["q"].shape
            o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
            idx = torch.empty((B, Hq, 128), dtype=torch.int32, device="cuda")
            args = (shape, x["q"], x["k"], x["v"], x["seq_lens"], None, 128, mode, 40 + rep, o, idx, ws)
            if rep == 1:
                santa.santa_score_pass(*args)
                santa.santa_sample_pass(*args)
            else:
                santa.santa_decode(*args)
            torch.cuda.synchronize()
            H.check_all(x, 128, mode, 40 + rep, o.cpu(), idx.cpu())
    assert santa.workspace_error(ws) == 0
    # between calls the whole workspace is zero
    assert torch.count_nonzero(ws) == 0


def test_sample_pass_without_score_pass_sets_error():
    """A sample pass whose records no score pass wrote flags the error word at once
    (no wait) and leaves the workspace usable after santa_workspace_init."""
    x = _inputs(lens=(1000, 1537, 64))
    S, mode = 64, 1
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
    B, Hq, d = x["q"].shape
    o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, Hq, S), dtype=torch.int32, device="cuda")
    ws = santa.allocate_workspace(shape, S, mode, "cuda")
    args = (shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, 5, o, idx, ws)
    santa.santa_sample_pass(*args)                 # fresh workspace: no records
    torch.cuda.synchronize()
    assert santa.workspace_error(ws) != 0
    assert santa.santa_workspace_status(ws) != 0
    # every group gave up: NaN outputs and idx = -1 (sequences with keys)
    assert torch.isnan(o).all() and bool((idx == -1).all())
    santa.santa_workspace_init(ws)
    assert santa.santa_workspace_status(ws) == 0
    santa.santa_score_pass(*args)
    santa.santa_sample_pass(*args)
    torch.cuda.synchronize()
    assert santa.workspace_error(ws) == 0
    H.check_all(x, S, mode, 5, o.cpu(), idx.cpu())
    santa.santa_sample_pass(*args)                 # records already consumed
    torch.cuda.synchronize()
    assert santa.workspace_error(ws) != 0
    santa.santa_workspace_init(ws)
    santa.santa_decode(*args)
    torch.cuda.synchronize()
    assert santa.workspace_error(ws) == 0
    H.check_all(x, S, mode, 5, o.cpu(), idx.cpu())


def test_graph_replays_match_eager():
    """A captured decode call replays with the same indices (inputs rewritten between replays)."""
    x = _inputs(lens=(1000, 1537, 64, 17))
    S, mode = 128, 2
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
    B, Hq, d = x["q"].shape
    o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, Hq, S), dtype=torch.int32, device="cuda")
    ws = santa.allocate_workspace(shape, S, mode, "cuda")
    q_in = x["q"].clone()
    args = (shape, q_in, x["k"], x["v"], x["seq_lens"], None, S, mode, 77, o, idx, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        santa.santa_decode(*args)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        santa.santa_decode(*args)
    torch.cuda.synchronize()
    for rep in range(4):
        q_in.copy_(x["q"] * (1.0 + 0.25 * rep))
        graph.replay()
        torch.cuda.synchronize()
        o_g, i_g = o.cpu().clone(), idx.cpu().clone()
        santa.santa_decode(*args)
        torch.cuda.synchronize()
        assert torch.equal(i_g, idx.cpu()), rep
        assert torch.allclose(o_g, o.cpu(), rtol=1e-5, atol=1e-6), rep
    assert santa.workspace_error(ws) == 0


def test_toy_unbiased_over_4096_seeds():
    """Mean over seeds of the GPU estimate equals softmax(qK^T/sqrt d) V (toy workload)."""
    w = W.WORKLOADS["toy"]
    x = H.to_device(W.make_inputs(w, seed=0))
    shape = santa.make_shape(x["q"], x["k"])
    q = x["q"][0, 0].double().cpu().numpy()
    k = x["k"][0, :, 0].double().cpu().numpy()
    v = x["v"][0, :, 0].double().cpu().numpy()
    p = O.softmax(O.scores(q, k))
    dense = p @ v
    for mode in w.modes:
        ws = santa.allocate_workspace(shape, 64, mode, "cuda")
        o = torch.empty((1, 1, 64), dtype=torch.float32, device="cuda")
        idx = torch.empty((1, 1, 64), dtype=torch.int32, device="cuda")
        est = torch.empty((4096, 64), dtype=torch.float64, device="cuda")
        for seed in range(4096):
            santa.santa_decode(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, 64, mode, seed, o,
                               idx, ws)
            est[seed] = o[0, 0].double()
        e = est.cpu().numpy()
        se = e.std(0, ddof=1) / math.sqrt(4096)
        assert np.all(np.abs(e.mean(0) - dense) <= 4 * se + 1e-9), mode
        # and the first seeds agree with the oracle element by element
        for seed in range(4):
            santa.santa_decode(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, 64, mode, seed, o,
                               idx, ws)
            torch.cuda.synchronize()
            ref = H.oracle_head(x, 0, 0, 64, mode, seed)
            H.check_head(H.ParityReport(), ref, idx[0, 0].cpu().numpy().astype(np.int64),
                         o[0, 0].double().cpu().numpy(), f"toy seed {seed}")


@pytest.mark.parametrize("path", ["fused", "two_kernel", "flash"])
def test_call_on_a_workspace_in_error_poisons_every_group(path):
    """A workspace whose error word is set (here by the host) holds stale state: a call on it
    writes NaN to o and -1 to idx for every group instead of computing, leaves the word set,
    and santa_workspace_init makes the workspace usable again."""
    x = _inputs(lens=(1000, 1537, 64))
    S, mode = 64, 2
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
    B, Hq, d = x["q"].shape
    o = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    idx = torch.zeros((B, Hq, S), dtype=torch.int32, device="cuda")
    ws = santa.allocate_workspace(shape, S, mode, "cuda")
    ws[0:4].view(torch.int32).fill_(1)
    algo = santa.ALGO_FLASH if path == "flash" else santa.ALGO_PROP
    flags = santa.FLAG_TWO_KERNEL if path == "two_kernel" else 0
    args = (shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, 9, o, idx, ws)
    if path == "two_kernel":
        santa.santa_score_pass(*args)
        santa.santa_sample_pass(*args)
    else:
        santa.santa_decode_args(*args, algorithm=algo, flags=flags)
    assert santa.santa_workspace_status(ws) == 1
    assert torch.isnan(o).all() and bool((idx == -1).all())
    santa.santa_workspace_init(ws)
    santa.santa_decode_args(*args, algorithm=algo, flags=flags)
    assert santa.santa_workspace_status(ws) == 0
    if path == "flash":
        tile = santa.santa_workspace_layout_query(shape, S, mode).split_size
        H.check_flash(x, S, mode, 9, tile, o.cpu(), idx.cpu())
    else:
        H.check_all(x, S, mode, 9, o.cpu(), idx.cpu())


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_args_entry_point_and_forced_two_kernel_path(mode):
    """santa_decode_args gives santa_decode's indices on either path (the fused kernel by
    default on this shape, the score and sample passes with SANTA_FLAG_TWO_KERNEL), and
    santa_decode_flash's with SANTA_ALGO_FLASH."""
    x = _inputs(lens=(2000, 1537, 64, 1))
    S = 96
    shape = santa.make_shape(x["q"], x["k"], None, max_seq_len=x["workload"].seq_len)
    assert santa.santa_decode_path(shape, S, mode) == santa.PATH_FUSED
    B, Hq, d = x["q"].shape
    ws = santa.allocate_workspace(shape, S, mode, "cuda")
    outs = []
    for flags in (0, santa.FLAG_TWO_KERNEL):
        o = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((B, Hq, S), -7, dtype=torch.int32, device="cuda")
        santa.santa_decode_args(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, 21, o, idx, ws,
                                flags=flags)
        torch.cuda.synchronize()
        H.check_all(x, S, mode, 21, o.cpu(), idx.cpu())
        outs.append(idx.cpu())
    assert torch.equal(outs[0], outs[1])
    assert santa.santa_workspace_status(ws) == 0
    if mode != 0:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
        i1 = torch.empty((B, Hq, S), dtype=torch.int32, device="cuda")
        i2 = torch.empty_like(i1)
        santa.santa_decode_args(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, 21, o, i1, ws,
                                algorithm=santa.ALGO_FLASH)
        santa.santa_decode_flash(shape, x["q"], x["k"], x["v"], x["seq_lens"], None, S, mode, 21, o, i2, ws)
        torch.cuda.synchronize()
        assert torch.equal(i1.cpu(), i2.cpu())


@pytest.mark.parametrize("dtype,d,n,split", [("f32", 64, 1024, 0), ("bf16", 128, 4096, 0), ("bf16", 128, 3000, 256)])
def test_systematic_full_budget_uniform_scores_is_exact(dtype, d, n, split):
    """q = 0 makes every score 0, so p_i = 1/n exactly; systematic sampling with S = n
    then puts target m in key m's interval (the SANTA page, section 2.1 Construction):
    idx = 0 .. n-1 in order, and o = mean(V).  The offset is kept away from the
    interval edges, so no target is a boundary case."""
    w = W.Workload("uniform", batch=1, q_heads=4, kv_heads=1, head_dim=d, seq_len=n, dtype=dtype)
    x = W.make_inputs(w, seed=5)
    x["q"] = torch.zeros_like(x["q"])
    x = H.to_device(x)
    seed = next(s for s in range(100) if 0.01 < float(O.uniforms(s, 0, 0, [0])[0]) < 0.99 and
                all(0.01 < float(O.uniforms(s, 0, h, [0])[0]) < 0.99 for h in range(4)))
    print(f"[case] uniform scores {dtype} d={d} n={n} split={split} seed={seed}", flush=True)
    o, idx, ws, shape = H.run_hip(x, n, W.MODE_SYSTEMATIC, seed=seed, split=split)
    assert santa.santa_workspace_status(ws) == 0
    v = x["v"][0, :n, 0].double().cpu()
    for h in range(4):
        assert torch.equal(idx[0, h], torch.arange(n, dtype=torch.int32)), h
        err = float((o[0, h].double() - v.mean(0)).norm() / v.mean(0).norm())
        assert err < 1e-5, (h, err)
    H.check_all(x, n, W.MODE_SYSTEMATIC, seed, o, idx)
