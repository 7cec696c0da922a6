"""Pins of the oracle's estimator against what the pages and the mathematics fix.

"Stochastic Sparse Attention for Memory-Bound Inference":
* Appendix A.1/A.4: every sampling rule is unbiased, E[o_hat] = softmax(q K^T/sqrt(d)) V;
* Appendix A.2: for i.i.d. sampling Cov(o_hat) = Sigma_q / S (trace: the MSE);
* §2.1 / Appendix A.3: stratified sampling does not raise the variance of i.i.d. sampling;
* §2, Eq. 2: rows picked (1, 1, 3) give (2 V_1 + V_3) / 3.
The dense reference comes from torch's scaled_dot_product_attention (a library
implementation of Eq. 1, independent of the oracle).
"""
import json
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import santa as O


def _sdpa(q, k_rows, v_rows):
    """Dense attention of one query from torch (float64, CPU)."""
    qq = torch.as_tensor(q, dtype=torch.float64).view(1, 1, 1, -1)
    kk = torch.as_tensor(k_rows, dtype=torch.float64).view(1, 1, k_rows.shape[0], -1)
    vv = torch.as_tensor(v_rows, dtype=torch.float64).view(1, 1, v_rows.shape[0], -1)
    return F.scaled_dot_product_attention(qq, kk, vv).view(-1).numpy()


@pytest.fixture(scope="module")
def toy():
    w = W.WORKLOADS["toy"]
    x = W.make_inputs(w, seed=0)
    q = x["q"].double().numpy()[0, 0]
    k = x["k"].double().numpy()[0, :, 0]
    v = x["v"].double().numpy()[0, :, 0]
    return q, k, v


@pytest.fixture(scope="module")
def toy_runs(toy):
    """o_hat over 4096 seeds for every rule (toy workload, S = 64)."""
    q, k, v = toy
    s = O.scores(q, k)
    out = {}
    for mode in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC):
        est = np.empty((4096, v.shape[1]))
        for seed in range(4096):
            idx, _, _, _ = O.sample_head(s, 64, mode, seed, 0, 0)
            est[seed] = O.estimate(v, idx)
        out[mode] = est
    return out


def test_dense_reference_matches_torch_sdpa(toy):
    q, k, v = toy
    p = O.softmax(O.scores(q, k))
    assert np.allclose(p @ v, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_scores_softmax_against_logsumexp(toy):
    import scipy.special
    q, k, _ = toy
    s = O.scores(q, k)
    p = O.softmax(s)
    lse = scipy.special.logsumexp((k @ q) * (1.0 / 8.0))   # d = 64: 1/sqrt(d) = 1/8 exactly
    assert np.allclose(np.log(p), s - lse, rtol=0, atol=1e-12)
    F_ = O.cdf(p)
    assert F_[0] == 0.0 and abs(F_[-1] - 1.0) < 1e-13 and np.all(np.diff(F_) >= 0)


@pytest.mark.parametrize("mode", [O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC])
def test_unbiased_over_4096_seeds(toy, toy_runs, mode):
    """mean over seeds of o_hat = softmax(qK^T/sqrt d) V within 4 standard errors."""
    q, k, v = toy
    est = toy_runs[mode]
    dense = _sdpa(q, k, v)
    mean = est.mean(0)
    se = est.std(0, ddof=1) / math.sqrt(est.shape[0])
    assert np.all(np.abs(mean - dense) <= 4 * se + 1e-12)


def test_iid_mse_is_trace_over_S(toy, toy_runs):
    """Appendix A.2: E|o_hat - mu|^2 = tr(Sigma_q) / S for i.i.d. sampling."""
    q, k, v = toy
    p = O.softmax(O.scores(q, k))
    mu = p @ v
    tr_sigma = float(p @ ((v - mu) ** 2).sum(1))
    mse = float(((toy_runs[O.MULTINOMIAL] - mu) ** 2).sum(1).mean())
    assert abs(mse / (tr_sigma / 64) - 1.0) < 0.08


def test_stratified_variance_not_above_iid(toy, toy_runs):
    q, k, v = toy
    mu = O.softmax(O.scores(q, k)) @ v
    mse = {m: float(((toy_runs[m] - mu) ** 2).sum(1).mean()) for m in toy_runs}
    assert mse[O.STRATIFIED] <= mse[O.MULTINOMIAL]
    assert mse[O.SYSTEMATIC] <= mse[O.MULTINOMIAL]


def test_systematic_full_budget_uniform_scores_gives_exact_mean():
    """q = 0: p_j = 1/n; systematic with S = n puts one target in every key."""
    rng = np.random.default_rng(3)
    n, d = 1024, 64
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    s = O.scores(np.zeros(d), k)
    for seed in range(5):
        idx, _, _, _ = O.sample_head(s, n, O.SYSTEMATIC, seed, 0, 0)
        assert np.array_equal(idx, np.arange(n))
        assert np.allclose(O.estimate(v, idx), v.mean(0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("mode", [O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC])
def test_dominant_key_takes_every_sample(mode):
    rng = np.random.default_rng(4)
    v = rng.standard_normal((50, 8))
    s = rng.standard_normal(50)
    s[17] = 900.0
    idx, _, _, _ = O.sample_head(s, 33, mode, 5, 0, 0)
    assert np.all(idx == 17)
    assert np.allclose(O.estimate(v, idx), v[17], rtol=1e-15, atol=0)


def test_single_sample_is_the_same_draw_for_every_rule():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(200) * 2
    for seed in range(50):
        got = [O.sample_head(s, 1, m, seed, 2, 9)[0][0]
               for m in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC)]
        assert got[0] == got[1] == got[2]


def test_eq2_gather_example(golden_dir):
    with open(f"{golden_dir}/eq2_gather_example.json") as f:
        g = json.load(f)
    rng = np.random.default_rng(6)
    v = rng.standard_normal((g["num_rows"], 16))
    idx = np.array(g["indices_one_based"]) - 1
    want = np.array(g["row_weights"]) @ v
    assert np.allclose(O.estimate(v, idx), want, rtol=0, atol=1e-15)
    assert np.allclose(O.estimate(v, idx), (2 * v[0] + v[2]) / 3, rtol=0, atol=1e-15)


def test_tile_partition_against_logsumexp():
    import scipy.special
    rng = np.random.default_rng(7)
    s = rng.standard_normal(1000) * 5
    st = O.tile_partition(s, 256)
    assert st.shape == (4, 2)
    for t in range(4):
        tile = s[t * 256:(t + 1) * 256]
        assert st[t, 0] == tile.max()
        assert abs(st[t, 0] + math.log(st[t, 1]) - scipy.special.logsumexp(tile)) < 1e-12


def _small_inputs(page_size=0, seq_len=300, seq_len_min=50):
    w = W.Workload("small", batch=3, q_heads=8, kv_heads=2, head_dim=16, seq_len=seq_len,
                   seq_len_min=seq_len_min, page_size=page_size, dtype="f32", sinks=2,
                   sink_scale=4.0)
    return w, W.make_inputs(w, seed=9)


def test_decode_against_sdpa_per_head_and_gqa_mapping():
    w, x = _small_inputs()
    res = O.decode(x["q"].numpy(), x["k"].numpy(), x["v"].numpy(), x["seq_lens"].numpy(),
                   None, 0, S=32, mode=O.SYSTEMATIC, seed=1, want_dense=True)
    for b in range(w.batch):
        n = int(x["seq_lens"][b])
        for h in range(w.q_heads):
            g = h // w.group
            ref = _sdpa(x["q"][b, h].double().numpy(), x["k"][b, :n, g].double().numpy(),
                        x["v"][b, :n, g].double().numpy())
            assert np.allclose(res[(b, h)]["dense"], ref, rtol=0, atol=1e-12)
            assert res[(b, h)]["idx"].max() < n


def test_paged_layout_gives_identical_results():
    wc, xc = _small_inputs()
    ps = 16
    # lay the contiguous caches out in shuffled pages
    B, n_max = wc.batch, wc.seq_len
    npg = -(-n_max // ps)
    rng = np.random.default_rng(8)
    perm = rng.permutation(B * npg)
    bt = perm.reshape(B, npg)
    kc, vc = xc["k"].numpy(), xc["v"].numpy()
    kp = np.zeros((B * npg, ps) + kc.shape[2:])
    vp = np.zeros_like(kp)
    for b in range(B):
        for i in range(n_max):
            kp[bt[b, i // ps], i % ps] = kc[b, i]
            vp[bt[b, i // ps], i % ps] = vc[b, i]
    args = dict(S=48, mode=O.STRATIFIED, seed=3)
    rc = O.decode(xc["q"].numpy(), kc, vc, xc["seq_lens"].numpy(), None, 0, **args)
    rp = O.decode(xc["q"].numpy(), kp, vp, xc["seq_lens"].numpy(), bt, ps, **args)
    for key in rc:
        assert np.array_equal(rc[key]["idx"], rp[key]["idx"])
        assert np.array_equal(rc[key]["o"], rp[key]["o"])


def test_empty_sequence_gives_zero_and_minus_one():
    w, x = _small_inputs()
    lens = x["seq_lens"].numpy().copy()
    lens[1] = 0
    res = O.decode(x["q"].numpy(), x["k"].numpy(), x["v"].numpy(), lens, None, 0,
                   S=8, mode=O.MULTINOMIAL, seed=0)
    for h in range(w.q_heads):
        assert np.all(res[(1, h)]["o"] == 0) and np.all(res[(1, h)]["idx"] == -1)
        assert res[(0, h)]["idx"].min() >= 0


def test_boundary_distance_on_hand_built_cdf():
    """Appendix A.4: key j owns the half-open interval [F(j), F(j+1)); the
    distance of a target is to the nearer edge of its key's interval.  Dyadic
    CDF and targets, so every expected distance is exact."""
    p = np.array([0.25, 0.25, 0.0, 0.5])
    F = O.cdf(p)                                 # 0, 1/4, 1/2, 1/2, 1
    eps = 2.0 ** -30
    t = np.array([
        0.5 - eps,          # just below the upper edge of key 1
        0.25 + eps,         # just above the lower edge of key 1
        0.25,               # exactly on the lower edge of key 1 (half-open: key 1)
        0.375,              # middle of key 1
        0.5,                # lower edge of key 3 (key 2 has no mass)
        0.75 + eps,         # inside key 3, nearer its upper edge (by 1/4 - eps)
        1.0 - eps,          # just below F(n)
        1.0 + 2.0 ** -40,   # rounded past F(n): clamps to key 3
    ])
    idx = O.inverse_cdf(F, p, t)
    assert idx.tolist() == [1, 1, 1, 1, 3, 3, 3, 3]
    want = [eps, eps, 0.0, 0.125, 0.0, 0.25 - eps, eps, 2.0 ** -40]
    assert O.boundary_distance(F, idx, t).tolist() == want


def test_boundary_distance_is_nonnegative_and_small_for_flat_law():
    rng = np.random.default_rng(10)
    s = rng.standard_normal(4096)
    idx, t, F_, p = O.sample_head(s, 256, O.SYSTEMATIC, 2, 0, 0)
    delta = O.boundary_distance(F_, idx, t)
    assert np.all(delta >= 0)
    assert np.all(delta <= p[idx])
