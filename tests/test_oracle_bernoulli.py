"""Pins of the Bernoulli qK^T oracle (oracle/bernoulli.py) against what the
pages and the mathematics fix:

* the estimated scores are unbiased: their mean over 4096 seeds equals q . k
  within 4 standard errors (the property Eq. 5 and Eq. 6 are built on);
* stratified draws: a feature's count is always floor(B pi) or ceil(B pi), and
  ceil occurs with frequency frac(B pi);
* for one head (G = 1) the estimator is Eq. 5 itself: (norm / B) sum_n q_hat^(n)
  K^T with ternary samples q_hat^(n)_i = sign(q_i) [draw n keeps i], built
  here sample by sample from the same uniforms;
* special cases: features of equal mean magnitude are always kept (the scores
  are then exact), the largest feature is always kept B times, a query with
  one nonzero feature gives exact scores;
* the uniforms are bit-exact against NumPy's independent Philox4x64-10 with
  key (seed, 1);
* the SANTA stage on top samples from softmax(s_hat / sqrt(d)) exactly as the
  pinned SANTA oracle does;
* planted mistakes in the oracle each fail at least one of these pins.
"""
import math

import numpy as np
import pytest

from oracle import bernoulli as BQ
from oracle import santa as O
from tests.test_oracle_rng import _numpy_block


def _group(G=4, d=16, n=40, seed=0, scales=None):
    rng = np.random.default_rng(seed)
    c = np.exp(rng.standard_normal(d)) if scales is None else np.asarray(scales, dtype=np.float64)
    q = rng.standard_normal((G, d)) * c
    k = rng.standard_normal((n, d))
    return q, k


def test_uniforms_match_numpy_philox_with_key_one():
    for seed, b, g, i in [(0, 0, 0, 0), (7, 3, 5, 127), (2 ** 63 + 5, 63, 7, 64)]:
        u = BQ.feature_uniforms(seed, b, g, i, 6)
        want = [(_numpy_block([n, i, g, b], [seed, 1])[0] >> 11) * 2.0 ** -53 for n in range(6)]
        assert u.tolist() == want


@pytest.mark.parametrize("G", [1, 4])
def test_estimated_scores_are_unbiased_over_4096_seeds(G):
    q, k = _group(G=G, d=12, n=30, seed=G)
    est = np.stack([BQ.estimated_scores(q, k, 4, seed, 0, 0)[0] for seed in range(4096)])
    exact = q @ k.T
    se = est.std(0, ddof=1) / math.sqrt(len(est))
    assert np.all(np.abs(est.mean(0) - exact) <= 4 * se + 1e-12)
    assert np.any(se > 0)                      # the estimator is random here


def test_counts_are_stratified():
    q, _ = _group(G=4, d=32, seed=11)
    m = BQ.mean_group_query(q)
    for B in (1, 3, 8):
        pi = m / m.max()
        lo, frac = np.floor(B * pi), B * pi - np.floor(B * pi)
        counts = np.stack([BQ.feature_counts(m, B, seed, 1, 2) for seed in range(2000)])
        assert np.all((counts == lo) | (counts == lo + 1))
        hit = (counts == lo + 1).mean(0)
        se = np.sqrt(np.maximum(frac * (1 - frac), 1e-12) / len(counts))
        assert np.all(np.abs(hit - frac) <= 4 * se + 1e-12)


def test_single_head_is_eq5_ternary_samples():
    q, k = _group(G=1, d=10, n=25, seed=5)
    B, seed, b, g = 5, 42, 2, 1
    s_hat, counts = BQ.estimated_scores(q, k, B, seed, b, g)
    norm = np.abs(q[0]).max()
    acc = np.zeros(len(k))
    total = np.zeros(q.shape[1])
    for n_draw in range(B):
        q_hat = np.zeros(q.shape[1])
        for i in range(q.shape[1]):
            u = BQ.feature_uniforms(seed, b, g, i, B)[n_draw]
            if (n_draw + u) / B < abs(q[0, i]) / norm:
                q_hat[i] = np.sign(q[0, i])
        total += np.abs(q_hat)
        acc += q_hat @ k.T
    assert np.allclose(s_hat[0], norm / B * acc, rtol=1e-12, atol=1e-12)
    assert np.array_equal(counts, total.astype(np.int64))


def test_special_cases_are_exact():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 8))
    # equal mean magnitude in every feature: pi = 1 everywhere, every draw keeps every feature
    q = np.where(rng.random((4, 8)) < 0.5, -1.0, 1.0)
    s_hat, counts = BQ.estimated_scores(q, k, 3, 9, 0, 0)
    assert np.all(counts == 3) and np.allclose(s_hat, q @ k.T, rtol=0, atol=1e-12)
    # one nonzero feature
    q1 = np.zeros((1, 8))
    q1[0, 5] = -2.5
    s_hat, counts = BQ.estimated_scores(q1, k, 4, 1, 0, 0)
    assert counts.tolist() == [0, 0, 0, 0, 0, 4, 0, 0] and np.allclose(s_hat, q1 @ k.T, rtol=0, atol=1e-12)
    # the representative is the mean of the heads' absolute values (section 5.1): with
    # q_0 = (4, 1), q_1 = (0, 1) it is (2, 1), so with B = 2 the second feature is kept by
    # exactly one draw for every seed (B pi = 1); the per-feature maximum (4, 1) would give
    # B pi = 1/2
    q2 = np.array([[4.0, 1.0], [0.0, 1.0]])
    for seed in range(64):
        assert BQ.feature_counts(BQ.mean_group_query(q2), 2, seed, 0, 0).tolist() == [2, 1]
    # the largest mean feature is kept by every draw
    q, _ = _group(seed=8)
    m = BQ.mean_group_query(q)
    for seed in range(50):
        assert BQ.feature_counts(m, 6, seed, 0, 0)[np.argmax(m)] == 6


def test_santa_stage_samples_from_the_estimated_scores():
    q, k = _group(G=4, d=16, n=200, seed=2)
    v = np.random.default_rng(4).standard_normal((200, 16))
    heads, counts = BQ.decode_group(q, k, v, 64, O.SYSTEMATIC, 8, 5, 1, 3, 4)
    s_hat, c2 = BQ.estimated_scores(q, k, 8, 5, 1, 3)
    assert np.array_equal(counts, c2)
    for h in range(4):
        idx, t, F, p = O.sample_head(s_hat[h] / 4.0, 64, O.SYSTEMATIC, 5, 1, 3 * 4 + h)
        assert np.array_equal(heads[h]["idx"], idx)
        assert np.allclose(heads[h]["o"], v[idx].mean(0), rtol=0, atol=1e-12)


_orig_counts = BQ.feature_counts
_orig_mgq = BQ.mean_group_query
_orig_unif = BQ.feature_uniforms
_orig_scores = BQ.estimated_scores


def _independent_draws(m, B, seed, b, g):
    m = np.asarray(m, dtype=np.float64)
    u = BQ.feature_uniforms(seed, b, g, np.arange(len(m)), B)
    return (u < (m / m.max())[:, None]).sum(axis=1).astype(np.int64)


def _m_hat_without_norm(q_group, keys, B, seed, b, g):
    q_group = np.asarray(q_group, dtype=np.float64)
    m = BQ.mean_group_query(q_group)
    counts = BQ.feature_counts(m, B, seed, b, g)
    ratio = np.divide(counts / B, m, out=np.zeros_like(m), where=m > 0)
    return (q_group * ratio) @ np.asarray(keys).T, counts


def _m_hat_used_as_query(q_group, keys, B, seed, b, g):
    q_group = np.asarray(q_group, dtype=np.float64)
    m = BQ.mean_group_query(q_group)
    counts = BQ.feature_counts(m, B, seed, b, g)
    m_hat = (m.max() / B) * counts
    return np.tile(m_hat, (q_group.shape[0], 1)) @ np.asarray(keys).T, counts


def _swapped(seed, b, g, i, B):
    f = np.asarray(i, dtype=np.uint64)
    n = np.arange(B, dtype=np.uint64)
    w0 = O.philox4x64((f.reshape(-1, 1), n[None, :], np.uint64(g), np.uint64(b)), (seed, 1))[0]
    u = (w0 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return u[0] if f.ndim == 0 else u


MUTATIONS = {
    "independent_draws": ("feature_counts", _independent_draws),
    "max_instead_of_mean": ("mean_group_query", lambda qg: np.abs(np.asarray(qg, np.float64)).max(0)),
    "signed_mean": ("mean_group_query", lambda qg: np.abs(np.asarray(qg, np.float64).mean(0))),
    "m_hat_without_norm": ("estimated_scores", _m_hat_without_norm),
    "m_hat_used_as_query": ("estimated_scores", _m_hat_used_as_query),
    "santa_key": ("feature_uniforms", lambda seed, b, g, i, B: _orig_unif(seed ^ 1, b, g, i, B)),
    "draw_feature_swapped": ("feature_uniforms", lambda seed, b, g, i, B: _swapped(seed, b, g, i, B)),
}


def _pins():
    yield test_uniforms_match_numpy_philox_with_key_one
    yield lambda: test_estimated_scores_are_unbiased_over_4096_seeds(4)
    yield test_counts_are_stratified
    yield test_single_head_is_eq5_ternary_samples
    yield test_special_cases_are_exact


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(monkeypatch, name):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(BQ, attr, bad)
    failed = False
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed = True
            break
    assert failed, f"planted mistake {name} passed every pin"
