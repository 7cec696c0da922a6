"""Pins of the oracle's S^2ANTA-flash against what the pages and the mathematics fix.

"Stochastic Sparse Attention for Memory-Bound Inference", §3.3: every tile gets a
fixed, uniform budget, samples as if it held all the probability mass, and a final
merge weights each tile's partial output by its share of the true partition function.
* the merge weights are the tiles' shares of the softmax: checked against scipy's
  softmax of the whole row, summed per tile;
* uniform scores, systematic sampling, one sample per key: every key is drawn exactly
  once and the estimate is exactly mean(V);
* the estimator is unbiased (each tile's local estimate is unbiased for the tile's
  local attention, Appendix A.1/A.4, and the weights undo the local normalisation):
  the mean over 4096 seeds matches torch's dense attention within 4 standard errors;
* a key that holds nearly all the mass of its tile takes all of that tile's samples;
* the per-tile budgets add up to S and differ by at most one;
* the tile streams are Philox4x64-10 with counter (j, h, b, 1 + t), bit for bit
  against NumPy's independent implementation, and distinct from SANTA's stream.
Planted mistakes at the end each fail at least one of these.
"""
import math

import numpy as np
import pytest
import scipy.special

import workloads as W
from oracle import santa as O
from tests.test_oracle_estimator import _sdpa
from tests.test_oracle_rng import _numpy_block


@pytest.fixture(scope="module")
def toy():
    w = W.WORKLOADS["toy"]
    x = W.make_inputs(w, seed=0)
    q = x["q"].double().numpy()[0, 0]
    k = x["k"].double().numpy()[0, :, 0]
    v = x["v"].double().numpy()[0, :, 0]
    return q, k, v


def test_weights_are_tile_shares_of_the_softmax(toy):
    q, k, _ = toy
    s = O.scores(q, k)
    p = scipy.special.softmax(s)
    for tile in (64, 128, 300, 1024, 4096):
        r = O.sample_head_flash(s, 64, O.SYSTEMATIC, 3, 0, 0, tile)
        T = -(-len(s) // tile)
        shares = np.array([p[t * tile:(t + 1) * tile].sum() for t in range(T)])
        assert np.allclose(r["weight"], shares, rtol=1e-12, atol=1e-15)
        assert abs(r["weight"].sum() - 1.0) < 1e-12


@pytest.mark.parametrize("tile", [64, 128, 256])
def test_uniform_scores_one_sample_per_key_give_mean_of_values_exactly(tile):
    rng = np.random.default_rng(5)
    n, d = 1024, 16
    v = rng.standard_normal((n, d))
    s = np.zeros(n)                      # q = 0: every score equal
    r = O.sample_head_flash(s, n, O.SYSTEMATIC, 11, 0, 0, tile)
    assert np.array_equal(np.sort(r["idx"]), np.arange(n))
    o = O.estimate_flash(v, r["idx"], r["tile_of"], r["budget"], r["weight"])
    assert np.allclose(o, v.mean(axis=0), rtol=0, atol=1e-12)


@pytest.fixture(scope="module")
def flash_runs(toy):
    """o_hat over 4096 seeds for every rule (toy workload, S = 64 over 8 tiles of 128)."""
    q, k, v = toy
    s = O.scores(q, k)
    out = {}
    for mode in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC):
        est = np.empty((4096, v.shape[1]))
        for seed in range(4096):
            r = O.sample_head_flash(s, 64, mode, seed, 0, 0, 128)
            est[seed] = O.estimate_flash(v, r["idx"], r["tile_of"], r["budget"], r["weight"])
        out[mode] = est
    return out


@pytest.mark.parametrize("mode", [O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC])
def test_unbiased_over_4096_seeds(toy, flash_runs, mode):
    q, k, v = toy
    dense = _sdpa(q, k, v)
    est = flash_runs[mode]
    se = est.std(axis=0, ddof=1) / math.sqrt(len(est))
    assert np.all(np.abs(est.mean(axis=0) - dense) <= 4 * se + 1e-12)


def test_dominant_key_takes_its_tiles_samples():
    rng = np.random.default_rng(2)
    n, tile = 1000, 128
    s = rng.standard_normal(n)
    s[300] = 60.0                         # tile 2 = keys 256..383
    v = rng.standard_normal((n, 4))
    for mode in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC):
        r = O.sample_head_flash(s, 80, mode, 7, 0, 0, tile)
        assert np.all(r["idx"][r["tile_of"] == 2] == 300)
        assert r["weight"][2] >= 1 - 1e-15 and np.delete(r["weight"], 2).max() < 1e-20
        o = O.estimate_flash(v, r["idx"], r["tile_of"], r["budget"], r["weight"])
        assert np.allclose(o, v[300], atol=1e-12)


def test_budgets_add_up_and_are_uniform_up_to_one():
    assert list(O.tile_budgets(10, 4)) == [3, 3, 2, 2]
    assert list(O.tile_budgets(8, 8)) == [1] * 8
    for S, T in [(256, 64), (257, 64), (2048, 64), (100, 7), (5, 5)]:
        b = O.tile_budgets(S, T)
        assert b.sum() == S and b.max() - b.min() <= (0 if S % T == 0 else 1)
    with pytest.raises(ValueError):
        O.tile_budgets(3, 4)
    # the samples of a head come tile by tile, each tile's in its own block
    s = np.random.default_rng(0).standard_normal(700)
    r = O.sample_head_flash(s, 50, O.STRATIFIED, 1, 0, 0, 100)
    assert list(r["budget"]) == [8, 7, 7, 7, 7, 7, 7] and len(r["idx"]) == 50
    assert np.array_equal(r["tile_of"], np.repeat(np.arange(7), r["budget"]))
    assert np.all(r["idx"] // 100 == r["tile_of"])


def test_tile_streams_match_numpy_and_are_distinct():
    seed = 0x5EED
    for b, h, t in [(0, 0, 0), (3, 17, 5), (63, 31, 127)]:
        j = np.arange(5)
        got = O.tile_uniforms(seed, b, h, t, j)
        want = np.array([(_numpy_block([int(x), h, b, 1 + t], [seed, 0])[0] >> 11) * 2.0 ** -53 for x in j])
        assert np.array_equal(got, want)
    a = O.tile_uniforms(seed, 1, 2, 0, np.arange(64))
    assert not np.any(a == O.uniforms(seed, 1, 2, np.arange(64)))
    assert not np.any(a == O.tile_uniforms(seed, 1, 2, 1, np.arange(64)))


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin above.
# ---------------------------------------------------------------------------
_orig_sample = O.sample_head_flash
_orig_estimate = O.estimate_flash
_orig_tile_uniforms = O.tile_uniforms
_orig_budgets = O.tile_budgets


def _equal_weights(*a, **k):
    r = _orig_sample(*a, **k)
    r["weight"] = np.full(len(r["budget"]), 1.0 / len(r["budget"]))
    return r


def _global_cdf(s, S, mode, seed, b, h, tile):
    r = _orig_sample(s, S, mode, seed, b, h, tile)
    p = O.softmax(s)                       # samples each tile's block from the whole row's CDF
    F = O.cdf(p)
    out = []
    for t in range(len(r["budget"])):
        u = _orig_tile_uniforms(seed, b, h, t, np.arange(O.draws_needed(mode, int(r["budget"][t]))))
        out.append(O.inverse_cdf(F, p, O.targets_from_uniforms(mode, u, int(r["budget"][t]))))
    r["idx"] = np.concatenate(out)
    return r


def _no_budget_division(values, idx, tile_of, budget, weight):
    return _orig_estimate(values, idx, tile_of, np.ones_like(budget), weight)


def _floor_budgets(S, T):
    if S < T:
        raise ValueError("S < T")
    return np.full(T, S // T, dtype=np.int64)


MUTATIONS = {
    "equal_tile_weights": ("sample_head_flash", _equal_weights),
    "global_cdf_in_tiles": ("sample_head_flash", _global_cdf),
    "partial_not_divided_by_budget": ("estimate_flash", _no_budget_division),
    "budget_remainder_dropped": ("tile_budgets", _floor_budgets),
    "tile_stream_is_santa_stream": ("tile_uniforms", lambda seed, b, h, t, j: O.uniforms(seed, b, h, j)),
}


def _pins(toy):
    yield lambda: test_weights_are_tile_shares_of_the_softmax(toy)
    for tile in (64, 128):
        yield lambda tile=tile: test_uniform_scores_one_sample_per_key_give_mean_of_values_exactly(tile)
    yield test_dominant_key_takes_its_tiles_samples
    yield test_budgets_add_up_and_are_uniform_up_to_one
    yield test_tile_streams_match_numpy_and_are_distinct


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(toy, monkeypatch, name):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    failed = False
    for pin in _pins(toy):
        try:
            pin()
        except (AssertionError, ValueError):
            failed = True
            break
    assert failed, f"planted mistake {name} passed every pin"
