"""Pins of the top-k comparator oracle (oracle/topk.py) against what the
mathematics fixes, with no implementation to compare against:

* brute force on tiny inputs: among all k-subsets exactly one keeps only keys
  that precede every dropped key in (score descending, index ascending) order,
  and it is the oracle's selection;
* the estimate equals torch's scaled_dot_product_attention with the dropped
  keys masked out (a library routine, float64 on the CPU);
* special cases: k = n is dense attention, k = 1 returns the row of the best
  key, equal scores keep the first k keys, n < S pads idx with -1;
* planted mistakes in the oracle each fail at least one of these pins.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import topk as T


def _sdpa(q, k_rows, v_rows, keep=None):
    qq = torch.as_tensor(q, dtype=torch.float64).view(1, 1, 1, -1)
    kk = torch.as_tensor(k_rows, dtype=torch.float64).view(1, 1, len(k_rows), -1)
    vv = torch.as_tensor(v_rows, dtype=torch.float64).view(1, 1, len(v_rows), -1)
    mask = None
    if keep is not None:
        m = torch.zeros(len(k_rows), dtype=torch.bool)
        m[torch.as_tensor(keep)] = True
        mask = m.view(1, 1, 1, -1)
    return F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask).view(-1).numpy()


def _rng_case(n, d=8, seed=0, ties=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(d)
    k = rng.standard_normal((n, d))
    if ties:                      # duplicate rows make exactly equal scores
        k[n // 2:] = k[:n - n // 2]
    v = rng.standard_normal((n, d))
    return q, k, v


def test_selection_matches_brute_force_dominance():
    for n in range(1, 9):
        for seed in range(6):
            q, k, v = _rng_case(n, seed=seed, ties=seed % 2 == 1)
            s = T.scores(q, k)
            for kk in range(1, n + 1):
                rank = lambda i: (-s[i], i)          # smaller is better
                winners = [set(c) for c in itertools.combinations(range(n), kk)
                           if all(rank(a) < rank(b) for a in c for b in set(range(n)) - set(c))]
                assert len(winners) == 1
                assert set(T.select(s, kk).tolist()) == winners[0]
                assert list(T.select(s, kk)) == sorted(winners[0])


def test_estimate_is_masked_dense_attention():
    for seed in range(5):
        q, k, v = _rng_case(200, d=16, seed=seed)
        s = T.scores(q, k)
        for kk in (1, 7, 64, 199):
            kept = T.select(s, kk)
            assert np.allclose(T.estimate(s, v, kept), _sdpa(q, k, v, keep=kept), rtol=0, atol=1e-12)


def test_full_budget_is_dense_attention_and_one_is_argmax():
    q, k, v = _rng_case(300, d=16, seed=3)
    r = T.decode_head(q, k, v, 300)
    assert np.allclose(r["o"], _sdpa(q, k, v), rtol=0, atol=1e-12)
    assert r["idx"].tolist() == list(range(300))
    r1 = T.decode_head(q, k, v, 1)
    assert np.array_equal(r1["o"], v[np.argmax(T.scores(q, k))])


def test_equal_scores_keep_the_first_keys_and_short_sequences_pad():
    k = np.ones((10, 4))
    v = np.arange(40, dtype=np.float64).reshape(10, 4)
    r = T.decode_head(np.ones(4), k, v, 4)
    assert r["idx"].tolist() == [0, 1, 2, 3]
    assert np.allclose(r["o"], v[:4].mean(0))
    r = T.decode_head(np.ones(4), k[:3], v[:3], 5)
    assert r["idx"].tolist() == [0, 1, 2, -1, -1]
    r = T.decode_head(np.ones(4), k[:0], v[:0], 5)
    assert r["idx"].tolist() == [-1] * 5 and np.all(r["o"] == 0)


def test_threshold_is_the_kth_largest_score():
    q, k, v = _rng_case(50, seed=9)
    s = T.scores(q, k)
    for kk in (1, 10, 50):
        kept = T.select(s, kk)
        thr = T.threshold(s, kk)
        assert s[kept].min() == thr
        assert np.all(np.delete(s, kept) <= thr)


_orig_select = T.select
_orig_estimate = T.estimate

MUTATIONS = {
    "ties_keep_higher_index": ("select", lambda s, k: np.sort(np.lexsort((-np.arange(len(s)), -np.asarray(s)))[:min(k, len(s))])),
    "one_too_many": ("select", lambda s, k: _orig_select(s, k + 1)),
    "smallest_scores": ("select", lambda s, k: _orig_select(-np.asarray(s), k)),
    "unsorted_output": ("select", lambda s, k: np.lexsort((np.arange(len(s)), -np.asarray(s)))[:min(k, len(s))]),
    "normalised_over_all_keys": ("estimate", lambda s, v, kept: (np.exp(np.asarray(s)[kept] - np.max(s))[:, None]
                                                                 * np.asarray(v)[kept]).sum(0)
                                 / np.exp(np.asarray(s) - np.max(s)).sum()),
    "unweighted_mean": ("estimate", lambda s, v, kept: np.asarray(v)[kept].mean(0)),
}


def _pins():
    yield test_selection_matches_brute_force_dominance
    yield test_estimate_is_masked_dense_attention
    yield test_full_budget_is_dense_attention_and_one_is_argmax
    yield test_equal_scores_keep_the_first_keys_and_short_sequences_pad


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(monkeypatch, name):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(T, attr, bad)
    failed = False
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed = True
            break
    assert failed, f"planted mistake {name} passed every pin"
