"""Exact sampling law of the oracle on tiny inputs (n_k <= 8), by brute force.

The law of the sampled multiset is enumerated in exact rational arithmetic
straight from the definitions ("Stochastic Sparse Attention for Memory-Bound
Inference": §2 Eq. 3 for i.i.d. draws, §2.1 and its construction paragraph for
the strata I_m = [m/S, (m+1)/S), Appendix A.4 for the inverse CDF with
F(j-1) <= t < F(j)).  The oracle is then checked against it twice:

* its deterministic map from uniforms to indices, fed points inside every
  cell of the enumeration (exact agreement), and
* its full pipeline with its own random numbers over many seeds (chi-square).
"""
import itertools
import math
from collections import Counter
from fractions import Fraction as Fr

import numpy as np
import pytest
import scipy.stats

from oracle import santa as O

DISTRIBUTIONS = {
    "dyadic_with_zero": [Fr(1, 8), Fr(3, 8), Fr(0), Fr(1, 4), Fr(1, 4)],
    "thirds": [Fr(1, 3), Fr(1, 6), Fr(1, 2)],
    "eight_keys": [Fr(1, 16), Fr(3, 16), Fr(1, 10), Fr(0), Fr(1, 5), Fr(1, 20), Fr(3, 20), Fr(1, 4)],
}


def _cum(p):
    c = [Fr(0)]
    for x in p:
        c.append(c[-1] + x)
    return c


def _key_of(C, t):
    """Inverse CDF by linear scan in exact arithmetic: j with C[j] <= t < C[j+1]."""
    for j in range(len(C) - 1):
        if C[j] <= t < C[j + 1]:
            return j
    raise AssertionError("point outside [0, 1)")


def exact_law_systematic(p, S):
    """{count tuple: probability} for one shared offset U ~ U[0,1), t_m = (m + U)/S."""
    C = _cum(p)
    cuts = {Fr(0), Fr(1)}
    for c in C:
        for m in range(S):
            x = S * c - m
            if 0 < x < 1:
                cuts.add(x)
    cuts = sorted(cuts)
    law = Counter()
    cells = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        u = (a + b) / 2
        idx = [_key_of(C, (m + u) / S) for m in range(S)]
        counts = tuple(Counter(idx).get(j, 0) for j in range(len(p)))
        law[counts] += b - a
        cells.append((a, b, idx))
    return law, cells


def exact_law_stratified(p, S):
    """Independent U_m per stratum: P(idx_m = j) = S * |[C_j, C_{j+1}) n I_m|."""
    C = _cum(p)
    n = len(p)
    per_stratum = []
    for m in range(S):
        lo, hi = Fr(m, S), Fr(m + 1, S)
        probs = {}
        for j in range(n):
            ov = min(hi, C[j + 1]) - max(lo, C[j])
            if ov > 0:
                probs[j] = S * ov
        assert sum(probs.values()) == 1
        per_stratum.append(probs)
    law = Counter()
    for combo in itertools.product(*[list(d.items()) for d in per_stratum]):
        pr = Fr(1)
        for _, q in combo:
            pr *= q
        counts = tuple(Counter(j for j, _ in combo).get(j, 0) for j in range(n))
        law[counts] += pr
    return law, per_stratum


def exact_law_multinomial(p, S):
    """i.i.d. draws: counts ~ Multinomial(S, p), from scipy's pmf."""
    n = len(p)
    law = {}
    for counts in itertools.product(range(S + 1), repeat=n):
        if sum(counts) != S:
            continue
        if any(c and p[j] == 0 for j, c in enumerate(counts)):
            continue
        law[counts] = scipy.stats.multinomial.pmf(counts, S, [float(x) for x in p])
    return law


def _scores_for(p):
    """Scores whose softmax is p (zero mass: a score whose exponential underflows)."""
    return np.array([math.log(float(x)) if x > 0 else -2000.0 for x in p])


@pytest.mark.parametrize("name", list(DISTRIBUTIONS))
@pytest.mark.parametrize("S", [1, 2, 3, 4])
def test_exact_laws_are_unbiased(name, S):
    """E[count_j] = S p_j for all three rules (Appendix A.1, A.4)."""
    p = DISTRIBUTIONS[name]
    for law in (exact_law_systematic(p, S)[0], exact_law_stratified(p, S)[0]):
        assert sum(law.values()) == 1
        for j in range(len(p)):
            assert sum(pr * c[j] for c, pr in law.items()) == S * p[j]
    ml = exact_law_multinomial(p, S)
    for j in range(len(p)):
        assert abs(sum(pr * c[j] for c, pr in ml.items()) - S * float(p[j])) < 1e-12


@pytest.mark.parametrize("name", list(DISTRIBUTIONS))
@pytest.mark.parametrize("S", [1, 3, 4, 7])
def test_oracle_map_systematic_matches_enumeration(name, S):
    p = DISTRIBUTIONS[name]
    pf = np.array([float(x) for x in p])
    F = O.cdf(pf)
    _, cells = exact_law_systematic(p, S)
    for a, b, idx in cells:
        if b - a < Fr(1, 10 ** 9):
            continue
        u = float((a + b) / 2)
        t = O.targets_from_uniforms(O.SYSTEMATIC, np.array([u]), S)
        got = O.inverse_cdf(F, pf, t)
        assert list(got) == idx, (u, list(got), idx)


@pytest.mark.parametrize("name", list(DISTRIBUTIONS))
@pytest.mark.parametrize("S", [1, 3, 4])
def test_oracle_map_stratified_matches_enumeration(name, S):
    p = DISTRIBUTIONS[name]
    pf = np.array([float(x) for x in p])
    F = O.cdf(pf)
    C = _cum(p)
    _, per_stratum = exact_law_stratified(p, S)
    for m, probs in enumerate(per_stratum):
        for j in probs:
            # offsets u in this stratum that land on key j
            lo = max(Fr(0), S * C[j] - m)
            hi = min(Fr(1), S * C[j + 1] - m)
            u = np.zeros(S)
            u[m] = float((lo + hi) / 2)
            t = O.targets_from_uniforms(O.STRATIFIED, u, S)
            assert O.inverse_cdf(F, pf, t)[m] == j


@pytest.mark.parametrize("name", list(DISTRIBUTIONS))
def test_oracle_map_multinomial_matches_intervals(name):
    p = DISTRIBUTIONS[name]
    pf = np.array([float(x) for x in p])
    F = O.cdf(pf)
    C = _cum(p)
    pts, want = [], []
    for j in range(len(p)):
        if p[j] > 0:
            pts.append(float((C[j] + C[j + 1]) / 2))
            want.append(j)
    rng = np.random.default_rng(0)
    order = rng.permutation(len(pts))
    u = np.array(pts)[order]
    t = O.targets_from_uniforms(O.MULTINOMIAL, u, len(u))
    assert list(O.inverse_cdf(F, pf, t)) == want    # ascending targets, keys in order


def _chi2_pvalue(law, observed, N):
    keys = sorted(law, key=lambda k: -float(law[k]))
    exp_, obs_ = [], []
    acc_e = acc_o = 0.0
    for k in keys:
        e = float(law[k]) * N
        o = observed.get(k, 0)
        if e >= 5:
            exp_.append(e)
            obs_.append(o)
        else:
            acc_e += e
            acc_o += o
    extra = sum(v for k, v in observed.items() if k not in law)
    assert extra == 0, "oracle produced a multiset of probability zero"
    if acc_e > 0:
        exp_.append(acc_e)
        obs_.append(acc_o)
    if len(exp_) < 2:
        return 1.0
    return scipy.stats.chisquare(obs_, exp_).pvalue


@pytest.mark.parametrize("mode", [O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC])
@pytest.mark.parametrize("name,S", [("dyadic_with_zero", 3), ("thirds", 2), ("eight_keys", 2)])
def test_oracle_pipeline_chi_square(mode, name, S):
    p = DISTRIBUTIONS[name]
    if mode == O.SYSTEMATIC:
        law = exact_law_systematic(p, S)[0]
    elif mode == O.STRATIFIED:
        law = exact_law_stratified(p, S)[0]
    else:
        law = exact_law_multinomial(p, S)
    s = _scores_for(p)
    N = 6000
    obs = Counter()
    for seed in range(N):
        idx, _, _, _ = O.sample_head(s, S, mode, seed, b=0, h=0)
        obs[tuple(np.bincount(idx, minlength=len(p)))] += 1
    assert _chi2_pvalue(law, obs, N) > 1e-4


def test_zero_mass_keys_never_chosen():
    p = DISTRIBUTIONS["eight_keys"]
    s = _scores_for(p)
    for mode in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC):
        for seed in range(300):
            idx, _, _, _ = O.sample_head(s, 16, mode, seed, 0, 0)
            assert 3 not in idx


def test_target_at_or_above_one_takes_last_positive_key():
    pf = np.array([0.5, 0.5, 0.0, 0.0])
    F = O.cdf(pf)
    got = O.inverse_cdf(F, pf, np.array([0.25, 0.75, 1.0, 1.0 + 1e-12]))
    assert list(got) == [0, 1, 1, 1]


def test_half_open_intervals_at_exact_boundaries():
    """Appendix A.4: key j owns [F(j-1), F(j)); a point on an edge belongs to the key above it."""
    pf = np.array([0.25, 0.25, 0.0, 0.5])
    F = O.cdf(pf)                        # [0, .25, .5, .5, 1], all exact in binary
    got = O.inverse_cdf(F, pf, np.array([0.0, 0.25, 0.5, 0.75]))
    assert list(got) == [0, 1, 3, 3]


def test_multinomial_indices_come_in_ascending_target_order():
    rng = np.random.default_rng(12)
    s = rng.standard_normal(500)
    for seed in range(20):
        idx, t, _, _ = O.sample_head(s, 100, O.MULTINOMIAL, seed, 1, 2)
        assert np.all(np.diff(t) >= 0) and np.all(np.diff(idx) >= 0)
