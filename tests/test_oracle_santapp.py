"""Pins of the SANTA++ oracle (oracle/santapp.py) against what the pages and the
mathematics fix, independent of the oracle's own code:

* contiguous parents: the closed form of Algorithm 4;
* team construction: a hand-worked parent (first representative nearest the
  mean, farthest-first choices, nearest-representative assignment), the
  definition's post-conditions on random parents, and the tie rules with
  duplicate keys (lowest token index; earliest representative; self-ownership);
* the budget of Eq. 5 on the page's examples (S = 128 -> 32 teams, S = 124 ->
  31 with P = 16, R = 4);
* K = M is dense attention exactly (Algorithm 1, lines 4-5; Eq. 4 with c = 1);
* the Gumbel draws: bit-exact uniforms against NumPy's independent
  Philox4x64-10 with key (seed, 2), and the Gumbel(0, 1) law (KS test);
* the Gumbel-max law: the top perturbed score is team g with probability
  Z~_g / sum Z~ (the first-draw probability of section A);
* the inclusion correction: E[1{g in S} / c_g] = 1 for every team (Eq. 8),
  and the threshold is the (K+1)-th perturbed score on a worked example;
* the estimator's sums are unbiased, E[U_hat] = U and E[Z_hat] = Z (Eq. 9),
  with an exact suffix;
* planted mistakes each fail at least one of these pins.
"""
import math

import numpy as np
import pytest

from oracle import santapp as PP
from tests.test_oracle_rng import _numpy_block


def test_contiguous_parents_closed_form():
    parents = PP.contiguous_parents(37, 16)
    assert [p.tolist() for p in parents] == [list(range(16)), list(range(16, 32)), list(range(32, 37))]
    assert [len(p) for p in PP.contiguous_parents(32, 16)] == [16, 16]
    assert [len(p) for p in PP.contiguous_parents(5, 16)] == [5]


def test_team_build_worked_example():
    # one parent of six 2-D keys: the mean is (23/6, 20/6); k1 is nearest to it,
    # k4 farthest from k1, then k3 farthest from {k1, k4}; every other key joins
    # its nearest representative
    keys = np.array([[0, 0], [1, 0], [10, 0], [11, 0], [0, 10], [1, 10]], dtype=np.float64)
    teams = PP.build_teams(keys, [np.arange(6)], 3)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([0, 1], 1), ([4, 5], 4), ([2, 3], 3)]
    # R = 1: one team holding the parent, represented by the key nearest the mean
    teams = PP.build_teams(keys, [np.arange(6)], 1)
    assert [(t[0].tolist(), t[1]) for t in teams] == [(list(range(6)), 1)]


def _brute_check(keys, parent, teams_of_parent, R):
    """The definition of section 2.2 / Algorithm 2 checked on an output."""
    kc = keys[parent]
    r = min(R, len(parent))
    assert len(teams_of_parent) == r
    reps = [t[1] for t in teams_of_parent]
    mu = kc.mean(axis=0)
    d_mu = ((kc - mu) ** 2).sum(1)
    assert np.isclose(d_mu[list(parent).index(reps[0])], d_mu.min(), rtol=1e-12, atol=0)
    for u in range(1, r):
        chosen = [list(parent).index(x) for x in reps[:u]]
        md = np.array([min(((kc[i] - kc[j]) ** 2).sum() for j in chosen) for i in range(len(parent))])
        md[chosen] = -1.0
        assert np.isclose(md[list(parent).index(reps[u])], md.max(), rtol=1e-12, atol=0)
    members = np.concatenate([t[0] for t in teams_of_parent])
    assert sorted(members.tolist()) == sorted(parent.tolist())        # a partition of the parent
    for u, (mem, rep) in enumerate(teams_of_parent):
        assert rep in mem.tolist()                                    # each representative owns its row
        for i in mem:
            if i in reps:
                continue
            dist = [((keys[i] - keys[x]) ** 2).sum() for x in reps]
            assert dist[u] <= min(dist) * (1 + 1e-12)                # nearest representative


def test_team_build_satisfies_the_definition_on_random_parents():
    rng = np.random.default_rng(5)
    keys = rng.standard_normal((200, 8)) * np.exp(rng.standard_normal(8))
    parents = PP.contiguous_parents(200, 16)
    teams = PP.build_teams(keys, parents, 4)
    assert len(teams) == sum(min(4, len(p)) for p in parents)
    at = 0
    for p in parents:
        r = min(4, len(p))
        _brute_check(keys, p, teams[at:at + r], 4)
        at += r


def test_team_build_ties_and_self_ownership():
    # identical keys: every distance is 0, so the representatives are the first r
    # tokens of the parent, each owns itself and the rest join the first one
    keys = np.ones((6, 3))
    teams = PP.build_teams(keys, [np.arange(6)], 3)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([0, 3, 4, 5], 0), ([1], 1), ([2], 2)]
    # a key equidistant from two representatives joins the one chosen first
    keys = np.array([[0.0, 0.0], [-1.0, 0.0], [1.0, 0.0]])
    teams = PP.build_teams(keys, [np.arange(3)], 2)
    # the mean is (0, 0): k0 first; k1 and k2 tie as farthest -> k1 (lower index);
    # k2 is a representative only if r = 3, here it joins the nearer: k0 (distance 1)
    # versus k1 (distance 4)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([0, 2], 0), ([1], 1)]
    keys = np.array([[0.0, 0.0], [2.0, 0.0], [1.0, 0.0], [5.0, 5.0]])
    teams = PP.build_teams(keys, [np.arange(4)], 2)
    # mean (2, 1.25): k1 nearest (1.5625); k3 farthest from k1 (34); k2 is at
    # distance 1 from k1 and 41 from k3; k0 at 4 from k1 and 50 from k3
    assert [(t[0].tolist(), t[1]) for t in teams] == [([0, 1, 2], 1), ([3], 3)]
    keys = np.array([[0.0], [2.0], [1.0], [10.0]])
    teams = PP.build_teams(keys, [np.arange(3)], 2)
    # mean 1: k2 first; k0 and k1 tie as farthest (distance 1) -> k0; then k1 is at
    # distance 1 from k2 and 4 from k0 -> k2's team
    assert [(t[0].tolist(), t[1]) for t in teams] == [([1, 2], 2), ([0], 0)]
    keys = np.array([[0.0], [2.0], [4.0]])
    teams = PP.build_teams(keys, [np.arange(3)], 3)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([1], 1), ([0], 0), ([2], 2)]
    keys = np.array([[1.0], [0.0], [2.0], [1.0]])
    # mean 1: k0 and k3 tie at distance 0 -> k0; farthest from k0: k1 and k2
    # (distance 1) -> k1; k2 is at 1 from k0 and 4 from k1 -> k0; k3 at 0 from k0
    teams = PP.build_teams(keys, [np.arange(4)], 2)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([0, 2, 3], 0), ([1], 1)]
    keys = np.array([[0.0], [4.0], [2.0]])
    # mean 2: k2 first; k0 and k1 tie at distance 4 -> k0; k1 is at 4 from k2
    # and 16 from k0 -> k2
    teams = PP.build_teams(keys, [np.arange(3)], 2)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([1, 2], 2), ([0], 0)]
    keys = np.array([[0.0], [4.0], [2.0], [3.0], [1.0]])
    # mean 2: k2; farthest k0 (4, lower index than k1); third: k1 (min(4, 16) = 4);
    # k3: distances 1 (k2), 9 (k0), 1 (k1) -> tie, the earlier representative k2;
    # k4: 1 (k2), 1 (k0), 9 (k1) -> k2
    teams = PP.build_teams(keys, [np.arange(5)], 3)
    assert [(t[0].tolist(), t[1]) for t in teams] == [([2, 3, 4], 2), ([0], 0), ([1], 1)]


def test_team_budget_examples():
    assert PP.team_budget(10 ** 6, 128, 16, 4) == 32
    assert PP.team_budget(10 ** 6, 124, 16, 4) == 31
    assert PP.team_budget(20, 128, 16, 4) == 20
    with pytest.raises(ValueError):
        PP.team_budget(100, 130, 16, 4)
    with pytest.raises(ValueError):
        PP.team_budget(100, 128, 16, 3)


def _problem(n=60, N=48, d=8, seed=0, scale=1.0, P=8, R=2):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((n, d)) * scale
    values = rng.standard_normal((n, d))
    q = rng.standard_normal(d) * scale
    teams = PP.build_teams(keys[:N], PP.contiguous_parents(N, P), R)
    return q, keys, values, teams


def test_all_teams_is_dense_attention():
    q, keys, values, teams = _problem(scale=2.0)
    M = len(teams)
    for K in (M, M + 5):
        r = PP.decode_head(q, keys, values, teams, 48, 60, K, 3, 0, 0)
        s = keys @ q / math.sqrt(len(q))
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(r["o"], p @ values, rtol=0, atol=1e-12)
        assert np.all(r["c"] == 1.0) and r["tau"] is None


def test_gumbel_uniforms_match_numpy_philox_and_law():
    for seed, b, h, g in [(0, 0, 0, 0), (9, 2, 27, 8191), (2 ** 64 - 1, 63, 5, 123456)]:
        want = _numpy_block([g, h, b, 0], [seed, 2])[0]
        u = ((want >> 11) + 0.5) * 2.0 ** -53
        assert PP.gumbel(seed, b, h, g) == -math.log(-math.log(u))
    G = PP.gumbel(7, 1, 3, np.arange(200000))
    from scipy import stats
    assert stats.kstest(G, lambda x: np.exp(-np.exp(-x))).pvalue > 1e-3


def _selections(phi, K, seeds):
    out = []
    for seed in seeds:
        G = PP.gumbel(seed, 0, 0, np.arange(len(phi)))
        out.append(PP.select_teams(phi, G, K))
    return out


def test_gumbel_max_draws_teams_in_proportion_to_their_mass():
    q = np.array([1.0, -0.5])
    rep = np.array([[0.3, 0.1], [-0.2, 0.8], [1.0, 1.0], [0.0, 0.0]])
    sizes = np.array([1, 4, 2, 7])
    phi = PP.routing_logits(q, rep, sizes)
    mass = sizes * np.exp(rep @ q / math.sqrt(2))          # Eq. 3: Z~_g = n_g exp(q . l_g / sqrt(d))
    p = mass / mass.sum()
    T = 16000
    first = np.zeros(4)
    for seed in range(T):
        Y = phi + PP.gumbel(seed, 0, 0, np.arange(4))
        first[np.argmax(Y)] += 1
    se = np.sqrt(p * (1 - p) / T)
    assert np.all(np.abs(first / T - p) <= 4 * se)


def test_threshold_is_the_next_perturbed_score():
    phi = np.zeros(5)
    G = np.array([0.5, 2.0, -1.0, 1.5, 0.7])
    sel, c, tau, thr = PP.select_teams(phi, G, 2)
    assert sel.tolist() == [1, 3] and tau == 0.7 and thr == 4
    assert np.allclose(c, 1 - np.exp(-np.exp(-0.7)), rtol=1e-15)
    # equal perturbed scores: the lower team index ranks first
    sel, c, tau, thr = PP.select_teams(np.zeros(4), np.array([1.0, 2.0, 1.0, 1.0]), 2)
    assert sel.tolist() == [0, 1] and thr == 2


def test_inclusion_correction_reweights_to_one():
    """Eq. 8: for every team, E[1{g in S} / c_g] = 1."""
    phi = np.log(np.array([1.0, 3.0, 2.0, 6.0, 1.0, 4.0])) + np.array([0.2, -1.0, 0.5, 0.0, 1.5, -0.3])
    T = 8000
    acc = np.zeros((T, 6))
    for t, (sel, c, tau, thr) in enumerate(_selections(phi, 2, range(T))):
        acc[t, sel] = 1.0 / c
    mean, se = acc.mean(0), acc.std(0, ddof=1) / math.sqrt(T)
    assert np.all(np.abs(mean - 1.0) <= 4 * se + 1e-12)


def test_unnormalised_sums_are_unbiased_with_a_suffix():
    """Eq. 9: E[U_hat] = U and E[Z_hat] = Z over the Gumbel draws."""
    q, keys, values, teams = _problem(n=40, N=32, d=4, seed=2, P=8, R=4)
    M = len(teams)
    rep = keys[[t[1] for t in teams]]
    sizes = np.array([len(t[0]) for t in teams])
    phi = PP.routing_logits(q, rep, sizes)
    s = keys @ q / 2.0
    Z = np.exp(s).sum()
    U = np.exp(s) @ values
    T = 3000
    est_Z = np.zeros(T)
    est_U = np.zeros((T, keys.shape[1]))
    for t, (sel, c, tau, thr) in enumerate(_selections(phi, 3, range(T))):
        est_U[t], est_Z[t] = PP.estimate_sums(q, keys, values, teams, np.arange(32, 40), sel, c)
    assert M > 3
    assert abs(est_Z.mean() - Z) <= 4 * est_Z.std(ddof=1) / math.sqrt(T)
    assert np.all(np.abs(est_U.mean(0) - U) <= 4 * est_U.std(0, ddof=1) / math.sqrt(T))


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------
_orig_select = PP.select_teams
_orig_logits = PP.routing_logits
_orig_build = PP.build_teams
_orig_gumbel = PP.gumbel
_orig_sums = PP.estimate_sums


def _tau_kth(phi, G, K):
    sel, c, tau, thr = _orig_select(phi, G, K)
    if thr is None:
        return sel, c, tau, thr
    Y = phi + G
    kth = np.min(Y[sel])
    return sel, -np.expm1(-np.exp(phi[sel] - kth)), kth, thr


def _first_draw(phi, G, K):
    sel, c, tau, thr = _orig_select(phi, G, K)
    if thr is None:
        return sel, c, tau, thr
    p = np.exp(phi) / np.exp(phi).sum()
    return sel, p[sel], tau, thr


def _build_variant(keys, parents, R, farthest="min", first="nearest", own=True, ties="first"):
    keys = np.asarray(keys, dtype=np.float64)
    teams = []
    for C in parents:
        C = np.asarray(C)
        r = min(R, len(C))
        kc = keys[C]
        mu = kc.sum(axis=0) / len(C)
        dm = ((kc - mu) ** 2).sum(1)
        chosen = [int(np.argmin(dm) if first == "nearest" else np.argmax(dm))]
        for _ in range(1, r):
            dd = np.stack([((kc - kc[j]) ** 2).sum(1) for j in chosen])
            near = dd.min(0) if farthest == "min" else dd.max(0)
            near[chosen] = -np.inf
            chosen.append(int(np.argmax(near)))
        dist = np.stack([((kc - kc[j]) ** 2).sum(1) for j in chosen])
        owner = np.argmin(dist, 0) if ties == "first" else (len(chosen) - 1 - np.argmin(dist[::-1], 0))
        if own:
            for u, j in enumerate(chosen):
                owner[j] = u
        for u, j in enumerate(chosen):
            teams.append((C[owner == u], int(C[j])))
    return teams


def _z_uncorrected(q, keys, values, teams, suffix, sel, c):
    U, _ = _orig_sums(q, keys, values, teams, suffix, sel, c)
    _, Z1 = _orig_sums(q, keys, values, teams, suffix, sel, np.ones(len(sel)))
    return U, Z1


MUTATIONS = {
    "no_log_size": ("routing_logits", lambda q, rep, n: np.asarray(rep, np.float64) @ np.asarray(q, np.float64)
                    / math.sqrt(len(q))),
    "tau_is_kth": ("select_teams", _tau_kth),
    "first_draw_probability": ("select_teams", _first_draw),
    "gumbel_sign": ("gumbel", lambda seed, b, h, g: -_orig_gumbel(seed, b, h, g)),
    "farthest_by_max": ("build_teams", lambda k, p, R: _build_variant(k, p, R, farthest="max")),
    "first_farthest_from_mean": ("build_teams", lambda k, p, R: _build_variant(k, p, R, first="farthest")),
    "no_self_ownership": ("build_teams", lambda k, p, R: _build_variant(k, p, R, own=False)),
    "assignment_ties_last": ("build_teams", lambda k, p, R: _build_variant(k, p, R, ties="last")),
    "z_not_corrected": ("estimate_sums", _z_uncorrected),
}


def _pins():
    yield test_team_build_worked_example
    yield test_team_build_satisfies_the_definition_on_random_parents
    yield test_team_build_ties_and_self_ownership
    yield test_all_teams_is_dense_attention
    yield test_threshold_is_the_next_perturbed_score
    yield test_gumbel_uniforms_match_numpy_philox_and_law
    yield test_gumbel_max_draws_teams_in_proportion_to_their_mass
    yield test_inclusion_correction_reweights_to_one
    yield test_unnormalised_sums_are_unbiased_with_a_suffix


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(monkeypatch, name):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(PP, attr, bad)
    failed = False
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            failed = True
            break
    assert failed, f"planted mistake {name} passed every pin"
