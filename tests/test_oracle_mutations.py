"""Planted mistakes in the oracle must each fail at least one pin.

Each case swaps one oracle function for a plausible wrong version (on the CPU,
through monkeypatch) and runs the pins that should catch it.
"""
import numpy as np
import pytest

import workloads as W
from oracle import santa as O
from tests import test_oracle_estimator as E
from tests import test_oracle_law as L
from tests import test_oracle_rng as R

_orig = {name: getattr(O, name) for name in
         ("scores", "cdf", "inverse_cdf", "targets_from_uniforms", "estimate", "uniforms",
          "sequence_keys", "softmax", "boundary_distance")}


def _toy():
    w = W.WORKLOADS["toy"]
    x = W.make_inputs(w, seed=0)
    return x["q"].double().numpy()[0, 0], x["k"].double().numpy()[0, :, 0], x["v"].double().numpy()[0, :, 0]


def _fails(fn, *a):
    try:
        fn(*a)
    except AssertionError:
        return True
    return False


def _law_pins():
    yield lambda: L.test_oracle_map_systematic_matches_enumeration("thirds", 3)
    yield lambda: L.test_oracle_map_stratified_matches_enumeration("dyadic_with_zero", 3)
    yield lambda: L.test_oracle_map_multinomial_matches_intervals("eight_keys")
    yield L.test_half_open_intervals_at_exact_boundaries
    yield L.test_target_at_or_above_one_takes_last_positive_key
    for mode in (O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC):
        yield lambda mode=mode: L.test_oracle_pipeline_chi_square(mode, "dyadic_with_zero", 3)


def _any_fails(pins):
    return any(_fails(p) for p in pins)


MUTATIONS = {
    "scale_dropped": ("scores", lambda q, k: np.asarray(k, np.float64) @ np.asarray(q, np.float64)),
    "scale_by_d": ("scores", lambda q, k: (np.asarray(k, np.float64) @ np.asarray(q, np.float64)) / len(q)),
    "cdf_inclusive": ("cdf", lambda p: np.concatenate((np.cumsum(p), [1.0]))),
    "search_left": ("inverse_cdf", lambda F, p, t: np.minimum(np.searchsorted(F[1:], t, side="left"), len(p) - 1)),
    "no_clamp": ("inverse_cdf", lambda F, p, t: np.searchsorted(F[1:], t, side="right")),
    "strat_shared_offset": ("targets_from_uniforms",
                            lambda mode, u, S: _orig["targets_from_uniforms"](
                                O.SYSTEMATIC if mode == O.STRATIFIED else mode, u, S)),
    "sys_per_stratum": ("targets_from_uniforms",
                        lambda mode, u, S: (np.arange(S) + O.uniforms(7, 0, 0, np.arange(S))) / S
                        if mode == O.SYSTEMATIC else _orig["targets_from_uniforms"](mode, u, S)),
    "strata_off_by_one": ("targets_from_uniforms",
                          lambda mode, u, S: _orig["targets_from_uniforms"](mode, u, S) if mode == O.MULTINOMIAL
                          else (np.arange(S) + (u[:S] if mode == O.STRATIFIED else u[0])) / (S + 1)),
    "iid_unsorted": ("targets_from_uniforms",
                     lambda mode, u, S: np.asarray(u[:S], np.float64) if mode == O.MULTINOMIAL
                     else _orig["targets_from_uniforms"](mode, u, S)),
    "mean_over_unique": ("estimate", lambda v, idx: np.asarray(v, np.float64)[np.unique(idx)].mean(0)),
    "counter_b_h_swapped": ("uniforms", lambda seed, b, h, j: _orig["uniforms"](seed, h, b, j)),
    "u_low_bits": ("uniforms", lambda seed, b, h, j: (O.philox4x64(
        (np.asarray(j, np.uint64), np.uint64(h), np.uint64(b), np.uint64(0)), (seed, 0))[0]
        & np.uint64((1 << 53) - 1)).astype(np.float64) * 2.0 ** -53),
    "softmax_no_normalise": ("softmax", lambda s: np.exp(np.asarray(s) - np.max(s))),
    "boundary_distance_zero": ("boundary_distance", lambda F, idx, t: np.zeros(len(t))),
    "boundary_distance_lower_edge_only": ("boundary_distance", lambda F, idx, t: np.asarray(t) - F[idx]),
    "boundary_distance_upper_edge_only": ("boundary_distance", lambda F, idx, t: F[idx + 1] - np.asarray(t)),
    "boundary_distance_signed": ("boundary_distance",
                                 lambda F, idx, t: np.minimum(np.asarray(t) - F[idx], F[idx + 1] - np.asarray(t))),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    toy = _toy()
    pins = list(_law_pins())
    pins += [
        lambda: E.test_dense_reference_matches_torch_sdpa(toy),
        lambda: E.test_eq2_gather_example("tests/golden"),
        lambda: E.test_systematic_full_budget_uniform_scores_gives_exact_mean(),
        lambda: E.test_decode_against_sdpa_per_head_and_gqa_mapping(),
        R.test_uniforms_follow_counter_layout,
        L.test_multinomial_indices_come_in_ascending_target_order,
        E.test_boundary_distance_on_hand_built_cdf,
    ]
    assert _any_fails(pins), f"no pin caught the planted mistake {name!r}"


def test_gqa_mapping_mistake_is_caught(monkeypatch):
    """Query head h must read KV head h // G, not h % Hkv."""
    real_decode = O.decode

    def bad_decode(q, k, v, lens, bt, ps, S, mode, seed, heads=None, want_dense=False):
        Hq, Hkv = q.shape[1], k.shape[2]
        perm = [h % Hkv * (Hq // Hkv) + h // Hkv for h in range(Hq)]   # interleaved grouping
        return real_decode(q[:, perm], k, v, lens, bt, ps, S, mode, seed, heads, want_dense)

    monkeypatch.setattr(O, "decode", bad_decode)
    assert _fails(E.test_decode_against_sdpa_per_head_and_gqa_mapping)


def test_paging_mistake_is_caught(monkeypatch):
    def bad_keys(cache, n, b, bt, ps):
        if bt is None:
            return np.asarray(cache[b, :n])
        i = np.arange(n)
        return np.asarray(cache)[np.asarray(bt)[b, i % ps], i // ps % ps]
    monkeypatch.setattr(O, "sequence_keys", bad_keys)
    assert _fails(E.test_paged_layout_gives_identical_results)
