"""Pins of the oracle's random numbers.

The oracle restates Philox4x64-10 from its published definition; here it is
checked bit for bit against NumPy's independent implementation (with random
and edge-case counters and keys), and its uniforms against the uniform law.
"""
import numpy as np
import pytest
import scipy.stats

from oracle import santa as O

_M64 = (1 << 64) - 1


def _numpy_block(counter, key):
    """NumPy's Philox returns, as its first block, the block of counter + 1."""
    c = sum(int(v) << (64 * i) for i, v in enumerate(counter))
    cm = (c - 1) % (1 << 256)
    ctr = np.array([(cm >> (64 * i)) & _M64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=ctr, key=np.array(key, dtype=np.uint64))
    return [int(x) for x in bg.random_raw(4)]


def test_philox_matches_numpy():
    rng = np.random.default_rng(1234)
    for trial in range(400):
        ctr = [int(x) for x in rng.integers(0, 2 ** 64, 4, dtype=np.uint64)]
        if trial % 4 == 0:
            ctr[0] = 0                       # counter - 1 borrows across words
        if trial % 4 == 1:
            ctr = [trial, 3, 5, 0]           # small counters like the decode layout
        key = [int(x) for x in rng.integers(0, 2 ** 64, 2, dtype=np.uint64)]
        got = [int(x) for x in O.philox4x64([np.uint64(v) for v in ctr], key)]
        assert got == _numpy_block(ctr, key), (ctr, key)


def test_philox_vectorised_matches_scalar_calls():
    j = np.arange(300, dtype=np.uint64)
    words = O.philox4x64((j, np.uint64(7), np.uint64(2), np.uint64(0)), (99, 0))
    for jj in (0, 1, 17, 299):
        ref = _numpy_block([jj, 7, 2, 0], [99, 0])
        assert [int(w[jj]) for w in words] == ref


def test_uniforms_grid_and_range():
    u = O.uniforms(5, 0, 3, np.arange(20000))
    assert np.all(u >= 0.0) and np.all(u < 1.0)
    k = u * 2.0 ** 53
    assert np.all(k == np.floor(k))          # on the 2**-53 grid


def test_uniforms_follow_counter_layout():
    # draw j of head h of sequence b is word 0 of the block at counter (j, h, b, 0), key (seed, 0)
    for seed, b, h, j in [(0, 0, 0, 0), (1, 3, 31, 255), (2 ** 63 + 5, 15, 7, 1023)]:
        w0 = _numpy_block([j, h, b, 0], [seed, 0])[0]
        assert O.uniforms(seed, b, h, [j])[0] == (w0 >> 11) * 2.0 ** -53


def test_uniforms_ks_and_independence():
    u = O.uniforms(11, 1, 2, np.arange(200000))
    assert scipy.stats.kstest(u, "uniform").pvalue > 1e-3
    v = O.uniforms(11, 1, 3, np.arange(200000))    # next head: another stream
    assert abs(np.corrcoef(u, v)[0, 1]) < 0.01
    assert scipy.stats.kstest(v, "uniform").pvalue > 1e-3


@pytest.mark.parametrize("mode", [O.MULTINOMIAL, O.STRATIFIED, O.SYSTEMATIC])
def test_targets_lie_in_unit_interval_and_strata(mode):
    S = 64
    u = O.uniforms(3, 0, 0, np.arange(O.draws_needed(mode, S)))
    t = O.targets_from_uniforms(mode, u, S)
    assert np.all(t >= 0) and np.all(t < 1) and np.all(np.diff(t) >= 0)
    if mode != O.MULTINOMIAL:
        # one point per stratum I_m = [m/S, (m+1)/S)
        assert np.array_equal(np.floor(t * S), np.arange(S))
    if mode == O.SYSTEMATIC:
        assert np.allclose(np.diff(t), 1.0 / S, rtol=0, atol=1e-15)
