"""CPU oracle for SANTA decode-step attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path
(``sampling_sparse_attention_amd``) never does: it shares no code, header,
table or constant with this file.

What it computes is SANTA as defined in "Stochastic Sparse Attention for
Memory-Bound Inference" (Lee et al.):

* §2, Eq. 1: attention ``softmax(q K^T / sqrt(d_k)) V = A V`` for one query.
* §2, Eq. 3: SANTA treats the softmax row as a categorical distribution, draws
  ``S`` indices and returns ``(1/S) * sum_s V[i_s]`` (Eq. 2: duplicates count
  with multiplicity; nothing is materialised as one-hot vectors).
* §2.1 and its "Construction" paragraph: stratified (one uniform per stratum
  ``I_m = [m/S, (m+1)/S)``) and systematic (one shared uniform offset) sampling.
* Appendix A.4: the index for a point ``t`` of the unit interval is the inverse
  CDF, key ``j`` such that ``F(j-1) <= t < F(j)``.

Everything is float64 NumPy, plain loops over (sequence, query head), with no
blocking or fusion.  Readings of points the pages leave open (all listed with
their reasons in the design notes of this repository):

1. stratified targets ``t_m = (m + U_m) / S`` with independent ``U_m``;
   systematic targets ``t_m = (m + U) / S`` with one ``U`` (the construction
   paragraph keeps only the strata ``I_m``; these are the plainest targets that
   put one point in each stratum);
2. multinomial (i.i.d.) sampling uses the inverse CDF of ``S`` i.i.d. uniforms,
   returned in ascending order of the uniforms (the estimator does not depend
   on the order, Eq. 3);
3. ``U`` is ``(w0 >> 11) * 2**-53`` where ``w0`` is word 0 of a Philox4x64-10
   block (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as
   1, 2, 3", SC 2011) with key ``(seed, 0)`` and counter ``(j, h, b, 0)`` for
   draw ``j`` of query head ``h`` of sequence ``b``; the pages fix no generator;
4. a target that rounds to ``t >= F(n)`` selects the last key of positive mass;
5. every query head of a GQA group samples independently (its own ``h`` in the
   counter);
6. a sequence of length 0 gives ``o = 0`` and ``idx = -1``.

It also computes S^2ANTA-flash (§3.3 of the same page: a fixed, uniform budget
per tile, local sampling as if the tile held all the mass, and a final merge
that down-weights each tile's partial output by its share of the true
partition function).  The pseudocode appendix it points to is not in the
pages; the readings taken are

7. a tile is ``tile`` consecutive keys of the sequence (the score pass's
   split), so a sequence of ``n`` keys has ``T = ceil(n / tile)`` tiles;
8. the tiles share exactly ``S`` samples, tile ``t`` taking ``floor(S / T)``
   plus one for ``t < S mod T`` (uniform up to one, and ``idx`` keeps ``S``
   entries, tile by tile); ``S >= T``, so every tile is sampled and the
   estimator stays unbiased;
9. tile ``t`` applies the chosen rule with its own ``S_t`` to its own softmax
   (the same targets and inverse CDF as above), drawing its uniforms from the
   Philox counter ``(j, h, b, 1 + t)``;
10. ``o = sum_t (Z_t / Z) * (1/S_t) * sum_j V[idx_tj]``, where ``Z_t`` is the
    tile's partition function and ``Z`` their sum.
"""
from __future__ import annotations

import math

import numpy as np

MULTINOMIAL = 0
STRATIFIED = 1
SYSTEMATIC = 2

# ---------------------------------------------------------------------------
# Philox4x64-10, restated from Salmon et al. (SC 2011): the S-box is a pair of
# 64x64->128 multiplications, the key schedule a Weyl sequence.
# ---------------------------------------------------------------------------
_MASK32 = np.uint64(0xFFFFFFFF)
_SH32 = np.uint64(32)
PHILOX_M0 = 0xD2E7470EE14C6C93      # multiplier applied to counter word 0
PHILOX_M1 = 0xCA5A826395121157      # multiplier applied to counter word 2
PHILOX_W0 = 0x9E3779B97F4A7C15      # key increment, word 0 (golden ratio)
PHILOX_W1 = 0xBB67AE8584CAA73B      # key increment, word 1 (sqrt(3) - 1)


def _mulhilo64(a: np.ndarray, b: int):
    """(high, low) 64-bit halves of the 128-bit product a * b, element-wise."""
    b = np.uint64(b)
    a0, a1 = a & _MASK32, a >> _SH32
    b0, b1 = b & _MASK32, b >> _SH32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _SH32) + (p01 & _MASK32) + (p10 & _MASK32)
    hi = p11 + (p01 >> _SH32) + (p10 >> _SH32) + (mid >> _SH32)
    lo = a * b                      # uint64 multiplication wraps modulo 2**64
    return hi, lo


def philox4x64(counter, key, rounds: int = 10):
    """Philox4x64-R block function.

    ``counter`` is a sequence of 4 uint64 arrays (broadcastable), ``key`` a
    sequence of 2.  Returns the 4 output words as uint64 arrays.
    """
    with np.errstate(over="ignore"):
        x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) for c in counter)
        x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
        k0, k1 = (np.uint64(int(k) & 0xFFFFFFFFFFFFFFFF) for k in key)
        for r in range(rounds):
            if r:
                k0 = np.uint64((int(k0) + PHILOX_W0) & 0xFFFFFFFFFFFFFFFF)
                k1 = np.uint64((int(k1) + PHILOX_W1) & 0xFFFFFFFFFFFFFFFF)
            hi0, lo0 = _mulhilo64(x0, PHILOX_M0)
            hi1, lo1 = _mulhilo64(x2, PHILOX_M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def uniforms(seed: int, b: int, h: int, j) -> np.ndarray:
    """U[0, 1) draws ``j`` (array) of query head ``h`` of sequence ``b`` (reading 3)."""
    j = np.asarray(j, dtype=np.uint64)
    w0, _, _, _ = philox4x64((j, np.uint64(h), np.uint64(b), np.uint64(0)), (seed, 0))
    return (w0 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


# ---------------------------------------------------------------------------
# The method, one query head at a time.
# ---------------------------------------------------------------------------
def scores(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """``q K^T / sqrt(d_k)`` for one query ``q [d]`` and keys ``[n, d]`` (§2, Eq. 1)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    return (keys @ q) / math.sqrt(q.shape[0])


def softmax(s: np.ndarray) -> np.ndarray:
    """The softmax row ``A_q`` of §2, Eq. 1 (shifted by the maximum, summed with fsum)."""
    s = np.asarray(s, dtype=np.float64)
    w = np.exp(s - s.max())
    return w / math.fsum(w)


def cdf(p: np.ndarray) -> np.ndarray:
    """``F`` with ``F[0] = 0`` and ``F[j+1] = F[j] + p[j]`` (Appendix A.4's F(j))."""
    return np.concatenate(([0.0], np.cumsum(np.asarray(p, dtype=np.float64))))


def targets_from_uniforms(mode: int, u: np.ndarray, S: int) -> np.ndarray:
    """Points of [0, 1) whose inverse CDF gives the samples (§2, §2.1, readings 1-2).

    multinomial: the S i.i.d. uniforms, in ascending order;
    stratified:  ``(m + u_m) / S`` -- one independent point per stratum I_m;
    systematic:  ``(m + u_0) / S`` -- one offset shared by all strata.
    """
    u = np.asarray(u, dtype=np.float64)
    m = np.arange(S, dtype=np.float64)
    if mode == MULTINOMIAL:
        return np.sort(u[:S])
    if mode == STRATIFIED:
        return (m + u[:S]) / S
    if mode == SYSTEMATIC:
        return (m + u[0]) / S
    raise ValueError(f"unknown mode {mode}")


def draws_needed(mode: int, S: int) -> int:
    return 1 if mode == SYSTEMATIC else S


def inverse_cdf(F: np.ndarray, p: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Key ``j`` with ``F[j] <= t < F[j+1]`` for every point ``t`` (Appendix A.4).

    Keys of zero mass have an empty interval and are never chosen.  A point at
    or above ``F[n]`` (only reachable through rounding) takes the last key of
    positive mass (reading 4).
    """
    n = len(p)
    idx = np.searchsorted(F[1:], t, side="right")
    last = int(np.nonzero(np.asarray(p) > 0)[0][-1])
    return np.where(idx >= n, last, idx).astype(np.int64)


def estimate(values: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """``(1/S) * sum_s V[i_s]`` with duplicates counted (§2, Eq. 2 and Eq. 3)."""
    values = np.asarray(values, dtype=np.float64)
    return values[np.asarray(idx)].sum(axis=0) / len(idx)


def boundary_distance(F: np.ndarray, idx: np.ndarray, t: np.ndarray) -> np.ndarray:
    """Distance of each target ``t`` from the nearer edge of the interval
    ``[F[idx], F[idx+1])`` of the key it selected (Appendix A.4's half-open
    intervals): ``min(|t - F[idx]|, |F[idx+1] - t|)``.  A target that rounded to
    ``t >= F[n]`` (reading 4) lies past the upper edge of the last key of
    positive mass, so its distance is ``t - F[idx+1] >= 0``, not negative."""
    F = np.asarray(F, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    return np.minimum(np.abs(t - F[idx]), np.abs(F[idx + 1] - t))


def sample_head(s: np.ndarray, S: int, mode: int, seed: int, b: int, h: int):
    """SANTA's sampling step for one query head from its scores ``s``.

    Returns ``(idx, t, F, p)``: the sampled keys in ascending target order,
    the targets, the CDF and the softmax row.
    """
    p = softmax(s)
    F = cdf(p)
    u = uniforms(seed, b, h, np.arange(draws_needed(mode, S)))
    t = targets_from_uniforms(mode, u, S)
    return inverse_cdf(F, p, t), t, F, p


def tile_partition(s: np.ndarray, tile: int):
    """Per-tile statistics of a tiled score pass (§3.2, Pass 1: local partition
    functions ``Z_tile``): for every tile of ``tile`` consecutive keys its maximum
    score ``m`` and ``l = sum exp(s - m)``."""
    s = np.asarray(s, dtype=np.float64)
    out = []
    for t0 in range(0, len(s), tile):
        st = s[t0:t0 + tile]
        m = st.max()
        out.append((m, math.fsum(np.exp(st - m))))
    return np.array(out, dtype=np.float64).reshape(-1, 2)


def sequence_keys(cache: np.ndarray, n: int, b: int, block_table, page_size: int) -> np.ndarray:
    """Logical rows ``[n, Hkv, d]`` of sequence ``b`` of a contiguous
    ``[B, n_max, Hkv, d]`` or paged ``[pages, page_size, Hkv, d]`` cache."""
    if block_table is None:
        return np.asarray(cache[b, :n])
    i = np.arange(n)
    pages = np.asarray(block_table)[b, i // page_size]
    return np.asarray(cache)[pages, i % page_size]


# ---------------------------------------------------------------------------
# S^2ANTA-flash (§3.3; readings 7-10 above), one query head at a time.
# ---------------------------------------------------------------------------
def tile_uniforms(seed: int, b: int, h: int, t: int, j) -> np.ndarray:
    """U[0, 1) draws ``j`` (array) of tile ``t`` of query head ``h`` of sequence ``b``
    (reading 9: counter ``(j, h, b, 1 + t)``, a stream of its own per tile)."""
    j = np.asarray(j, dtype=np.uint64)
    w0, _, _, _ = philox4x64((j, np.uint64(h), np.uint64(b), np.uint64(1 + t)), (seed, 0))
    return (w0 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def tile_budgets(S: int, T: int) -> np.ndarray:
    """Samples of each of ``T`` tiles: ``S`` in all, uniform up to one (reading 8)."""
    if S < T:
        raise ValueError(f"S = {S} < {T} tiles: a tile without samples would bias the estimate")
    return np.array([S // T + (1 if t < S % T else 0) for t in range(T)], dtype=np.int64)


def sample_head_flash(s: np.ndarray, S: int, mode: int, seed: int, b: int, h: int, tile: int):
    """S^2ANTA-flash's sampling for one query head from its scores ``s``.

    Returns a dict: ``idx`` (``[S]``, tile by tile, each tile's keys in ascending
    target order), ``tile_of`` (the tile of each sample), ``budget`` (``S_t``),
    ``weight`` (``Z_t / Z``), ``t`` (each sample's target in its tile's unit
    interval), ``F`` (the list of the tiles' local CDFs) and ``delta`` (boundary
    distances in the local CDFs).
    """
    s = np.asarray(s, dtype=np.float64)
    n = len(s)
    T = -(-n // tile)
    budget = tile_budgets(S, T)
    M = s.max()
    Zt = np.array([math.fsum(np.exp(s[t * tile:(t + 1) * tile] - M)) for t in range(T)])
    idx, tile_of, targets, delta, Fs = [], [], [], [], []
    for t in range(T):
        st = s[t * tile:(t + 1) * tile]
        p = softmax(st)                       # the tile as if it held all the mass
        F = cdf(p)
        u = tile_uniforms(seed, b, h, t, np.arange(draws_needed(mode, int(budget[t]))))
        tt = targets_from_uniforms(mode, u, int(budget[t]))
        local = inverse_cdf(F, p, tt)
        idx.append(t * tile + local)
        tile_of.append(np.full(len(local), t, dtype=np.int64))
        targets.append(tt)
        delta.append(boundary_distance(F, local, tt))
        Fs.append(F)
    return dict(idx=np.concatenate(idx), tile_of=np.concatenate(tile_of), budget=budget,
                weight=Zt / math.fsum(Zt), t=np.concatenate(targets), delta=np.concatenate(delta), F=Fs)


def estimate_flash(values: np.ndarray, idx: np.ndarray, tile_of: np.ndarray, budget: np.ndarray,
                   weight: np.ndarray) -> np.ndarray:
    """The deferred-normalisation merge (reading 10): each tile's mean of its sampled
    rows, weighted by the tile's share ``Z_t / Z`` of the partition function."""
    values = np.asarray(values, dtype=np.float64)
    o = np.zeros(values.shape[1])
    for t in range(len(budget)):
        rows = values[np.asarray(idx)[tile_of == t]]
        o += weight[t] * rows.sum(axis=0) / budget[t]
    return o


def decode(q, k_cache, v_cache, seq_lens, block_table, page_size, S, mode, seed,
           heads=None, want_dense=False):
    """SANTA decode for a batch of single-token queries.

    ``q [B, Hq, d]``, caches as in :func:`sequence_keys`, float arrays (bf16
    data widened exactly by the caller).  ``heads`` optionally restricts the
    work to a list of ``(b, h)`` pairs.  Returns a dict of per-(b, h) results:
    ``o`` (fp64 estimate), ``idx`` (int64 ``[S]``), ``t`` (targets), ``delta``
    (boundary distances), ``n``, and ``dense`` (``A V``) when asked.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = {}
    rows_cache = {}
    for b, h in heads:
        n = int(seq_lens[b])
        g = h // G
        if n == 0:
            out[(b, h)] = dict(o=np.zeros(d), idx=np.full(S, -1, dtype=np.int64),
                               t=None, delta=None, n=0, dense=np.zeros(d))
            continue
        if (b, g) not in rows_cache:
            rows_cache.clear()
            keys = sequence_keys(k_cache, n, b, block_table, page_size)[:, g, :]
            vals = sequence_keys(v_cache, n, b, block_table, page_size)[:, g, :]
            rows_cache[(b, g)] = (np.asarray(keys, np.float64), np.asarray(vals, np.float64))
        keys, vals = rows_cache[(b, g)]
        s = scores(q[b, h], keys)
        idx, t, F, p = sample_head(s, S, mode, seed, b, h)
        res = dict(o=estimate(vals, idx), idx=idx, t=t, delta=boundary_distance(F, idx, t),
                   n=n, s=s, F=F)
        if want_dense:
            res["dense"] = p @ vals
        out[(b, h)] = res
    return out
