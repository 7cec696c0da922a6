"""CPU oracle of SANTA++ (representative-key routing) -- TEST INFRASTRUCTURE ONLY
(only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it; the product path never does).

What it computes is the method of "SANTA++: Sampling Attention through
Representative Keys":

* Appendix A, Algorithm 4: contiguous parent groups of ``P`` prompt tokens;
* Appendix A, Algorithm 2 (section 2.2): in each parent, up to ``R`` actual
  keys as representatives -- the first nearest the parent's mean key, each
  later one the member farthest from its nearest representative so far --
  and every member joins the team of its nearest representative, each
  representative owning its own row;
* Appendix A, Eq. 5: ``K = min(M, S / (P / R))`` teams for a nominal budget S;
* section 2.3, Eq. 3 and Algorithm 1: routing logits ``phi_g = log n_g +
  q . l_g / sqrt(d)``, Gumbel-top-K selection, the threshold ``tau`` (the
  (K+1)-th largest perturbed score), the conditional inclusion correction
  ``c_g = 1 - exp(-exp(phi_g - tau))`` (Eq. 7), and the estimator of Eq. 4,
  ``o = U_hat / Z_hat`` with ``U_hat = U_E + sum_S U_g / c_g`` and ``Z_hat =
  Z_E + sum_S Z_g / c_g`` over the exact suffix E and the selected teams.

Everything is fp64 NumPy, one parent or one query head at a time.  Readings
of points the pages leave open:

1. parents are contiguous (Algorithm 4); the k-means parents of Algorithm 3
   depend on a particular minibatch k-means implementation and are not built;
2. distances are squared Euclidean in fp64 on the keys widened exactly from
   their storage type, the parent mean is the fp64 sum in token order divided
   by the parent size; ties: representative selection takes the lowest token
   index, assignment the earliest-chosen representative (both as the page
   states);
3. teams are numbered parent by parent, and within a parent in the order
   their representatives were chosen; members are kept in token order;
4. the Gumbel draw of team g for query head h of sequence b is
   ``G = -log(-log U)`` with ``U = ((w0 >> 11) + 1/2) * 2**-53`` (strictly
   inside (0, 1)), ``w0`` word 0 of Philox4x64-10 with key ``(seed, 2)`` and
   counter ``(g, h, b, 0)`` (the SANTA sampler uses key ``(seed, 0)``, the
   Bernoulli query sampler ``(seed, 1)``);
5. perturbed scores are ranked by value, equal values by lower team index
   first; the selection is the first K of that order and ``tau`` the value of
   the (K+1)-th;
6. the suffix is the rows of the current cache after the N prompt rows, with
   weight 1; ``o`` is computed from the sums shifted by their largest score
   (the ratio does not change);
7. every query head of a GQA group selects independently with its own
   threshold; the group shares the teams (section 2.3, last paragraph).
"""
from __future__ import annotations

import math

import numpy as np

from . import santa as O


# ---------------------------------------------------------------------------
# Preparation after prefill (Algorithms 4 and 2)
# ---------------------------------------------------------------------------
def contiguous_parents(N: int, P: int):
    """Algorithm 4: parents ``[uP, min((u+1)P, N))`` for ``u < ceil(N / P)``."""
    return [np.arange(u * P, min((u + 1) * P, N)) for u in range(-(-N // P))]


def _sqdist(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances of the rows of ``a`` to the vector ``b``."""
    diff = a - b
    return (diff * diff).sum(axis=1)


def build_teams(keys: np.ndarray, parents, R: int):
    """Algorithm 2: team records ``(members, representative)`` -- members ascending
    token indices, representative a token index -- parent by parent (readings 2-3)."""
    keys = np.asarray(keys, dtype=np.float64)
    teams = []
    for C in parents:
        C = np.asarray(C)
        r = min(R, len(C))
        kc = keys[C]
        mu = kc.sum(axis=0) / len(C)
        chosen = [int(np.argmin(_sqdist(kc, mu)))]          # positions within C
        for _ in range(1, r):
            nearest = np.min(np.stack([_sqdist(kc, kc[j]) for j in chosen]), axis=0)
            nearest[chosen] = -np.inf                         # only members not chosen yet
            chosen.append(int(np.argmax(nearest)))
        dist = np.stack([_sqdist(kc, kc[j]) for j in chosen])  # [r, |C|]
        owner = np.argmin(dist, axis=0)
        for u, j in enumerate(chosen):
            owner[j] = u                                      # representative self-ownership
        for u, j in enumerate(chosen):
            teams.append((C[owner == u], int(C[j])))
    return teams


def team_budget(M: int, S: int, P: int, R: int) -> int:
    """Eq. 5: ``K = min(M, S / (P / R))`` (P divisible by R, S by P / R)."""
    if P % R or S % (P // R):
        raise ValueError("P must be divisible by R and S by P / R")
    return min(M, S // (P // R))


# ---------------------------------------------------------------------------
# Decoding (Algorithm 1)
# ---------------------------------------------------------------------------
def gumbel(seed: int, b: int, h: int, g) -> np.ndarray:
    """Gumbel(0, 1) draws of teams ``g`` (array) for query head h of sequence b (reading 4)."""
    g = np.asarray(g, dtype=np.uint64)
    w0, _, _, _ = O.philox4x64((g, np.uint64(h), np.uint64(b), np.uint64(0)), (seed, 2))
    u = ((w0 >> np.uint64(11)).astype(np.float64) + 0.5) * 2.0 ** -53
    return -np.log(-np.log(u))


def routing_logits(q: np.ndarray, rep_keys: np.ndarray, sizes: np.ndarray) -> np.ndarray:
    """Eq. 3: ``phi_g = log n_g + q . l_g / sqrt(d)``."""
    q = np.asarray(q, dtype=np.float64)
    return np.log(np.asarray(sizes, dtype=np.float64)) + np.asarray(rep_keys, np.float64) @ q / math.sqrt(len(q))


def select_teams(phi: np.ndarray, G: np.ndarray, K: int):
    """Gumbel-top-K (Algorithm 1, lines 3-12): the selected teams (ascending), their
    corrections c_g, the threshold tau and the team holding it (None when K = M)."""
    M = len(phi)
    K = min(K, M)
    if K == M:
        return np.arange(M), np.ones(M), None, None
    Y = phi + G
    order = np.lexsort((np.arange(M), -Y))          # Y descending, lower index first
    sel = np.sort(order[:K])
    thr = int(order[K])
    tau = Y[thr]
    c = -np.expm1(-np.exp(phi[sel] - tau))           # Eq. 7: 1 - exp(-exp(phi - tau))
    return sel, c, tau, thr


def estimate_sums(q, keys, values, teams, suffix, sel, c):
    """Eq. 4 with unshifted exponentials: ``(U_hat, Z_hat)`` for the selected teams
    ``sel`` with corrections ``c`` and the exact suffix rows ``suffix``."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d = len(q)
    U = np.zeros(values.shape[1])
    Z = 0.0
    for i in suffix:
        a = math.exp(float(keys[i] @ q) / math.sqrt(d))
        U = U + a * values[i]
        Z += a
    for g, cg in zip(sel, c):
        members = teams[g][0]
        a = np.exp(keys[members] @ q / math.sqrt(d))
        U = U + (a @ values[members]) / cg
        Z += float(a.sum()) / cg
    return U, Z


def estimate(q, keys, values, teams, suffix, sel, c) -> np.ndarray:
    """``o = U_hat / Z_hat`` (reading 6: exponentials shifted by the largest score)."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    d = len(q)
    rows = [np.asarray(suffix, dtype=np.int64)] + [teams[g][0] for g in sel]
    weight = [np.ones(len(rows[0]))] + [np.full(len(teams[g][0]), 1.0 / cg) for g, cg in zip(sel, c)]
    rows = np.concatenate(rows)
    weight = np.concatenate(weight)
    if len(rows) == 0:
        return np.zeros(values.shape[1])
    s = keys[rows] @ q / math.sqrt(d)
    a = np.exp(s - s.max()) * weight
    return (a @ values[rows]) / a.sum()


def decode_head(q, keys, values, teams, N: int, n: int, K: int, seed: int, b: int, h: int):
    """SANTA++ for one query head (Algorithm 1): ``dict(sel, c, tau, thr, phi, Y, o)``.
    ``keys``/``values`` are the sequence's ``n`` rows, the first ``N`` the prompt
    that ``teams`` partitions; rows ``N .. n-1`` are the exact suffix."""
    rep = np.asarray(keys, dtype=np.float64)[[t[1] for t in teams]]
    sizes = np.array([len(t[0]) for t in teams])
    phi = routing_logits(q, rep, sizes)
    Gd = gumbel(seed, b, h, np.arange(len(teams)))
    sel, c, tau, thr = select_teams(phi, Gd, K)
    o = estimate(q, keys, values, teams, np.arange(N, n), sel, c)
    return dict(sel=sel, c=c, tau=tau, thr=thr, phi=phi, Y=phi + Gd, o=o)
