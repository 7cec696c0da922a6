"""CPU oracle of the deterministic top-k attention comparator -- TEST
INFRASTRUCTURE ONLY (only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; the product path never does).

"Stochastic Sparse Attention for Memory-Bound Inference" compares SANTA with
top-k attention at a matched budget k = S (§3.4; §6, Related Work: top-k
truncates the value stage deterministically and is biased).  The appendix that
defines the comparator is not in the pages; the "Stratified Sparse Attention"
page's second decode stage is a radix top-k over a score array, returned
unsorted.  Readings taken here:

1. the scores are the exact ``s_i = q . k_i / sqrt(d)`` (§2, Eq. 1) over the
   whole cache;
2. the kept set is the ``k = min(S, n)`` keys with the largest scores; among
   keys with equal scores the lower token index is kept first (a deterministic
   rule; the pages give none);
3. the output is attention restricted to the kept set and renormalised,
   ``o = sum_{i in T} exp(s_i) v_i / sum_{i in T} exp(s_i)``;
4. ``idx`` lists the kept keys in ascending token order (the order of a radix
   selection is arbitrary; ascending order makes the output layout unique),
   padded with -1 when ``n < S``; a sequence of length 0 gives ``o = 0``.

Everything is float64 NumPy, one query head at a time.
"""
from __future__ import annotations

import math

import numpy as np


def scores(q: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """``q K^T / sqrt(d)`` for one query (Eq. 1)."""
    q = np.asarray(q, dtype=np.float64)
    return (np.asarray(keys, dtype=np.float64) @ q) / math.sqrt(q.shape[0])


def select(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the ``min(k, n)`` largest scores, lower index first among equal
    scores (reading 2), returned in ascending index order (reading 4)."""
    s = np.asarray(s, dtype=np.float64)
    k = min(int(k), len(s))
    order = np.lexsort((np.arange(len(s)), -s))      # by score descending, then index ascending
    return np.sort(order[:k]).astype(np.int64)


def threshold(s: np.ndarray, k: int) -> float:
    """The k-th largest score (the selection boundary)."""
    s = np.sort(np.asarray(s, dtype=np.float64))[::-1]
    return float(s[min(int(k), len(s)) - 1])


def estimate(s: np.ndarray, values: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Softmax over the kept keys only, applied to their value rows (reading 3)."""
    s = np.asarray(s, dtype=np.float64)[kept]
    w = np.exp(s - s.max())
    return (w[:, None] * np.asarray(values, dtype=np.float64)[kept]).sum(axis=0) / math.fsum(w)


def decode_head(q, keys, values, S: int):
    """Top-k attention for one query head: ``dict(idx, o, s, thr)`` with ``idx``
    padded to ``S`` entries by -1."""
    n = len(keys)
    if n == 0:
        return dict(idx=np.full(S, -1, dtype=np.int64), o=np.zeros(np.asarray(q).shape[0]), s=None, thr=None)
    s = scores(q, keys)
    kept = select(s, S)
    idx = np.full(S, -1, dtype=np.int64)
    idx[:len(kept)] = kept
    return dict(idx=idx, o=estimate(s, values, kept), s=s, thr=threshold(s, S))
