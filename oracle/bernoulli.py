"""CPU oracle of Bernoulli qK^T with the mean group query, combined with SANTA
-- TEST INFRASTRUCTURE ONLY (only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may use it; the product path never
does).

"Stochastic Sparse Attention for Memory-Bound Inference", section 5: Bernoulli
sampling of the query zeroes out features, so that only the key features the
sampled query keeps are read, and the score is estimated as
``p_hat = (norm / B) * sum_n q_hat^(n) K^T`` (Eq. 5) from B samples ("B
stratified samples", Table 7).  Section 5.1: a GQA group uses one
representative query, the mean of its queries' absolute values, ``m``, whose
Monte Carlo estimate ``m_hat`` selects the features for the whole group, and
every head's score is ``p_hat = (m_hat * q / m) K^T`` (Eq. 6).  Section 5.3
feeds these scores to SANTA.  The appendix with the sampler is not in the
pages; the readings taken here:

1. ``m_i = (1/G) sum_h |q_{h,i}|`` over the group's G query heads (fp64, heads
   summed in order);
2. feature i is kept by draw n with probability ``pi_i = m_i / max_j m_j``:
   draws are stratified, draw n keeps i iff ``(n + U_{i,n}) / B < pi_i``, so
   the number of draws that keep i is ``floor(B pi_i)`` or ``ceil(B pi_i)``
   with mean ``B pi_i``;
3. ``m_hat_i = (max_j m_j / B) * count_i``, an unbiased estimate of ``m_i``;
   for a single head (G = 1) this is Eq. 5 with ternary samples
   ``q_hat^(n)_i = sign(q_i) [draw n keeps i]`` and ``norm = max_i |q_i|``;
4. ``s_hat_{h,j} = sum_i (m_hat_i / m_i) q_{h,i} k_{j,i}`` (features with
   ``m_i = 0`` contribute nothing), unbiased for ``q_h . k_j``;
5. ``U_{i,n}`` is ``(w0 >> 11) * 2**-53`` of Philox4x64-10 with key
   ``(seed, 1)`` and counter ``(n, i, g, b)`` (the SANTA sampler uses key
   ``(seed, 0)``; the same published generator as oracle/santa.py);
6. SANTA then runs on the estimated scores exactly as in oracle/santa.py:
   ``softmax(s_hat / sqrt(d))``, the sampling rule, and the gather-mean of the
   sampled value rows.

The decisions ``(n + U)/B < pi_i`` are taken in IEEE fp64 (sums in a fixed
order, correctly rounded division), as the GPU takes them.
"""
from __future__ import annotations

import math

import numpy as np

from . import santa as O


def feature_uniforms(seed: int, b: int, g: int, feature, B: int) -> np.ndarray:
    """U[0, 1) draws n = 0 .. B-1 of feature(s) ``feature`` of group (b, g) (reading 5):
    shape ``[B]`` for one feature, ``[len(feature), B]`` for an array of them."""
    n = np.arange(B, dtype=np.uint64)
    f = np.asarray(feature, dtype=np.uint64)
    w0, _, _, _ = O.philox4x64((n[None, :], f.reshape(-1, 1), np.uint64(g), np.uint64(b)), (seed, 1))
    u = (w0 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    return u[0] if f.ndim == 0 else u


def mean_group_query(q_group: np.ndarray) -> np.ndarray:
    """``m = (1/G) sum_h |q_h|`` (reading 1), heads summed in order."""
    q_group = np.asarray(q_group, dtype=np.float64)
    acc = np.zeros(q_group.shape[1])
    for h in range(q_group.shape[0]):
        acc = acc + np.abs(q_group[h])
    return acc / q_group.shape[0]


def feature_counts(m: np.ndarray, B: int, seed: int, b: int, g: int) -> np.ndarray:
    """How many of the B stratified draws keep each feature (reading 2)."""
    m = np.asarray(m, dtype=np.float64)
    top = m.max()
    if top == 0.0:
        return np.zeros(len(m), dtype=np.int64)
    pi = m / top
    u = feature_uniforms(seed, b, g, np.arange(len(m)), B)            # [d, B]
    keep = (np.arange(B, dtype=np.float64)[None, :] + u) / B < pi[:, None]
    return keep.sum(axis=1).astype(np.int64)


def estimated_scores(q_group: np.ndarray, keys: np.ndarray, B: int, seed: int, b: int, g: int):
    """``s_hat [G, n]`` (before the 1/sqrt(d) scale) and the feature counts of the group
    (readings 1-4): ``s_hat_h = (m_hat * q_h / m) K^T``."""
    q_group = np.asarray(q_group, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    m = mean_group_query(q_group)
    counts = feature_counts(m, B, seed, b, g)
    m_hat = (m.max() / B) * counts if m.max() > 0 else np.zeros_like(m)
    ratio = np.divide(m_hat, m, out=np.zeros_like(m), where=m > 0)
    return (q_group * ratio) @ keys.T, counts


def decode_group(q_group, keys, values, S: int, mode: int, B: int, seed: int, b: int, g: int, G: int):
    """Bernoulli qK^T + SANTA for the G heads of group (b, g): per head ``dict(idx, t,
    F, p, delta, o, s)`` and the group's feature counts (reading 6).  Head h of the
    group is query head ``g * G + h``; its SANTA draws use that index."""
    d = np.asarray(q_group).shape[1]
    s_hat, counts = estimated_scores(q_group, keys, B, seed, b, g)
    out = []
    for h in range(G):
        s = s_hat[h] / math.sqrt(d)
        idx, t, F, p = O.sample_head(s, S, mode, seed, b, g * G + h)
        out.append(dict(idx=idx, t=t, F=F, p=p, s=s, delta=O.boundary_distance(F, idx, t),
                        o=O.estimate(values, idx)))
    return out, counts
