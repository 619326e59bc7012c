"""Blocked online-softmax attention in float64 -- the pages' tiling algorithm.

Source: "11.11 Flash Attention" (algomaster.io), sections "Flash Attention: The
Key Insight" (a running maximum and a running sum of exponentials, with earlier
partial results corrected when a later tile reveals a larger value) and "The
Tiling Algorithm" (Q in blocks of B_r rows, K/V in blocks of B_c rows; per tile:
local scores, local row max, new running max, exponentials against the new
max, rescaled running sum, rescaled output). Section "Flash Attention 2" of the
same page swaps the loop order (Q blocks outer, K/V blocks inner) and trims the
non-matmul work; that variant keeps the output unnormalised and divides by the
running sum once at the end.

This module exists only to pin the oracle: the tests require both loop orders
to agree with the two-pass definition in ``attention.py`` to ~1e-12 for block
sizes that do and do not divide N, which is the pages' claim that the tiled
computation is exact rather than an approximation. The pages' listing omits
the score scale; here ``scale`` multiplies Q K^T as in the formula.
"""

import numpy as np


def _tile_scores(qi, kj, scale, causal, i0, j0):
    s = scale * (qi @ kj.T)
    if causal:
        rows = i0 + np.arange(qi.shape[0])[:, None]
        cols = j0 + np.arange(kj.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def online_forward_kv_outer(q, k, v, scale, causal, block_r, block_c):
    """K/V blocks in the outer loop, Q blocks inner (the pages' v1 order).

    The normalised output O_i, the running max m_i and the running sum l_i of
    every Q block live in (simulated) HBM and are read and rewritten at each
    step: O_i <- (e^{m_i - m_new} l_i O_i + P_ij V_j) / l_new.
    One head, inputs [N, d]. Returns (O, LSE).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    o = np.zeros((n, d))
    l = np.zeros(n)
    m = np.full(n, -np.inf)
    for j0 in range(0, n, block_c):
        kj, vj = k[j0:j0 + block_c], v[j0:j0 + block_c]
        for i0 in range(0, n, block_r):
            sl = slice(i0, i0 + block_r)
            s = _tile_scores(q[sl], kj, scale, causal, i0, j0)
            m_tile = np.max(s, axis=1)
            m_new = np.maximum(m[sl], m_tile)
            seen = np.isfinite(m_new)  # rows with at least one visible key so far
            safe = np.where(seen, m_new, 0.0)
            keep = np.where(seen, np.exp(m[sl] - safe), 0.0)  # e^{m_old - m_new}
            p = np.exp(s - safe[:, None])                     # masked -> 0
            l_new = keep * l[sl] + np.sum(p, axis=1)
            num = (keep * l[sl])[:, None] * o[sl] + p @ vj
            o[sl] = np.where(seen[:, None], num / np.where(seen, l_new, 1.0)[:, None], 0.0)
            l[sl] = l_new
            m[sl] = m_new
    return o, m + np.log(l)


def online_forward_q_outer(q, k, v, scale, causal, block_r, block_c):
    """Q blocks in the outer loop, K/V blocks inner (the pages' v2 order).

    Per Q block the accumulator stays unnormalised: acc <- alpha acc + P V_j,
    l <- alpha l + rowsum(P), alpha = e^{m_old - m_new}; one division by l at
    the end. One head, inputs [N, d]. Returns (O, LSE).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    o = np.empty((n, d))
    lse = np.empty(n)
    for i0 in range(0, n, block_r):
        qi = q[i0:i0 + block_r]
        r = qi.shape[0]
        acc = np.zeros((r, d))
        l = np.zeros(r)
        m = np.full(r, -np.inf)
        for j0 in range(0, n, block_c):
            s = _tile_scores(qi, k[j0:j0 + block_c], scale, causal, i0, j0)
            m_new = np.maximum(m, np.max(s, axis=1))
            seen = np.isfinite(m_new)
            safe = np.where(seen, m_new, 0.0)
            alpha = np.where(seen, np.exp(m - safe), 1.0)
            p = np.exp(s - safe[:, None])
            l = alpha * l + np.sum(p, axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j0 + block_c]
            m = m_new
        o[i0:i0 + r] = acc / l[:, None]
        lse[i0:i0 + r] = m + np.log(l)
    return o, lse
