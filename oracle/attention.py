"""Exact attention in float64 on the CPU, from the plain definition.

Sources (web pages on FlashAttention):
- "11.11 Flash Attention" (algomaster.io), section "Standard Attention: Step by
  Step": Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V computed as three
  steps -- S = Q K^T, P = softmax(S), O = P V.
- Same page, section "Flash Attention: The Key Insight": the safe softmax of a
  row needs that row's maximum (for stability) and the sum of its
  exponentials.
- "Walk through the FlashAttention algorithm..." (zenaique.com), interviewer
  follow-up on the backward pass: the forward keeps only Q, K, V and the
  per-row statistics m and l, and the backward recomputes attention from them.
  Here the statistics are saved folded into one number per row,
  LSE_i = m_i + ln(l_i), since exp(S_ij - LSE_i) = exp(S_ij - m_i) / l_i.

Readings where the pages are silent:
- ``scale`` multiplies Q K^T (the pages' formula uses 1/sqrt(d_k); their
  tiling pseudocode omits it). LSE is in natural-log units of the scaled
  scores.
- Causal: query i sees keys 0..i (N_q = N_k = N); masked scores are -inf, so
  no row is ever fully masked.
- The backward is the chain rule through O = P V and the softmax Jacobian
  diag(p) - p p^T (the pages give no gradient formulas).

Layout: any leading dimensions ``[..., N, d]``; the functions loop over them
one head at a time, and over query rows in chunks so that a chunk of S never
exceeds ``chunk_elems`` float64 elements.
"""

import numpy as np

_DEFAULT_CHUNK_ELEMS = 1 << 25  # 256 MiB of float64 per score chunk


def scores(q, k, scale, causal, row0=0):
    """S = scale * q k^T for one head, with causal entries (key > query) = -inf.

    ``q`` holds query rows row0, row0+1, ... of the head (so a row chunk keeps
    its absolute query index for the causal mask); ``k`` holds all N keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T)
    if causal:
        rows = row0 + np.arange(q.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def softmax_rows(s):
    """Two-pass safe softmax of each row: returns (P, m, l).

    m_i = max_j S_ij; E_ij = exp(S_ij - m_i); l_i = sum_j E_ij; P = E / l.
    """
    m = np.max(s, axis=1)
    e = np.exp(s - m[:, None])
    l = np.sum(e, axis=1)
    return e / l[:, None], m, l


def _heads(x):
    x = np.asarray(x, dtype=np.float64)
    lead = x.shape[:-2]
    return x.reshape((-1,) + x.shape[-2:]), lead


def _row_chunk(n, chunk_elems):
    return max(1, min(n, chunk_elems // max(n, 1)))


def attention_forward(q, k, v, scale, causal, chunk_elems=_DEFAULT_CHUNK_ELEMS, q_offset=0):
    """O = softmax(scale q k^T [masked]) v and LSE_i = m_i + ln l_i.

    Inputs ``[..., N, d]`` (queries) and ``[..., Nk, d]`` (keys, values; Nk may
    differ from N); returns O ``[..., N, d]`` and LSE ``[..., N]`` (float64).
    ``q_offset`` is the position of the first query in the key sequence: with
    ``causal`` query i sees keys 0 .. q_offset + i. With N queries taken as the
    last N of Nk positions (decoding), q_offset = Nk - N; a row that sees no
    key at all gets O = 0 and LSE = -inf.
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    nh, n, _ = qh.shape
    dv = vh.shape[-1]
    o = np.empty((nh, n, dv))
    lse = np.empty((nh, n))
    rc = _row_chunk(n, chunk_elems)
    for h in range(nh):
        for r0 in range(0, n, rc):
            r1 = min(n, r0 + rc)
            s = scores(qh[h, r0:r1], kh[h], scale, causal, row0=q_offset + r0)
            empty = np.all(np.isneginf(s), axis=1)
            if np.any(empty):
                s = np.where(empty[:, None], 0.0, s)
            p, m, l = softmax_rows(s)
            o[h, r0:r1] = np.where(empty[:, None], 0.0, p @ vh[h])
            lse[h, r0:r1] = np.where(empty, -np.inf, m + np.log(l))
    return o.reshape(lead + (n, dv)), lse.reshape(lead + (n,))


def merge_partials(o_parts, lse_parts):
    """Combine attention over disjoint key sets into attention over their union.

    ``o_parts`` [P, ..., d] and ``lse_parts`` [P, ...] hold, for each part p,
    the normalised output O_p = sum_j exp(S_j - LSE_p) V_j and LSE_p =
    ln sum_j exp(S_j) over that part's keys. Over the union the softmax
    denominator is the sum of the parts' denominators, so
      LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p
    (the rescaling of partial results by exp(m_old - m_new) in "11.11 Flash
    Attention", section "Flash Attention: The Key Insight", applied once to
    whole parts). Parts with LSE_p = -inf (no visible key) contribute
    nothing; if every part is empty the result is O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=0)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    w = np.exp(lse_parts - m_safe[None])                # 0 for empty parts
    tot = np.sum(w, axis=0)
    lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    coef = np.where(tot[None] > 0, w / np.where(tot > 0, tot, 1.0)[None], 0.0)
    # an empty part's O is never read (its weight is exactly 0)
    o = np.sum(np.where(coef[..., None] > 0, coef[..., None] * o_parts, 0.0), axis=0)
    return o, lse


def attention_forward_rows(q, k, v, rows, scale, causal):
    """Forward for a subset of query rows of ONE head ([N, d] inputs).

    Each output row depends only on its own query row and all keys, so a
    sample of rows is computed with the same definition as the full forward.
    Returns (O[rows], LSE[rows]).
    """
    q = np.asarray(q, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.size, v.shape[1]))
    lse = np.empty(rows.size)
    for t, r in enumerate(rows):
        s = scores(q[r:r + 1], k, scale, causal, row0=int(r))
        p, m, l = softmax_rows(s)
        o[t] = (p @ v)[0]
        lse[t] = m[0] + np.log(l[0])
    return o, lse


def attention_backward(q, k, v, do, scale, causal,
                       chunk_elems=_DEFAULT_CHUNK_ELEMS, return_delta=False):
    """Gradients of L = <O, dO> with respect to q, k and v.

    With P the (masked) softmax of S = scale q k^T:
      dV = P^T dO
      dP = dO V^T
      D_i = sum_j P_ij dP_ij
      dS = P * (dP - D_i)            (masked entries have P = 0, hence dS = 0)
      dQ = scale dS K,   dK = scale dS^T Q
    P is recomputed from the definition (two-pass softmax), row chunk by row
    chunk; dK and dV accumulate over the chunks.
    """
    qh, lead = _heads(q)
    kh, _ = _heads(k)
    vh, _ = _heads(v)
    doh, _ = _heads(do)
    nh, n, d = qh.shape
    dq = np.empty_like(qh)
    dk = np.zeros_like(kh)
    dv = np.zeros_like(vh)
    delta = np.empty((nh, n))
    rc = _row_chunk(n, chunk_elems)
    for h in range(nh):
        for r0 in range(0, n, rc):
            r1 = min(n, r0 + rc)
            s = scores(qh[h, r0:r1], kh[h], scale, causal, row0=r0)
            p, _, _ = softmax_rows(s)
            dov = doh[h, r0:r1]
            dv[h] += p.T @ dov
            dp = dov @ vh[h].T
            dd = np.sum(p * dp, axis=1)
            ds = p * (dp - dd[:, None])
            dq[h, r0:r1] = scale * (ds @ kh[h])
            dk[h] += scale * (ds.T @ qh[h, r0:r1])
            delta[h, r0:r1] = dd
    out = (dq.reshape(lead + (n, d)), dk.reshape(lead + (n, d)),
           dv.reshape(lead + (n, vh.shape[-1])))
    if return_delta:
        return out + (delta.reshape(lead + (n,)),)
    return out


def counted_flops(b, h, n, d, causal, backward=False):
    """Counted FLOPs of the benchmark convention: 4*B*H*N^2*d for the forward
    (two N x N x d contractions at 2 FLOPs per multiply-add), exactly half when
    causal, and 2.5 times the forward for the backward (five contractions)."""
    f = 4.0 * b * h * n * n * d
    if causal:
        f *= 0.5
    return 2.5 * f if backward else f
