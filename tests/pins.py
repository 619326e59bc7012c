"""Checks that pin an attention forward implementation to facts fixed by the
mathematics (brute force, closed forms, invariants, library special cases).

Each check takes the implementation under test as ``fwd(q, k, v, scale, causal)
-> (O, LSE)`` so the same checks run on the oracle (must pass) and on oracle
copies with a planted mistake (must fail), on the CPU.
"""

import math

import numpy as np
import torch


def brute_force(q, k, v, scale, causal):
    """Triple loop with math.exp: the definition, one element at a time."""
    n, d = len(q), len(q[0])
    o = [[0.0] * d for _ in range(n)]
    lse = [0.0] * n
    for i in range(n):
        row = []
        for j in range(n):
            if causal and j > i:
                continue
            row.append((j, scale * sum(q[i][t] * k[j][t] for t in range(d))))
        mx = max(s for _, s in row)
        den = sum(math.exp(s - mx) for _, s in row)
        for j, s in row:
            w = math.exp(s - mx) / den
            for t in range(d):
                o[i][t] += w * v[j][t]
        lse[i] = mx + math.log(den)
    return np.array(o), np.array(lse)


def check_brute_force(fwd, rng, tol=1e-12):
    for n, d, causal in [(1, 3, False), (5, 2, True), (7, 4, False), (12, 5, True), (9, 3, False)]:
        q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
        scale = float(rng.uniform(0.2, 1.5))
        o, lse = fwd(q, k, v, scale, causal)
        ob, lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        if not (np.max(np.abs(o - ob)) <= tol and np.max(np.abs(lse - lb)) <= tol):
            return False
    return True


def check_sdpa(fwd, rng, tol=1e-11):
    """torch's CPU float64 scaled_dot_product_attention and logsumexp."""
    for n, d, causal in [(33, 8, False), (40, 16, True)]:
        q, k, v = (rng.standard_normal((2, n, d)) for _ in range(3))
        scale = 1.0 / math.sqrt(d)
        o, lse = fwd(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale).numpy()
        s = scale * torch.matmul(tq, tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        lt = torch.logsumexp(s, dim=-1).numpy()
        if not (np.max(np.abs(o - ot)) <= tol and np.max(np.abs(lse - lt)) <= tol):
            return False
    return True


def check_closed_forms(fwd, rng, tol=1e-12):
    d = 6
    # one key: O = V_0, LSE = scale q.k
    q, k, v = (rng.standard_normal((1, d)) for _ in range(3))
    o, lse = fwd(q, k, v, 0.7, False)
    if not (np.allclose(o, v, atol=tol, rtol=0) and abs(lse[0] - 0.7 * float(q[0] @ k[0])) <= tol):
        return False
    # constant V rows: O rows all equal that row
    n = 11
    q, k = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    row = rng.standard_normal(d)
    for causal in (False, True):
        o, _ = fwd(q, k, np.tile(row, (n, 1)), 0.9, causal)
        if np.max(np.abs(o - row)) > tol:
            return False
    # causal row 0: O_0 = V_0, LSE_0 = scale q_0.k_0
    v = rng.standard_normal((n, d))
    o, lse = fwd(q, k, v, 0.9, True)
    if np.max(np.abs(o[0] - v[0])) > tol or abs(lse[0] - 0.9 * float(q[0] @ k[0])) > tol:
        return False
    # Q = 0: uniform weights. Non-causal O = column mean of V, LSE = ln N;
    # causal O_i = mean(V_0..V_i), LSE_i = ln(i + 1)
    z = np.zeros((n, d))
    o, lse = fwd(z, k, v, 1.3, False)
    if np.max(np.abs(o - v.mean(axis=0))) > tol or np.max(np.abs(lse - math.log(n))) > tol:
        return False
    o, lse = fwd(z, k, v, 1.3, True)
    cm = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    if np.max(np.abs(o - cm)) > tol or np.max(np.abs(lse - np.log(np.arange(1, n + 1)))) > tol:
        return False
    return True


def check_row_shift_invariance(fwd, rng, tol=1e-12):
    """Adding c_i to every score of row i leaves O unchanged and moves LSE_i by c_i.

    A per-row score shift is produced through the inputs: append a column to q
    holding c_i / scale and a column of ones to k.
    """
    n, d = 10, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    c = rng.uniform(-5, 5, size=n)
    scale = 0.8
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, scale, causal)
        q2 = np.concatenate([q, (c / scale)[:, None]], axis=1)
        k2 = np.concatenate([k, np.ones((n, 1))], axis=1)
        o2, l2 = fwd(q2, k2, v, scale, causal)
        if np.max(np.abs(o1 - o2)) > tol or np.max(np.abs(l2 - (l1 + c))) > 1e-11:
            return False
    return True


ALL_FORWARD_CHECKS = (check_brute_force, check_sdpa, check_closed_forms, check_row_shift_invariance)
