"""Pins for the oracle's rectangular forward (fewer queries than keys, with a
query offset for the causal mask) and for its merge of partial results over
disjoint key sets. CPU only.

Reading (not on the pages): with Nq queries over Nk keys the queries are the
last Nq positions of the key sequence (q_offset = Nk - Nq), so causal query i
sees keys 0 .. Nk - Nq + i; for Nq = Nk this is the square causal mask. A row
that sees no key has O = 0 and LSE = -inf.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def brute_rect(q, k, v, scale, causal, q_offset):
    """Triple loop with math.exp over a rectangular score matrix."""
    nq, nk, d = len(q), len(k), len(v[0])
    o = np.zeros((nq, d))
    lse = np.full(nq, -np.inf)
    for i in range(nq):
        row = [(j, scale * sum(q[i][t] * k[j][t] for t in range(len(q[0]))))
               for j in range(nk) if not (causal and j > q_offset + i)]
        if not row:
            continue
        mx = max(s for _, s in row)
        den = sum(math.exp(s - mx) for _, s in row)
        for j, s in row:
            for t in range(d):
                o[i, t] += math.exp(s - mx) / den * v[j][t]
        lse[i] = mx + math.log(den)
    return o, lse


@pytest.fixture
def rng():
    return np.random.default_rng(4242)


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 9), (3, 5), (4, 16), (7, 7), (2, 30)])
@pytest.mark.parametrize("causal", [False, True])
def test_rect_forward_brute_force(rng, nq, nk, causal):
    d = 3
    q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    for off in sorted({nk - nq, 0, nk - 1, -1}):
        o, lse = oracle.attention_forward(q, k, v, 0.7, causal, q_offset=off)
        ob, lb = brute_rect(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, off)
        assert np.max(np.abs(o - ob)) <= 1e-12
        fin = np.isfinite(lb)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - lb[fin]), initial=0.0) <= 1e-12


def test_offset_rows_match_square_causal(rng):
    # the last nq rows of square causal attention are the rectangular problem
    n, nq, d = 40, 6, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o_sq, l_sq = oracle.attention_forward(q, k, v, 0.3, True)
    o, lse = oracle.attention_forward(q[-nq:], k, v, 0.3, True, q_offset=n - nq)
    assert np.max(np.abs(o - o_sq[-nq:])) <= 1e-13
    assert np.max(np.abs(lse - l_sq[-nq:])) <= 1e-13


def test_rect_matches_torch_sdpa_bottom_right(rng):
    nq, nk, d = 5, 37, 16
    q = rng.standard_normal((2, nq, d))
    k, v = rng.standard_normal((2, nk, d)), rng.standard_normal((2, nk, d))
    allowed = torch.arange(nk)[None, :] <= (nk - nq) + torch.arange(nq)[:, None]
    for causal in (False, True):
        o, _ = oracle.attention_forward(q, k, v, 0.25, causal, q_offset=nk - nq)
        ot = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.25,
            attn_mask=allowed if causal else None).numpy()
        assert np.max(np.abs(o - ot)) <= 1e-12


# ---------------------------------------------------------------- merge

def _parts_of(q, k, v, scale, index_sets):
    outs = [oracle.attention_forward(q, k[ix], v[ix], scale, False) for ix in index_sets]
    return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])


def check_merge_union(merge, rng):
    """Merging attention over disjoint key sets gives attention over their union."""
    for nq, nk, parts, contiguous in [(3, 20, 4, True), (2, 31, 3, False), (1, 8, 8, True)]:
        d = 4
        q, k, v = rng.standard_normal((nq, d)), rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
        perm = np.arange(nk) if contiguous else rng.permutation(nk)
        sets = np.array_split(perm, parts)
        o_p, l_p = _parts_of(q, k, v, 0.9, sets)
        o, lse = merge(o_p, l_p)
        ob, lb = brute_rect(q.tolist(), k.tolist(), v.tolist(), 0.9, False, 0)
        if not (np.max(np.abs(o - ob)) <= 1e-12 and np.max(np.abs(lse - lb)) <= 1e-12):
            return False
    return True


def check_merge_closed_forms(merge, rng):
    o1, o2 = rng.standard_normal((2, 3, 5))
    a = rng.standard_normal(3)
    # one part: unchanged
    o, lse = merge(o1[None], a[None])
    if not (np.allclose(o, o1, atol=1e-15, rtol=0) and np.allclose(lse, a, atol=1e-15, rtol=0)):
        return False
    # two parts with equal LSE: the average, LSE + ln 2
    o, lse = merge(np.stack([o1, o2]), np.stack([a, a]))
    if not (np.allclose(o, (o1 + o2) / 2, atol=1e-14, rtol=0)
            and np.allclose(lse, a + math.log(2), atol=1e-14, rtol=0)):
        return False
    # an empty part (LSE = -inf) is ignored whatever its O holds
    junk = np.full_like(o1, np.nan)
    o, lse = merge(np.stack([o1, junk]), np.stack([a, np.full(3, -np.inf)]))
    if not (np.allclose(o, o1, atol=1e-15, rtol=0) and np.allclose(lse, a, atol=1e-15, rtol=0)):
        return False
    # large LSE values: no overflow (the merge works relative to the max)
    o, lse = merge(np.stack([o1, o2]), np.stack([a + 1000.0, a + 1000.0]))
    if not (np.all(np.isfinite(o)) and np.allclose(lse, a + 1000.0 + math.log(2), atol=1e-12, rtol=0)):
        return False
    # every part empty: O = 0, LSE = -inf
    o, lse = merge(np.stack([junk, junk]), np.full((2, 3), -np.inf))
    return bool(np.all(o == 0.0) and np.all(np.isneginf(lse)))


MERGE_CHECKS = [check_merge_union, check_merge_closed_forms]


@pytest.mark.parametrize("check", MERGE_CHECKS)
def test_merge_pins(check, rng):
    assert check(oracle.merge_partials, rng)


def _mutant_merge(kind):
    def merge(o_parts, lse_parts):
        o_parts = np.asarray(o_parts, dtype=np.float64)
        lse_parts = np.asarray(lse_parts, dtype=np.float64)
        m = np.max(lse_parts, axis=0)
        m_safe = np.where(np.isneginf(m), 0.0, m)
        if kind == "no_max_shift":
            w = np.exp(lse_parts)
            tot = np.sum(w, axis=0)
            lse = np.log(tot)
            o = np.sum((w / tot)[..., None] * np.nan_to_num(o_parts), axis=0)
            return o, lse
        w = np.exp(lse_parts - m_safe[None])
        tot = np.sum(w, axis=0)
        lse = m_safe + np.log(np.where(tot > 0, tot, 1.0))
        if kind == "lse_is_max":
            lse = m
        coef = w / np.where(tot > 0, tot, 1.0)[None]
        if kind == "unnormalised":
            coef = w
        o = np.sum(np.where(coef[..., None] > 0, coef[..., None] * o_parts, 0.0), axis=0)
        return o, np.where(tot > 0, lse, -np.inf)
    return merge


@pytest.mark.parametrize("kind", ["no_max_shift", "lse_is_max", "unnormalised"])
def test_planted_merge_mistakes_are_caught(kind, rng):
    mutant = _mutant_merge(kind)
    with np.errstate(over="ignore", invalid="ignore"):
        assert not all(check(mutant, np.random.default_rng(4242)) for check in MERGE_CHECKS)
