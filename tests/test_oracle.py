"""Pins of the CPU oracle to facts fixed outside it (CPU only).

The oracle is checked against brute force, hand-derived golden cases, closed
forms, invariants, torch's float64 library routines, the pages' own tiled
recurrence (both loop orders) and finite differences. A set of oracle copies
with planted mistakes must each fail at least one check, which shows the
checks can see those mistakes.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as att
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def oracle_fwd(q, k, v, scale, causal):
    return oracle.attention_forward(q, k, v, scale, causal)


@pytest.fixture
def rng():
    return np.random.default_rng(12345)


# ---------------------------------------------------------------- forward pins

@pytest.mark.parametrize("check", pins.ALL_FORWARD_CHECKS, ids=lambda f: f.__name__)
def test_forward_pins(check, rng):
    assert check(oracle_fwd, rng)


def test_golden_forward():
    cases = json.load(open(GOLDEN))["forward"]
    for c in cases:
        o, lse = oracle.attention_forward(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                          c["scale"], c["causal"])
        np.testing.assert_allclose(o, np.array(c["o"]), atol=1e-14, rtol=0, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["lse"]), atol=1e-14, rtol=0, err_msg=c["name"])


def test_softmax_rows_properties(rng):
    n = 37
    q, k = rng.standard_normal((n, 8)), rng.standard_normal((n, 8))
    for causal in (False, True):
        p, m, l = oracle.softmax_rows(oracle.scores(q, k, 0.5, causal))
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-14 * n
        if causal:
            assert np.all(p[np.triu_indices(n, 1)] == 0)
            assert p[0, 0] == 1.0
        # shift invariance of the softmax itself
        c = rng.uniform(-30, 30, size=(n, 1))
        p2, _, _ = oracle.softmax_rows(oracle.scores(q, k, 0.5, causal) + c)
        assert np.max(np.abs(p - p2)) <= 1e-13


def test_large_scores_are_stable(rng):
    """Scores near 1e3 overflow exp() unless the row max is subtracted first."""
    n, d = 16, 4
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = oracle.attention_forward(q * 60, k * 60, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    ob, lb = pins.brute_force((q * 60).tolist(), (k * 60).tolist(), v.tolist(), 1.0, False)
    np.testing.assert_allclose(o, ob, atol=1e-9, rtol=0)


def test_row_chunking_is_exact(rng):
    n, d = 50, 8
    q, k, v, do = (rng.standard_normal((2, n, d)) for _ in range(4))
    for causal in (False, True):
        o1, l1 = oracle.attention_forward(q, k, v, 0.3, causal)
        o2, l2 = oracle.attention_forward(q, k, v, 0.3, causal, chunk_elems=7 * n)
        np.testing.assert_allclose(o1, o2, atol=1e-14, rtol=0)
        np.testing.assert_allclose(l1, l2, atol=1e-14, rtol=0)
        g1 = oracle.attention_backward(q, k, v, do, 0.3, causal)
        g2 = oracle.attention_backward(q, k, v, do, 0.3, causal, chunk_elems=3 * n)
        for a, b in zip(g1, g2):
            np.testing.assert_allclose(a, b, atol=1e-13, rtol=0)


def test_forward_rows_matches_full(rng):
    n, d = 40, 8
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    rows = np.array([0, 1, 17, 39])
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.4, causal)
        o2, l2 = oracle.attention_forward_rows(q, k, v, rows, 0.4, causal)
        np.testing.assert_allclose(o2, o[rows], atol=1e-14, rtol=0)
        np.testing.assert_allclose(l2, lse[rows], atol=1e-14, rtol=0)


# ----------------------------------------------------- the pages' tiled recurrence

@pytest.mark.parametrize("order", ["kv_outer", "q_outer"])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_two_pass(order, causal, rng):
    fn = oracle.online_forward_kv_outer if order == "kv_outer" else oracle.online_forward_q_outer
    n, d = 53, 16
    q, k, v = (rng.standard_normal((n, d)) * 2 for _ in range(3))
    o_ref, l_ref = oracle.attention_forward(q, k, v, 0.25, causal)
    for br, bc in [(8, 8), (16, 5), (7, 13), (53, 53), (64, 4), (1, 1)]:
        o, lse = fn(q, k, v, 0.25, causal, br, bc)
        assert np.max(np.abs(o - o_ref)) <= 1e-12, (br, bc)
        assert np.max(np.abs(lse - l_ref)) <= 1e-12, (br, bc)


# --------------------------------------------------------------- backward pins

def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_forward(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(causal, rng):
    n, d, scale, h = 7, 3, 0.6, 1e-6
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*grad.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            num[idx] = (_loss(*args_p, do, scale, causal) - _loss(*args_m, do, scale, causal)) / (2 * h)
        rel = np.linalg.norm(num - grad) / max(np.linalg.norm(grad), 1e-30)
        assert rel <= 1e-6, (which, rel)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_autograd_fp64(causal, rng):
    n, d, scale = 29, 8, 1 / math.sqrt(8)
    q, k, v, do = (rng.standard_normal((2, n, d)) for _ in range(4))
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, scale, causal)
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), atol=1e-12, rtol=0)


def test_backward_invariants(rng):
    n, d, scale = 31, 8, 0.35
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        dq, dk, dv, delta = oracle.attention_backward(q, k, v, do, scale, causal, return_delta=True)
        o, _ = oracle.attention_forward(q, k, v, scale, causal)
        # D_i = sum_j P_ij dP_ij equals sum_k dO_ik O_ik
        np.testing.assert_allclose(delta, np.sum(do * o, axis=1), atol=1e-12, rtol=0)
        # rows of dS sum to zero => sum_j dK_j = 0
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
        # rows of P sum to one => sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12, rtol=0)
    # one key: O = V_0 whatever q and k are, so dQ = dK = 0 and dV = dO
    q1, k1, v1, do1 = (rng.standard_normal((1, d)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward(q1, k1, v1, do1, 0.9, False)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv, do1, atol=1e-15, rtol=0)


def test_golden_backward():
    for c in json.load(open(GOLDEN))["backward"]:
        dq, dk, dv = oracle.attention_backward(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                               np.array(c["do"]), c["scale"], c["causal"])
        np.testing.assert_allclose(dq, np.array(c["dq"]), atol=1e-15, rtol=0)
        np.testing.assert_allclose(dk, np.array(c["dk"]), atol=1e-15, rtol=0)
        np.testing.assert_allclose(dv, np.array(c["dv"]), atol=1e-15, rtol=0)


# ------------------------------------------------------------------ e4m3 codec

def test_e4m3_known_codes():
    dec = oracle.e4m3_decode
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, val in known.items():
        assert dec(np.array([c]))[0] == val, hex(c)
    assert np.isnan(dec(np.array([0x7F]))[0]) and np.isnan(dec(np.array([0xFF]))[0])
    assert np.sum(np.isnan(dec(np.arange(256)))) == 2
    pos = dec(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E increase strictly


def test_e4m3_matches_torch_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.e4m3_decode(np.arange(256))
    same = (t == ours) | (np.isnan(t) & np.isnan(ours))
    assert np.all(same)


def test_e4m3_encode(rng):
    enc, dec = oracle.e4m3_encode, oracle.e4m3_decode
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)])
    assert np.all(enc(dec(finite)) == finite)  # round trip of every finite code
    # midpoint between 1.0 (0x38, even) and 1.125 (0x39) rounds to even 0x38;
    # midpoint between 1.125 and 1.25 (0x3A, even) rounds to 0x3A
    assert enc(np.array([1.0625]))[0] == 0x38
    assert enc(np.array([1.1875]))[0] == 0x3A
    assert enc(np.array([1e6, -1e6, 449.0, 464.0]))[0] == 0x7E
    assert enc(np.array([-1e6]))[0] == 0xFE
    assert enc(np.array([np.nan]))[0] == 0x7F
    x = rng.standard_normal(100000) * 50
    x = np.clip(x, -448, 448)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = enc(x)
    # -0.0 aside (sign of zero is not used by the kernels), codes agree
    assert np.all((t == ours) | ((t & 0x7F) == 0) & ((ours & 0x7F) == 0))
    # rounding error within half a unit in the last place
    err = np.abs(dec(ours) - x)
    ulp = np.where(np.abs(x) < 2 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2 ** -6))) - 3))
    assert np.all(err <= ulp / 2 + 1e-300)


def test_counted_flops():
    # forward 4*B*H*N^2*d, halved when causal; backward 2.5x
    assert oracle.counted_flops(1, 2, 128, 64, False) == 8388608
    assert abs(oracle.counted_flops(8, 16, 4096, 128, True) - 549.755813888e9) < 1
    assert abs(oracle.counted_flops(8, 16, 4096, 128, True, backward=True) - 1374.38953472e9) < 1


# ----------------------------------------- planted mistakes must fail the pins

def _mutant_forward(kind):
    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        if q.ndim == 3:
            outs = [fwd(q[i], k[i], v[i], scale, causal) for i in range(q.shape[0])]
            return np.stack([o for o, _ in outs]), np.stack([l for _, l in outs])
        n = q.shape[0]
        s = (q @ k.T) * (1.0 if kind == "no_scale" else scale)
        if kind == "sqrt_d_scale":
            s = (q @ k.T) / math.sqrt(q.shape[1])
        if causal:
            mask = np.tril(np.ones((n, n)), -1) > 0 if kind == "mask_transposed" else np.triu(np.ones((n, n)), 1) > 0
            s = np.where(mask, -np.inf, s)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        p = e / l[:, None]
        if kind == "p_transposed":
            p = p.T
        if kind == "column_softmax":
            e2 = np.exp(s - s.max(axis=0)[None, :])
            p = e2 / e2.sum(axis=0)[None, :]
        o = p @ v
        lse = m + np.log(l)
        if kind == "lse_log2":
            lse = m + np.log2(l)
        if kind == "lse_max_only":
            lse = m
        if kind == "k_for_v":
            o = p @ k[:, :v.shape[1]] if k.shape[1] >= v.shape[1] else p @ np.resize(k, v.shape)
        return o, lse
    return fwd


@pytest.mark.parametrize("kind", ["no_scale", "sqrt_d_scale", "mask_transposed", "p_transposed",
                                  "column_softmax", "lse_log2", "lse_max_only", "k_for_v"])
def test_planted_forward_mistakes_are_caught(kind):
    fwd = _mutant_forward(kind)
    caught = [not chk(fwd, np.random.default_rng(7)) for chk in pins.ALL_FORWARD_CHECKS]
    assert any(caught), kind


def test_unmutated_copy_passes_pins():
    fwd = _mutant_forward("none")
    assert all(chk(fwd, np.random.default_rng(7)) for chk in pins.ALL_FORWARD_CHECKS)
