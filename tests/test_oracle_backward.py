"""Pins for the attention backward oracle (oracle.attention.backward), CPU only.

Pins: central finite differences of L = sum(dO * O) through the scalar brute-force
forward, a two-token closed form, the softmax-gradient invariants, exact zeros, the GQA
sum rule and torch autograd in float64."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, brute


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("s,Hq,Hkv,d,causal,cu", [
    (5, 2, 1, 3, True, None),
    (6, 2, 2, 2, True, [0, 2, 6]),
    (4, 2, 1, 2, False, None),
])
def test_finite_differences(s, Hq, Hkv, d, causal, cu):
    rng = np.random.default_rng(20 + s)
    q, k, v, do = _rand(rng, s, Hq, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hq, d)
    scale = 0.8
    dq, dk, dv = attention.backward(q, k, v, do, scale, causal, cu)
    fq, fk, fv = brute.finite_diff_grads(q.copy(), k.copy(), v.copy(), do, scale, causal, cu)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-7)


def test_two_token_closed_form():
    # s=2, d=1, scale 1, dO = 1: row 1 has p = e^2/(e^2+e^-2) on key 0.
    q = np.array([[[1.0]], [[2.0]]])
    k = np.array([[[1.0]], [[-1.0]]])
    v = np.array([[[1.0]], [[3.0]]])
    do = np.ones((2, 1, 1))
    dq, dk, dv = attention.backward(q, k, v, do, 1.0, True)
    p = math.exp(2) / (math.exp(2) + math.exp(-2))
    o1 = p * 1 + (1 - p) * 3
    assert abs(dv[0, 0, 0] - (1 + p)) < 1e-15 and abs(dv[1, 0, 0] - (1 - p)) < 1e-15
    assert dq[0, 0, 0] == 0.0
    assert abs(dq[1, 0, 0] - (p * (1 - o1) * 1 + (1 - p) * (3 - o1) * (-1))) < 1e-14
    assert abs(dk[0, 0, 0] - 2 * p * (1 - o1)) < 1e-14
    assert abs(dk[1, 0, 0] - 2 * (1 - p) * (3 - o1)) < 1e-14


@pytest.mark.parametrize("cu", [None, [0, 9, 10, 30, 48]])
def test_invariants(cu):
    """Per document and kv head: sum_j dK_j = 0 (rows of dS sum to 0) and
    sum_j dV_j = sum of dO over the rows and q heads that read the kv head (rows of P sum to 1)."""
    rng = np.random.default_rng(30)
    s, Hq, Hkv, d = 48, 4, 2, 5
    G = Hq // Hkv
    q, k, v, do = _rand(rng, s, Hq, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hq, d)
    dq, dk, dv = attention.backward(q, k, v, do, 0.5, True, cu)
    bounds = cu if cu is not None else [0, s]
    for a, b in zip(bounds[:-1], bounds[1:]):
        for g in range(Hkv):
            np.testing.assert_allclose(dk[a:b, g].sum(axis=0), 0.0, atol=1e-12)
            want = do[a:b, g * G:(g + 1) * G].sum(axis=(0, 1))
            np.testing.assert_allclose(dv[a:b, g].sum(axis=0), want, rtol=1e-12, atol=1e-12)


def test_exact_zeros():
    rng = np.random.default_rng(31)
    s, H, d = 12, 2, 4
    q, k, v, do = _rand(rng, s, H, d), _rand(rng, s, H, d), _rand(rng, s, H, d), _rand(rng, s, H, d)
    _, dk, _ = attention.backward(np.zeros_like(q), k, v, do, 0.5)
    assert (dk == 0).all()  # Q = 0: dK = scale * dS^T Q = 0
    dq, _, _ = attention.backward(q, np.zeros_like(k), v, do, 0.5)
    assert (dq == 0).all()  # K = 0: dQ = scale * dS K = 0
    dq, _, _ = attention.backward(q, k, v, do, 0.5)
    # row 0 sees one key: its softmax is constant (zero up to the rounding of dO.V_0 - dO.O_0)
    np.testing.assert_allclose(dq[0], 0.0, atol=1e-15)


def test_gqa_grads_are_sums_of_mha_grads():
    rng = np.random.default_rng(32)
    s, Hkv, G, d = 14, 2, 3, 4
    q, k, v, do = _rand(rng, s, Hkv * G, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv * G, d)
    dq, dk, dv = attention.backward(q, k, v, do, 0.6)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dq2, dk2, dv2 = attention.backward(q, kr, vr, do, 0.6)
    np.testing.assert_allclose(dq, dq2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(s, Hkv, G, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(s, Hkv, G, d).sum(axis=2), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_torch_autograd_float64(causal):
    rng = np.random.default_rng(33)
    s, H, d = 21, 2, 8
    q, k, v, do = _rand(rng, s, H, d), _rand(rng, s, H, d), _rand(rng, s, H, d), _rand(rng, s, H, d)
    dq, dk, dv = attention.backward(q, k, v, do, 1 / math.sqrt(d), causal)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2).clone().requires_grad_(True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    o.backward(torch.from_numpy(do).permute(1, 0, 2))
    for mine, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(mine, ref.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


def test_subsets_match_full():
    rng = np.random.default_rng(34)
    s, Hq, Hkv, d = 1030, 2, 1, 3
    cu = [0, 400, 401, 1030]
    q, k, v, do = _rand(rng, s, Hq, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hq, d)
    dq, dk, dv = attention.backward(q, k, v, do, 0.4, True, cu)
    rows = np.array([0, 5, 399, 400, 401, 777, 1029])
    cols = np.array([400, 1000, 1029])
    dq2, dk2, dv2 = attention.backward(q, k, v, do, 0.4, True, cu, q_rows=rows, kv_cols=cols)
    np.testing.assert_allclose(dq2, dq[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk2, dk[cols], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dv2, dv[cols], rtol=1e-12, atol=1e-13)
    # keys in two documents, noncausal too
    cols = np.array([3, 390, 1020])
    for causal in (True, False):
        dq, dk, dv = attention.backward(q, k, v, do, 0.4, causal, cu)
        _, dk2, dv2 = attention.backward(q, k, v, do, 0.4, causal, cu, q_rows=np.zeros(0, int), kv_cols=cols)
        np.testing.assert_allclose(dk2, dk[cols], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dv2, dv[cols], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("cu", [None, [0, 7, 8, 20, 31]])
def test_rows_attending_is_exact(causal, cu):
    """By brute force over the mask: the rows that see at least one of the keys."""
    s = 31
    for keys in ([0], [30], [5, 6], [7], [3, 19, 25], [8, 30]):
        want = [i for i in range(s) if attention.allowed([i], keys, causal, cu).any()]
        assert list(attention.rows_attending(keys, s, causal, cu)) == want


def test_planted_missing_D_term_is_caught(monkeypatch):
    """The backward with D_i dropped (dS = P * dP) must fail the finite-difference pin."""
    rng = np.random.default_rng(35)
    s, d = 5, 2
    q, k, v, do = _rand(rng, s, 1, d), _rand(rng, s, 1, d), _rand(rng, s, 1, d), _rand(rng, s, 1, d)
    real_sum = np.sum

    def no_d(a, axis=None, **kw):
        r = real_sum(a, axis=axis, **kw)
        return r * 0.0 if axis == 1 else r
    monkeypatch.setattr(attention.np, "sum", no_d)
    dq, dk, _ = attention.backward(q, k, v, do, 0.9)
    monkeypatch.undo()
    fq, fk, _ = brute.finite_diff_grads(q.copy(), k.copy(), v.copy(), do, 0.9)
    assert not np.allclose(dq, fq, atol=1e-6) or not np.allclose(dk, fk, atol=1e-6)
