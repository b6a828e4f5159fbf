"""Pins of the Ring Attention oracle: the ring over all ranks equals attention over the whole
sequence (forward and backward, causal and not, GQA), the LSE merge equals the softmax over
the union of the key blocks, and the hop schedule covers exactly the visible blocks."""
import numpy as np
import pytest

from oracle import attention, ring


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("P,causal", [(1, True), (3, True), (4, False), (4, True)])
def test_hops_cover_the_visible_blocks(P, causal):
    for r in range(P):
        h = ring.hops(P, r, causal)
        assert h[0] == r                                   # the rank's own block first
        assert sorted(h) == (list(range(r + 1)) if causal else list(range(P)))


@pytest.mark.parametrize("P,Hq,Hkv,causal", [(4, 4, 2, True), (3, 2, 2, False), (2, 6, 3, True), (1, 2, 1, True)])
def test_ring_forward_equals_unsharded(P, Hq, Hkv, causal):
    rng = np.random.default_rng(P * 10 + Hq)
    s_l, d = 7, 4
    q, k, v = _rand(rng, P * s_l, Hq, d), _rand(rng, P * s_l, Hkv, d), _rand(rng, P * s_l, Hkv, d)
    split = lambda x: [x[p * s_l:(p + 1) * s_l] for p in range(P)]
    wo, wl = attention.forward(q, k, v, 0.6, causal)
    for r in range(P):
        o, lse = ring.forward(split(q), split(k), split(v), r, 0.6, causal)
        np.testing.assert_allclose(o, wo[r * s_l:(r + 1) * s_l], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, wl[:, r * s_l:(r + 1) * s_l], rtol=1e-12, atol=1e-13)


def test_merge_equals_softmax_over_the_union():
    """Two halves of one key set, merged, give the softmax over all of it (closed form: the
    unmasked attention of the concatenated keys)."""
    rng = np.random.default_rng(5)
    s, d = 6, 3
    q, k, v = _rand(rng, s, 2, d), _rand(rng, 2 * s, 1, d), _rand(rng, 2 * s, 1, d)
    S = 0.5 * np.einsum("ihd,jd->hij", q, k[:, 0])
    m = S.max(-1, keepdims=True)
    e = np.exp(S - m)
    want_o = np.einsum("hij,jd->ihd", e / e.sum(-1, keepdims=True), v[:, 0])
    want_l = (m[..., 0] + np.log(e.sum(-1)))
    parts = [attention.forward(q, k[:s], v[:s], 0.5, causal=False),
             attention.forward(q, k[s:], v[s:], 0.5, causal=False)]
    o, l = ring.merge(parts)
    np.testing.assert_allclose(o, want_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, want_l, rtol=1e-12, atol=1e-13)
    o1, l1 = ring.merge(parts[:1])                        # one part: unchanged
    np.testing.assert_allclose(o1, parts[0][0], rtol=1e-14)
    np.testing.assert_allclose(l1, parts[0][1], rtol=1e-14)


@pytest.mark.parametrize("P,Hq,Hkv,causal", [(4, 4, 2, True), (3, 2, 2, False), (2, 2, 1, True)])
def test_ring_backward_equals_unsharded(P, Hq, Hkv, causal):
    rng = np.random.default_rng(P + 3 * Hq)
    s_l, d = 6, 4
    q, k, v, do = (_rand(rng, P * s_l, H, d) for H in (Hq, Hkv, Hkv, Hq))
    split = lambda x: [x[p * s_l:(p + 1) * s_l] for p in range(P)]
    wq, wk, wv = attention.backward(q, k, v, do, 0.6, causal)
    dk = [np.zeros((s_l, Hkv, d)) for _ in range(P)]
    dv = [np.zeros((s_l, Hkv, d)) for _ in range(P)]
    for r in range(P):
        dq, contrib = ring.backward(split(q), split(k), split(v), split(do), r, 0.6, causal)
        np.testing.assert_allclose(dq, wq[r * s_l:(r + 1) * s_l], rtol=1e-11, atol=1e-12)
        for src, (a, b) in contrib.items():
            dk[src] += a
            dv[src] += b
    np.testing.assert_allclose(np.concatenate(dk), wk, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(np.concatenate(dv), wv, rtol=1e-11, atol=1e-12)


def test_planted_wrong_merge_weight_is_caught(monkeypatch):
    """A merge that forgets to renormalise (weights exp(LSE_i) instead of exp(LSE_i - LSE))
    fails the unsharded-equality pin."""
    rng = np.random.default_rng(8)
    P, s_l, d = 3, 5, 4
    q, k, v = (_rand(rng, P * s_l, 2, d) for _ in range(3))
    split = lambda x: [x[p * s_l:(p + 1) * s_l] for p in range(P)]

    def bad(parts):
        lses = np.stack([l for _, l in parts])
        return sum(o_i * np.exp(l_i).T[:, :, None] for (o_i, _), l_i in zip(parts, lses)), np.log(np.exp(lses).sum(0))
    monkeypatch.setattr(ring, "merge", bad)
    o, _ = ring.forward(split(q), split(k), split(v), 2, 0.6, True)
    wo, _ = attention.forward(q, k, v, 0.6, True)
    assert not np.allclose(o, wo[2 * s_l:])
