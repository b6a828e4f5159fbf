"""Pins for the attention forward oracle (oracle.attention.forward), CPU only.

A mistake anywhere in the oracle (a dropped scale, a transposed mask, a wrong GQA head
map, a wrong document boundary, a missing normaliser) fails at least one pin here; the
planted-mistake tests at the end check that for several such mistakes."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, brute, permute

RTOL = 1e-12


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _cases():
    # (s, Hq, Hkv, d, causal, cu)
    return [
        (7, 2, 2, 3, True, None),
        (9, 4, 2, 4, True, None),
        (8, 2, 1, 3, False, None),
        (10, 2, 1, 4, True, [0, 3, 4, 10]),
        (12, 4, 2, 2, True, [0, 5, 12]),
        (6, 2, 2, 3, False, [0, 2, 6]),
    ]


@pytest.mark.parametrize("s,Hq,Hkv,d,causal,cu", _cases())
def test_matches_brute_force(s, Hq, Hkv, d, causal, cu):
    rng = np.random.default_rng(s * 31 + Hq)
    q, k, v = _rand(rng, s, Hq, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d)
    scale = 0.7
    o, lse = attention.forward(q, k, v, scale, causal, cu)
    ob, lb = brute.forward(q.tolist(), k.tolist(), v.tolist(), scale, causal, cu)
    np.testing.assert_allclose(o, np.array(ob), rtol=RTOL, atol=1e-13)
    np.testing.assert_allclose(lse, np.array(lb), rtol=RTOL, atol=1e-13)


def _read_q0(golden_dir):
    vals = {}
    for line in open(os.path.join(golden_dir, "q0_prefix_means.txt")):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        if parts[0] == "V":
            vals["V"] = np.array([float(x) for x in parts[1:]]).reshape(4, 1, 2)
        else:
            vals[(parts[0], parts[1])] = np.array([float(x) for x in parts[2:]])
    return vals


def test_q0_golden(golden_dir):
    g = _read_q0(golden_dir)
    v = g["V"]
    q = np.zeros((4, 1, 2))
    k = np.random.default_rng(0).standard_normal((4, 1, 2))
    for tag, cu in (("causal", None), ("packed", [0, 2, 4])):
        o, lse = attention.forward(q, k, v, 0.3, True, cu)
        np.testing.assert_allclose(o[:, 0].ravel(), g[(tag, "O")], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0], np.log(g[(tag, "N")]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("cu", [None, [0, 17, 18, 40, 64]])
def test_q0_prefix_means(cu):
    rng = np.random.default_rng(5)
    s, d = 64, 5
    q = np.zeros((s, 2, d))
    k, v = _rand(rng, s, 1, d), _rand(rng, s, 1, d)
    o, lse = attention.forward(q, k, v, 0.2, True, cu)
    lo = attention.doc_start(np.arange(s), cu)
    for i in range(s):
        want = v[lo[i]:i + 1, 0].mean(axis=0)
        for h in range(2):
            np.testing.assert_allclose(o[i, h], want, rtol=1e-13, atol=1e-14)
            assert abs(lse[h, i] - math.log(i - lo[i] + 1)) < 1e-13


def test_two_token_closed_form():
    # s=2, d=1, scale 1: row 0 sees key 0 only; row 1 sees scores 2 and -2.
    q = np.array([[[1.0]], [[2.0]]])
    k = np.array([[[1.0]], [[-1.0]]])
    v = np.array([[[1.0]], [[3.0]]])
    o, lse = attention.forward(q, k, v, 1.0, True)
    a, b = math.exp(2.0), math.exp(-2.0)
    assert o[0, 0, 0] == 1.0 and lse[0, 0] == 1.0
    assert abs(o[1, 0, 0] - (a + 3 * b) / (a + b)) < 1e-15
    assert abs(lse[0, 1] - math.log(a + b)) < 1e-15


def test_single_token_returns_v():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 1, 4, 8), _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 8)
    o, lse = attention.forward(q, k, v, 0.5, True)
    np.testing.assert_array_equal(o, v[:, [0, 0, 1, 1]])
    np.testing.assert_allclose(lse[:, 0], 0.5 * np.einsum("hd,hd->h", q[0], k[0, [0, 0, 1, 1]]), rtol=1e-15)


def test_value_scaling_is_linear():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 16, 2, 4), _rand(rng, 16, 1, 4), _rand(rng, 16, 1, 4)
    o1, l1 = attention.forward(q, k, v, 0.5)
    o2, l2 = attention.forward(q, k, 3.0 * v, 0.5)
    np.testing.assert_allclose(o2, 3.0 * o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("G", [2, 4])
def test_gqa_equals_mha_with_repeated_kv(G):
    rng = np.random.default_rng(G)
    s, Hkv, d = 20, 2, 6
    q, k, v = _rand(rng, s, Hkv * G, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d)
    o, l = attention.forward(q, k, v, 0.4)
    kr = torch.from_numpy(k).repeat_interleave(G, dim=1).numpy()
    vr = torch.from_numpy(v).repeat_interleave(G, dim=1).numpy()
    o2, l2 = attention.forward(q, kr, vr, 0.4)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_packed_equals_per_document_runs():
    rng = np.random.default_rng(6)
    cu = [0, 5, 6, 19, 40]
    s, d = cu[-1], 4
    q, k, v = _rand(rng, s, 4, d), _rand(rng, s, 2, d), _rand(rng, s, 2, d)
    o, l = attention.forward(q, k, v, 0.6, True, cu)
    for a, b in zip(cu[:-1], cu[1:]):
        od, ld = attention.forward(q[a:b], k[a:b], v[a:b], 0.6, True)
        np.testing.assert_allclose(o[a:b], od, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l[:, a:b], ld, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("P,G", [(2, 1), (4, 2), (2, 4)])
def test_sharded_then_permuted_equals_unsharded(P, G):
    """Each rank: pack -> attention on its heads -> unpack; together = attention on all heads."""
    rng = np.random.default_rng(10 + P)
    s_l, Hkv, d = 6, 2 * P, 3
    Hq = Hkv * G
    s = P * s_l
    qg, kg, vg = _rand(rng, s, Hq, d), _rand(rng, s, Hkv, d), _rand(rng, s, Hkv, d)
    want, _ = attention.forward(qg, kg, vg, 0.5)
    split = lambda a: [a[p * s_l:(p + 1) * s_l].copy() for p in range(P)]
    qs, ks, vs = split(qg), split(kg), split(vg)
    outs = [np.zeros((s_l, Hq, d)) for _ in range(P)]
    for r in range(P):
        o, _ = attention.forward(permute.pack(qs, r), permute.pack(ks, r), permute.pack(vs, r), 0.5)
        outs = permute.unpack(o, r, outs)
    np.testing.assert_array_equal(np.concatenate(outs, axis=0), want)


@pytest.mark.parametrize("causal", [True, False])
def test_library_sdpa_float64(causal):
    rng = np.random.default_rng(7)
    s, H, d = 33, 3, 8
    q, k, v = _rand(rng, s, H, d), _rand(rng, s, H, d), _rand(rng, s, H, d)
    o, _ = attention.forward(q, k, v, 1 / math.sqrt(d), causal)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_row_subset_matches_full():
    rng = np.random.default_rng(8)
    s = 1100  # spans three row blocks
    q, k, v = _rand(rng, s, 2, 4), _rand(rng, s, 1, 4), _rand(rng, s, 1, 4)
    cu = [0, 300, 301, 1100]
    o, l = attention.forward(q, k, v, 0.3, True, cu)
    rows = np.array([0, 299, 300, 301, 512, 1023, 1099])
    o2, l2 = attention.forward(q, k, v, 0.3, True, cu, rows=rows)
    # a different row block spans a different key range, so BLAS may round differently
    np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, l[:, rows], rtol=1e-13, atol=1e-14)


# ---- planted mistakes: each variant of the oracle must fail a pin above -------------

def _brute_mismatch(monkeypatch_target=None):
    rng = np.random.default_rng(11)
    cu = [0, 4, 9]
    q, k, v = _rand(rng, 9, 4, 3), _rand(rng, 9, 2, 3), _rand(rng, 9, 2, 3)
    o, l = attention.forward(q, k, v, 0.7, True, cu)
    ob, lb = brute.forward(q.tolist(), k.tolist(), v.tolist(), 0.7, True, cu)
    return not (np.allclose(o, ob, rtol=1e-10) and np.allclose(l, lb, rtol=1e-10))


def test_planted_transposed_mask_is_caught(monkeypatch):
    real = attention.allowed
    # key j visible to row i iff i <= j: the causal mask transposed
    monkeypatch.setattr(attention, "allowed", lambda r, c, causal, cu: real(c, r, causal, cu).T)
    monkeypatch.setattr(attention, "_key_range", lambda br, s, causal: np.arange(s))
    assert _brute_mismatch()


def test_planted_document_boundary_off_by_one_is_caught(monkeypatch):
    real = attention.allowed
    monkeypatch.setattr(attention, "allowed",
                        lambda r, c, causal, cu: real(r, c, causal, None if cu is None else [x + (0 < x < cu[-1]) for x in cu]))
    assert _brute_mismatch()


def test_planted_gqa_map_is_caught(monkeypatch):
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 8, 4, 3), _rand(rng, 8, 2, 3), _rand(rng, 8, 2, 3)
    ob, _ = brute.forward(q.tolist(), k.tolist(), v.tolist(), 0.5, True)
    # the oracle with q head h reading kv head h % Hkv instead of h // G
    o = np.zeros_like(q)
    for h in range(4):
        o1, _ = attention.forward(q[:, h:h + 1], k[:, [h % 2]], v[:, [h % 2]], 0.5)
        o[:, h] = o1[:, 0]
    assert not np.allclose(o, ob)
    o_ok, _ = attention.forward(q, k, v, 0.5)
    assert np.allclose(o_ok, ob, rtol=1e-12)


@pytest.mark.parametrize("P,Hq,Hkv", [(4, 8, 2), (8, 8, 1), (4, 8, 4)])
def test_replicated_then_sharded_equals_unsharded(P, Hq, Hkv):
    """Kv heads fewer than the ranks (replicated: each kv head goes to the P / Hkv ranks whose q
    heads read it), the exchange as send-side permute + all-to-all + receive-side permute: every
    rank's local attention, with the gradients of a replicated kv head summed over its ranks on
    the way back, equals attention on the unsharded tensors (float64)."""
    from oracle import permute
    rng = np.random.default_rng(P + Hq + Hkv)
    s_l, d = 5, 4
    s = P * s_l
    glob = {n: rng.standard_normal((s, H, d)) for n, H in (("q", Hq), ("k", Hkv), ("v", Hkv), ("do", Hq))}
    shards = {n: [g[p * s_l:(p + 1) * s_l] for p in range(P)] for n, g in glob.items()}
    exch = lambda bufs: [np.stack([bufs[p][r] for p in range(P)]) for r in range(P)]
    recv = {n: exch([permute.send_pack(x, P) for x in shards[n]]) for n in shards}
    heads = lambda n, r: recv[n][r].reshape(s, recv[n][r].shape[2], d)
    o_h, dq_h, dk_h, dv_h = [], [], [], []
    for r in range(P):
        q, k, v, do = (heads(n, r) for n in ("q", "k", "v", "do"))
        o_h.append(attention.forward(q, k, v, 0.5, True)[0])
        dq, dk, dv = attention.backward(q, k, v, do, 0.5, True)
        dq_h.append(dq), dk_h.append(dk), dv_h.append(dv)
    back = lambda outs, H: np.concatenate([permute.recv_unpack(b, P, H)
                                           for b in exch([x.reshape(P, s_l, x.shape[1], d) for x in outs])])
    wo, _ = attention.forward(glob["q"], glob["k"], glob["v"], 0.5, True)
    wq, wk, wv = attention.backward(glob["q"], glob["k"], glob["v"], glob["do"], 0.5, True)
    np.testing.assert_allclose(back(o_h, Hq), wo, atol=1e-12)
    np.testing.assert_allclose(back(dq_h, Hq), wq, atol=1e-12)
    np.testing.assert_allclose(back(dk_h, Hkv), wk, atol=1e-12)
    np.testing.assert_allclose(back(dv_h, Hkv), wv, atol=1e-12)
