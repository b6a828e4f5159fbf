"""Pins for the headwise-chunked forward oracle (oracle.chunked), CPU only.

UPipe changes only which heads are resident at once (tilnote.io commentary, section on
activation memory), so the chunked result must equal the unchunked pack -> attention ->
unpack bit for bit, and its buffer accounting must reproduce the page's 87.5% figure for
q-shaped intermediates at one head per chunk out of eight."""
import numpy as np
import pytest

from oracle import attention, chunked, permute
from workloads import bits_to_f64


def _f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


@pytest.mark.parametrize("u", [1, 2, 3, 4])
@pytest.mark.parametrize("cu", [None, [0, 7, 20, 24]])
def test_chunked_equals_unchunked(u, cu):
    rng = np.random.default_rng(40 + u)
    P, s_l, Hq, Hkv, d = 2, 12, 8, 4, 3    # Hq_l = 4, Hkv_l = 2, G = 2
    to64 = lambda b: bits_to_f64(b, "f32")
    mk = lambda H: [_f32_bits(rng.standard_normal((s_l, H, d))) for _ in range(P)]
    qs, ks, vs = mk(Hq), mk(Hkv), mk(Hkv)
    os_ = [np.zeros((s_l, Hq, d), dtype=np.uint32) for _ in range(P)]
    for r in range(P):
        got, lse = chunked.forward(qs, ks, vs, os_, r, u, 0.5, True, cu, to_f64=to64, from_f64=_f32_bits)
        o, lse_ref = attention.forward(to64(permute.pack(qs, r)), to64(permute.pack(ks, r)),
                                       to64(permute.pack(vs, r)), 0.5, True, cu)
        want = permute.unpack(_f32_bits(o), r, os_)
        for a, b in zip(got, want):
            np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(lse, lse_ref)


def test_workspace_matches_upipe_reduction():
    s, Hq_l, G, d = 262144, 8, 8, 128
    full = 2 * s * Hq_l * d + 2 * s * (Hq_l // G) * d          # Q, O head shards + K, V
    u1 = chunked.workspace_elems(s, Hq_l, G, d, 1)
    u2 = chunked.workspace_elems(s, Hq_l, G, d, 2)
    assert full * 2 == 1152 * 2**20 and u1 * 2 == 256 * 2**20 and u2 * 2 == 384 * 2**20
    q_full, q_u1 = 2 * s * Hq_l * d, 2 * s * 1 * d
    assert 1 - q_u1 / q_full == 0.875   # the 87.5% attention-intermediate reduction


def test_workspace_spans_kv_heads():
    # Hq_l = 4, G = 2: chunks of 3 heads span kv heads {0,1} then {1}
    assert chunked.workspace_elems(10, 4, 2, 2, 3) == 2 * 10 * 3 * 2 + 2 * 10 * 2 * 2


@pytest.mark.parametrize("u", [1, 3, 4])
@pytest.mark.parametrize("cu", [None, [0, 5, 17, 24]])
def test_chunked_backward_equals_unchunked(u, cu):
    """Summing per-chunk dK/dV over the chunks that read a kv head gives the unchunked
    GQA gradient; dQ of every head is that head's own gradient. u = 3 makes a chunk span
    two kv heads and the next chunk re-read one of them (Hq_l = 4, G = 2)."""
    rng = np.random.default_rng(70 + u)
    P, s_l, Hq, Hkv, d = 2, 12, 8, 4, 3
    to64 = lambda b: bits_to_f64(b, "f32")
    mk = lambda H: [_f32_bits(rng.standard_normal((s_l, H, d))) for _ in range(P)]
    qs, ks, vs, gs = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    for r in range(P):
        dq, dk, dv = chunked.backward(qs, ks, vs, gs, r, u, 0.5, True, cu, to_f64=to64)
        wq, wk, wv = attention.backward(*(to64(permute.pack(x, r)) for x in (qs, ks, vs, gs)), 0.5, True, cu)
        np.testing.assert_array_equal(dq, wq)
        np.testing.assert_allclose(dk, wk, rtol=0, atol=1e-12)
        np.testing.assert_allclose(dv, wv, rtol=0, atol=1e-12)
        assert np.abs(dk).max() > 0.1 and np.abs(dv).max() > 0.1


def test_chunked_backward_planted_drop_fails():
    """A schedule that forgets to sum a re-read kv head's earlier contribution (keeping
    only the last chunk's) must differ from the unchunked gradient: the check above can
    see that mistake."""
    rng = np.random.default_rng(5)
    P, s_l, Hq, Hkv, d = 2, 10, 8, 4, 3
    to64 = lambda b: bits_to_f64(b, "f32")
    mk = lambda H: [_f32_bits(rng.standard_normal((s_l, H, d))) for _ in range(P)]
    qs, ks, vs, gs = mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)
    # u = 1: each chunk holds one q head, so kv head g is read by two chunks
    qf, kf, vf, gf = (to64(permute.pack(x, 0)) for x in (qs, ks, vs, gs))
    _, wk, _ = attention.backward(qf, kf, vf, gf, 0.5, True, None)
    _, last_only, _ = attention.backward(qf[:, 1:2], kf[:, 0:1], vf[:, 0:1], gf[:, 1:2], 0.5, True, None)
    assert np.abs(last_only[:, 0] - wk[:, 0]).max() > 1e-3
    _, dk, _ = chunked.backward(qs, ks, vs, gs, 0, 1, 0.5, True, None, to_f64=to64)
    np.testing.assert_allclose(dk, wk, rtol=0, atol=1e-12)
