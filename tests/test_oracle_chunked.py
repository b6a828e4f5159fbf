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
