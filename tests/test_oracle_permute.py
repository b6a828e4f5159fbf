"""Pins for the permute oracle (oracle.permute), CPU only.

Each pin fixes the oracle from outside itself: a hand-derived fixture, the closed-form
index map, a library routine (numpy concatenate + slice), and the structural facts the
pages state (the second all-to-all undoes the first; across ranks the exchange moves
every element exactly once)."""
import os

import numpy as np
import pytest

from oracle import permute


def _index_shards(P, s_l, H, d):
    """Shard p holds, at (t, h, x), the flat index of (p, t, h, x) in a [P, s_l, H, d] array."""
    flat = np.arange(P * s_l * H * d, dtype=np.int32).reshape(P, s_l, H, d)
    return [flat[p].copy() for p in range(P)]


def test_golden_hand_derived(golden_dir):
    rows = [l for l in open(os.path.join(golden_dir, "permute_P2_r1.txt")) if not l.startswith("#")]
    P, s_l, H, d, r = map(int, rows[0].split())
    want = np.array([[int(x) for x in l.split()] for l in rows[1:]], dtype=np.int32)
    shards = []
    for p in range(P):
        a = np.zeros((s_l, H, d), dtype=np.int32)
        for t in range(s_l):
            for h in range(H):
                a[t, h, 0] = 100 * p + 10 * t + h
        shards.append(a)
    got = permute.pack(shards, r)
    assert got.shape == (P * s_l, H // P, d)
    np.testing.assert_array_equal(got[:, :, 0], want)


@pytest.mark.parametrize("P,s_l,H,d", [(2, 3, 4, 2), (4, 5, 8, 3), (3, 2, 6, 1), (1, 4, 2, 2)])
def test_closed_form_index_map(P, s_l, H, d):
    shards = _index_shards(P, s_l, H, d)
    Hl = H // P
    for r in range(P):
        y = permute.pack(shards, r)
        for row in range(P * s_l):
            for j in range(Hl):
                for x in range(d):
                    p, t = divmod(row, s_l)
                    assert y[row, j, x] == ((p * s_l + t) * H + r * Hl + j) * d + x


@pytest.mark.parametrize("P,s_l,H,d", [(2, 7, 4, 8), (4, 6, 8, 4), (8, 3, 8, 2)])
def test_matches_library_concatenate(P, s_l, H, d):
    rng = np.random.default_rng(1)
    shards = [rng.integers(0, 2**16, (s_l, H, d)).astype(np.uint16) for _ in range(P)]
    Hl = H // P
    for r in range(P):
        want = np.concatenate(shards, axis=0)[:, r * Hl:(r + 1) * Hl]
        np.testing.assert_array_equal(permute.pack(shards, r), want)


@pytest.mark.parametrize("P,s_l,H,d", [(2, 5, 4, 3), (4, 3, 8, 2)])
def test_unpack_inverts_pack(P, s_l, H, d):
    rng = np.random.default_rng(2)
    shards = [rng.integers(0, 2**32, (s_l, H, d), dtype=np.uint64).astype(np.uint32) for _ in range(P)]
    blank = [np.zeros_like(x) for x in shards]
    out = blank
    for r in range(P):
        out = permute.unpack(permute.pack(shards, r), r, out)
    for a, b in zip(out, shards):
        np.testing.assert_array_equal(a, b)


def test_all_ranks_move_every_element_once():
    P, s_l, H, d = 4, 3, 8, 2
    shards = _index_shards(P, s_l, H, d)
    seen = np.concatenate([permute.pack(shards, r).ravel() for r in range(P)])
    np.testing.assert_array_equal(np.sort(seen), np.arange(P * s_l * H * d))


def test_unpack_touches_only_own_heads():
    P, s_l, H, d = 2, 4, 4, 2
    shards = _index_shards(P, s_l, H, d)
    y = np.full((P * s_l, H // P, d), -1, dtype=np.int32)
    out = permute.unpack(y, 1, shards)
    for p in range(P):
        np.testing.assert_array_equal(out[p][:, :2], shards[p][:, :2])
        assert (out[p][:, 2:] == -1).all()


def test_head_subrange():
    P, s_l, H, d = 2, 3, 8, 2
    shards = _index_shards(P, s_l, H, d)
    full = permute.pack(shards, 1)
    part = permute.pack(shards, 1, h0=4 + 1, nh=2)
    np.testing.assert_array_equal(part, full[:, 1:3])


def test_heads_must_divide():
    shards = [np.zeros((2, 3, 1), dtype=np.uint16) for _ in range(2)]
    with pytest.raises(ValueError):
        permute.pack(shards, 0)


# ---- the send-side / receive-side permutes of a real all-to-all, and kv-head replication ----

def _exchange(bufs):
    """The all-to-all itself (test harness): block r of source rank p's buffer becomes block p
    of destination rank r's buffer."""
    P = len(bufs)
    return [np.stack([bufs[p][r] for p in range(P)]) for r in range(P)]


@pytest.mark.parametrize("P,H", [(1, 3), (2, 4), (4, 8), (4, 2), (8, 2), (4, 4), (8, 1)])
def test_send_pack_closed_form(P, H):
    s_l, d = 5, 3
    idx = np.arange(s_l * H * d, dtype=np.int32).reshape(s_l, H, d)
    out = permute.send_pack(idx, P)
    nh = max(H // P, 1)
    assert out.shape == (P, s_l, nh, d)
    for r in range(P):
        h0 = r * H // P
        for t in range(s_l):
            for j in range(nh):
                for x in range(d):
                    assert out[r, t, j, x] == (t * H + h0 + j) * d + x


@pytest.mark.parametrize("P,H", [(2, 4), (4, 8), (3, 6), (4, 4)])
def test_send_then_exchange_equals_pack(P, H):
    rng = np.random.default_rng(P * 10 + H)
    s_l, d = 6, 8
    shards = [rng.integers(0, 65535, size=(s_l, H, d), dtype=np.uint16) for _ in range(P)]
    recv = _exchange([permute.send_pack(x, P) for x in shards])
    Hl = H // P
    for r in range(P):
        got = recv[r].reshape(P * s_l, Hl, d)
        np.testing.assert_array_equal(got, permute.pack(shards, r))
        np.testing.assert_array_equal(got, np.concatenate(shards)[:, r * Hl:(r + 1) * Hl])


@pytest.mark.parametrize("P,H", [(4, 2), (8, 2), (8, 1), (4, 1)])
def test_replicated_heads_reach_their_ranks(P, H):
    rng = np.random.default_rng(P + 7 * H)
    s_l, d = 4, 8
    shards = [rng.integers(0, 65535, size=(s_l, H, d), dtype=np.uint16) for _ in range(P)]
    recv = _exchange([permute.send_pack(x, P) for x in shards])
    R = P // H
    for r in range(P):
        np.testing.assert_array_equal(recv[r].reshape(P * s_l, 1, d), np.concatenate(shards)[:, r // R:r // R + 1])
    # every head reaches exactly R ranks
    counts = np.zeros(H, int)
    for r in range(P):
        counts[permute.rank_heads(r, P, H)[0]] += 1
    assert (counts == R).all()


@pytest.mark.parametrize("P,H", [(2, 4), (4, 8), (4, 4), (1, 2)])
def test_recv_unpack_inverts_the_exchange(P, H):
    rng = np.random.default_rng(3 * P + H)
    s_l, d = 5, 8
    shards = [rng.integers(0, 65535, size=(s_l, H, d), dtype=np.uint16) for _ in range(P)]
    heads = [permute.pack(shards, r).reshape(P, s_l, H // P, d) for r in range(P)]   # every rank's head shard
    back = _exchange(heads)                                                          # to the token owners
    for p in range(P):
        np.testing.assert_array_equal(permute.recv_unpack(back[p], P, H), shards[p])


def test_f32_to_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ties = ((rng.integers(0, 0x7F80, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)   # exact ties, finite
    for v in (x, ties, np.array([0.0, -0.0, 1.0, -3.5], dtype=np.float32)):
        want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(permute.f32_to_bf16_bits(v), want)


@pytest.mark.parametrize("P,H", [(4, 2), (8, 2), (8, 1)])
def test_replica_sum_of_equal_copies(P, H):
    """R replicas holding the same bf16 values sum to R times them, exactly (R a power of two)."""
    import torch
    rng = np.random.default_rng(P * H)
    s_l, d = 3, 8
    x = torch.randn(s_l, d).to(torch.bfloat16)
    blocks = np.stack([x.view(torch.int16).numpy().view(np.uint16)[:, None, :]] * P)   # [P, s_l, 1, d]
    R = P // H
    want = (x * R).view(torch.int16).numpy().view(np.uint16)
    got = permute.recv_unpack(blocks, P, H)
    for h in range(H):
        np.testing.assert_array_equal(got[:, h, :], want)


@pytest.mark.parametrize("P,H", [(4, 2), (8, 1)])
def test_replica_sum_within_rounding_of_the_exact_sum(P, H):
    rng = np.random.default_rng(11 + P)
    s_l, d = 16, 32
    vals = rng.standard_normal((P, s_l, 1, d)).astype(np.float32)
    blocks = permute.f32_to_bf16_bits(vals)
    got = permute.recv_unpack(blocks, P, H)
    f = permute._bits_to_f32(blocks).astype(np.float64)
    R = P // H
    for h in range(H):
        exact = f[h * R:(h + 1) * R].sum(0)[:, 0, :]
        g = permute._bits_to_f32(got[:, h, :]).astype(np.float64)
        bound = np.abs(g) * 2.0 ** -8 + R * 2.0 ** -23 * np.abs(f[h * R:(h + 1) * R]).sum(0)[:, 0, :]
        assert (np.abs(g - exact) <= bound).all()
        # a dropped replica is far outside that bound
        assert (np.abs(g - (exact - f[h * R][:, 0, :])) > bound).any()
