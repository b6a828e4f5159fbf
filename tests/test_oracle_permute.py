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
