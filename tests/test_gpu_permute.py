"""GPU parity of the permutes (ulysses_pack / ulysses_unpack) against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import permute as OP
from tests.helpers import gen_shards, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return W.bits_from_torch(t)


def _rand_shards(P, s_l, H, d, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "bf16":
        host = [rng.integers(0, 2**16, (s_l, H, d), dtype=np.uint16) for _ in range(P)]
    else:
        host = [rng.integers(0, 2**32, (s_l, H, d), dtype=np.uint64).astype(np.uint32) for _ in range(P)]
    return host, [to_dev(x, dtype) for x in host]


@pytest.mark.parametrize("P,s_l,H,d,dtype", [
    (2, 256, 4, 64, "f32"),     # tiny fp32 case
    (4, 2048, 32, 128, "bf16"), # Qwen3-4B SP=4 share at 8K, q heads
    (4, 2048, 8, 128, "bf16"),  # same, kv heads
    (3, 13, 6, 64, "bf16"),     # ragged: odd rank count and token count
    (1, 5, 2, 64, "bf16"),      # one rank: a plain copy
    (8, 7, 8, 128, "f32"),      # eight ranks, one head each
    (64, 3, 64, 64, "bf16"),    # the largest rank count
])
def test_pack_unpack_bit_exact(P, s_l, H, d, dtype):
    print(f"case P={P} s_l={s_l} H={H} d={d} {dtype}", flush=True)
    host, dev = _rand_shards(P, s_l, H, d, dtype, seed=P * 1000 + s_l)
    for r in range(P):
        y = U.ulysses_pack(dev, r)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), OP.pack(host, r))
        # unpack a fresh head shard into copies of the shards
        fresh = np.random.default_rng(r).integers(0, 2**16, y.shape, dtype=np.uint64).astype(host[0].dtype)
        tgt = [t.clone() for t in dev]
        U.ulysses_unpack(to_dev(fresh, dtype), r, tgt)
        torch.cuda.synchronize()
        want = OP.unpack(fresh, r, host)
        for a, b in zip(tgt, want):
            np.testing.assert_array_equal(_bits(a), b)


def test_headline_size_pack_unpack_bit_exact():
    cfg = W.WORKLOADS["qwen_64k"]
    print("case qwen_64k pack/unpack rank 0", flush=True)
    for name in ("q", "k"):
        g, dev = gen_shards(cfg, name)
        host = W.shards_of(g, cfg.P)
        y = U.ulysses_pack(dev, 0)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(y), OP.pack(host, 0))
        back = [torch.zeros_like(t) for t in dev]
        U.ulysses_unpack(y, 0, back)
        torch.cuda.synchronize()
        Hl = g.shape[1] // cfg.P
        for a, b in zip(back, host):
            got = _bits(a)
            np.testing.assert_array_equal(got[:, :Hl], b[:, :Hl])
            assert not got[:, Hl:].any()


def test_upipe_size_pack_sampled_rows():
    """262144 tokens, 64 q heads, 8 ranks: 4 GiB of shards. Random bits; sampled rows vs the index map."""
    P, s_l, H, d = 8, 32768, 64, 128
    print("case upipe-size pack rank 3", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(0)
    dev = [torch.randint(-2**15, 2**15, (s_l, H, d), dtype=torch.int16, device="cuda", generator=gen)
           .view(torch.bfloat16) for _ in range(P)]
    r = 3
    y = U.ulysses_pack(dev, r)
    back = [torch.zeros_like(t) for t in dev]
    U.ulysses_unpack(y, r, back)
    torch.cuda.synchronize()
    Hl = H // P
    rows = np.unique(np.concatenate([np.arange(64), np.arange(P * s_l - 64, P * s_l),
                                     np.random.default_rng(0).integers(0, P * s_l, 512)]))
    ybits = _bits(y[torch.from_numpy(rows).cuda()])
    for i, row in enumerate(rows):
        p, t = divmod(int(row), s_l)
        np.testing.assert_array_equal(ybits[i], _bits(dev[p][t, r * Hl:(r + 1) * Hl]))
    for p in range(P):
        assert torch.equal(back[p][:, r * Hl:(r + 1) * Hl].view(torch.int16), dev[p][:, r * Hl:(r + 1) * Hl].view(torch.int16))
        assert not back[p][:, :r * Hl].view(torch.int16).any()


@pytest.mark.parametrize("P,s_l,Hs,d,dtype", [
    (4, 2048, (32, 8, 8), 128, "bf16"),   # Q, K, V of the 8K share
    (3, 13, (6, 3, 3), 64, "bf16"),       # ragged token count, odd rank count
    (2, 256, (4, 4), 64, "f32"),          # two tensors, fp32
    (8, 7, (8,), 128, "f32"),             # one tensor: the grouped call equals ulysses_pack
    (64, 3, (64, 64, 128), 64, "bf16"),   # the largest rank count, different head counts
])
def test_grouped_pack_unpack_bit_exact(P, s_l, Hs, d, dtype):
    """ulysses_pack_group / ulysses_unpack_group: every tensor bit-exact against the oracle's
    index-loop permute, for every rank; heads of other ranks untouched by the unpack."""
    print(f"case grouped P={P} s_l={s_l} H={Hs} d={d} {dtype}", flush=True)
    hosts, devs = zip(*[_rand_shards(P, s_l, H, d, dtype, seed=97 * i + P) for i, H in enumerate(Hs)])
    for r in range(P):
        ys = U.ulysses_pack_group(list(devs), r)
        torch.cuda.synchronize()
        for y, host in zip(ys, hosts):
            np.testing.assert_array_equal(_bits(y), OP.pack(host, r))
        fresh = [np.random.default_rng(r + 7 * i).integers(0, 2**16, y.shape, dtype=np.uint64).astype(hosts[i][0].dtype)
                 for i, y in enumerate(ys)]
        tgts = [[t.clone() for t in dev] for dev in devs]
        U.ulysses_unpack_group([to_dev(f, dtype) for f in fresh], r, tgts)
        torch.cuda.synchronize()
        for f, tgt, host in zip(fresh, tgts, hosts):
            for a, b in zip(tgt, OP.unpack(f, r, host)):
                np.testing.assert_array_equal(_bits(a), b)


def test_grouped_pack_headline_size_equals_single_calls():
    """Q, K, V of the 64K share packed by one launch: bit-identical to three ulysses_pack calls,
    and their unpack_group restores the rank's head slices."""
    cfg = W.WORKLOADS["qwen_64k"]
    print("case qwen_64k grouped pack/unpack rank 1", flush=True)
    devs = [gen_shards(cfg, name)[1] for name in ("q", "k", "v")]
    ys = U.ulysses_pack_group(devs, 1)
    singles = [U.ulysses_pack(dev, 1) for dev in devs]
    torch.cuda.synchronize()
    for y, ref in zip(ys, singles):
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    backs = [[torch.zeros_like(t) for t in dev] for dev in devs]
    U.ulysses_unpack_group(ys, 1, backs)
    torch.cuda.synchronize()
    for dev, back in zip(devs, backs):
        Hl = dev[0].shape[1] // cfg.P
        for a, b in zip(back, dev):
            assert torch.equal(a[:, Hl:2 * Hl].view(torch.int16), b[:, Hl:2 * Hl].view(torch.int16))
            assert not a[:, :Hl].view(torch.int16).any() and not a[:, 2 * Hl:].view(torch.int16).any()
