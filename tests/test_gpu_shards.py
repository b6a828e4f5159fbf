"""GPU parity of attn_fwd_shards / attn_bwd_shards: forward and backward reading the rank's
heads straight from the sequence shards and writing O (dQ, dK, dV) straight into the rank's
head slice of the output shards.

They run the same per-row arithmetic as ulysses_pack -> attn_fwd / attn_bwd ->
ulysses_unpack, only with other addresses, so every output must be bitwise equal to that
path; heads of other ranks in the output shards must be left untouched; and the results
are held to the oracle on the unsharded tensors at small sizes."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from tests.helpers import LSE_ABS, compare, dev_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _packed_path(dev, rank, scale, causal, cu_dev, with_lo=False, split=False):
    q, k, v = (U.ulysses_pack(dev[n], rank) for n in ("q", "k", "v"))
    o_lo = U.new_o_lo(q) if with_lo else None
    # split or not as the shard-reading forward it is compared with, bitwise
    o, lse = U.attn_fwd(q, k, v, scale, causal, cu_dev, o_lo=o_lo, split=split)
    o_sh = [torch.full_like(t, 3.0) for t in dev["q"]]
    U.ulysses_unpack(o, rank, o_sh)
    return (o_sh, lse, o_lo) if with_lo else (o_sh, lse)


CASES = [
    # P, s_l, Hq, Hkv, d, rank, causal, cu
    (4, 256, 32, 8, 128, 1, True, None),
    (2, 384, 8, 2, 64, 0, True, [0, 100, 101, 500, 768]),
    (8, 128, 64, 8, 128, 7, True, None),
    (4, 128, 8, 4, 128, 2, False, None),
    (2, 128, 4, 4, 128, 1, True, [0, 1, 255, 256]),
    (2, 256, 8, 2, 128, 0, False, [0, 128, 300, 512]),
]


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("P,s_l,Hq,Hkv,d,rank,causal,cu", CASES)
def test_shards_equal_packed_path(P, s_l, Hq, Hkv, d, rank, causal, cu, split):
    """These grids are short: with split=True both sides split their keys over several
    workgroups (the same counts) and must still agree bitwise."""
    print(f"case P={P} s_l={s_l} Hq={Hq} Hkv={Hkv} d={d} rank={rank} causal={causal} cu={cu is not None} "
          f"split={split}", flush=True)
    assert U.attn_fwd_workspace_bytes(P * s_l, Hq // P, d) > 0
    cfg = W.Config("shards_small", P=P, s_l=s_l, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", causal=causal)
    bits = {n: W.gen_global(cfg, n, seed=21) for n in ("q", "k", "v")}
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(bits[n], P)] for n in bits}
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    want_o, want_lse, want_lo = _packed_path(dev, rank, cfg.scale, causal, cu_dev, True, split)
    o_sh = [torch.full_like(t, 3.0) for t in dev["q"]]
    keep = [t.clone() for t in o_sh]
    o_lo = torch.full_like(want_lo, 5.0)
    lse = U.attn_fwd_shards(dev["q"], dev["k"], dev["v"], o_sh, rank, cfg.scale, causal, cu_dev, o_lo=o_lo,
                            split=split)
    torch.cuda.synchronize()
    assert torch.equal(o_lo.view(torch.int16), want_lo.view(torch.int16))
    Hl = Hq // P
    sl = slice(rank * Hl, (rank + 1) * Hl)
    for a, b, c in zip(o_sh, want_o, keep):
        assert torch.equal(a[:, sl].view(torch.int16), b[:, sl].view(torch.int16))
        assert torch.equal(torch.cat([a[:, :rank * Hl], a[:, (rank + 1) * Hl:]], 1),
                           torch.cat([c[:, :rank * Hl], c[:, (rank + 1) * Hl:]], 1))
    assert torch.equal(lse, want_lse)
    # and against the oracle on the unsharded head slice
    f = {n: W.bits_to_f64(W.head_slice(bits[n], P, rank), "bf16") for n in bits}
    wo, wl = OA.forward(f["q"], f["k"], f["v"], cfg.scale, causal, cu)
    compare("shards O", dev_to_f64(torch.cat(o_sh, 0)[:, sl]), wo, bf16=True)
    compare("shards LSE", lse.cpu().numpy(), wl, max_abs=LSE_ABS, rel_fro=1e-4)


def _packed_bwd(dev, o_sh, lse, rank, scale, causal, cu_dev, o_lo=None, split=False):
    q, k, v, o, g = (U.ulysses_pack(x, rank) for x in (dev["q"], dev["k"], dev["v"], o_sh, dev["do"]))
    dq, dk, dv = U.attn_bwd(q, k, v, o, lse, g, scale, causal, cu_dev, o_lo=o_lo, split=split)
    out = {}
    for n, y, like in (("dq", dq, dev["q"]), ("dk", dk, dev["k"]), ("dv", dv, dev["v"])):
        out[n] = [torch.full_like(t, 3.0) for t in like]
        U.ulysses_unpack(y, rank, out[n])
    return out


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("P,s_l,Hq,Hkv,d,rank,causal,cu", CASES)
def test_bwd_shards_equal_packed_path(P, s_l, Hq, Hkv, d, rank, causal, cu, split):
    """As the forward: unsplit, and with dK/dV and dQ split on both sides."""
    print(f"case P={P} s_l={s_l} Hq={Hq} Hkv={Hkv} d={d} rank={rank} causal={causal} cu={cu is not None} "
          f"split={split}", flush=True)
    cfg = W.Config("shards_bwd", P=P, s_l=s_l, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", causal=causal)
    bits = {n: W.gen_global(cfg, n, seed=23) for n in ("q", "k", "v", "do")}
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(bits[n], P)] for n in bits}
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    o_sh, lse, o_lo = _packed_path(dev, rank, cfg.scale, causal, cu_dev, True)
    want = _packed_bwd(dev, o_sh, lse, rank, cfg.scale, causal, cu_dev, o_lo, split)
    got = {n: [torch.full_like(t, 3.0) for t in want[n]] for n in want}
    U.attn_bwd_shards(dev["q"], dev["k"], dev["v"], o_sh, lse, dev["do"], got["dq"], got["dk"], got["dv"], rank,
                      cfg.scale, causal, cu_dev, o_lo=o_lo, split=split)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv"):
        for a, b in zip(got[n], want[n]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
    f = {n: W.bits_to_f64(W.head_slice(bits[n], P, rank), "bf16") for n in bits}
    wq, wk, wv = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, causal, cu)
    for n, w, H in (("dq", wq, Hq), ("dk", wk, Hkv), ("dv", wv, Hkv)):
        Hl = H // P
        compare(f"shards {n}", dev_to_f64(torch.cat(got[n], 0)[:, rank * Hl:(rank + 1) * Hl]), w, bf16=True)


def test_bwd_shards_workspace():
    """A delta workspace one byte short is rejected before any launch."""
    cfg = W.Config("shards_ws", P=2, s_l=128, Hq=4, Hkv=2, d=128, dtype="bf16")
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(W.gen_global(cfg, n, seed=4), cfg.P)]
           for n in ("q", "k", "v", "do")}
    o_sh, lse = _packed_path(dev, 1, cfg.scale, True, None)
    outs = [[torch.zeros_like(t) for t in dev[n]] for n in ("q", "k", "v")]
    need = U.delta_bytes(cfg.s, cfg.Hq_l)
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(U.UlyssesError):
        U.attn_bwd_shards(dev["q"], dev["k"], dev["v"], o_sh, lse, dev["do"], *outs, 1, workspace=short)
    torch.cuda.synchronize()
    assert all(not t.float().abs().sum().item() for x in outs for t in x)


def test_shards_rejects_unsupported():
    """s_l not a multiple of 128 and fp32 are refused before any launch."""
    cfg = W.Config("shards_bad", P=2, s_l=96, Hq=4, Hkv=2, d=128, dtype="bf16")
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(W.gen_global(cfg, n, seed=3), cfg.P)] for n in ("q", "k", "v")}
    o_sh = [torch.zeros_like(t) for t in dev["q"]]
    with pytest.raises(U.UlyssesError):
        U.attn_fwd_shards(dev["q"], dev["k"], dev["v"], o_sh, 0)
    cfg = W.Config("shards_f32", P=2, s_l=128, Hq=4, Hkv=2, d=64, dtype="f32")
    dev = {n: [to_dev(b, "f32") for b in W.shards_of(W.gen_global(cfg, n, seed=3), cfg.P)] for n in ("q", "k", "v")}
    o_sh = [torch.zeros_like(t) for t in dev["q"]]
    with pytest.raises(U.UlyssesError):
        U.attn_fwd_shards(dev["q"], dev["k"], dev["v"], o_sh, 0)
    torch.cuda.synchronize()
    assert all(not t.abs().sum().item() for t in o_sh)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("rank", [0, 3])
def test_shards_qwen_64k_share(rank):
    """The 64K headline share (4 shards of 16384 tokens, 32 q / 8 kv heads): bitwise equal
    to the packed path for ranks 0 and 3."""
    cfg = W.WORKLOADS["qwen_64k"]
    print(f"generating qwen_64k shards for rank {rank}", flush=True)
    dev = {n: [to_dev(W.gen_rows(cfg, n, p * cfg.s_l, (p + 1) * cfg.s_l), "bf16") for p in range(cfg.P)]
           for n in ("q", "k", "v")}
    want_o, want_lse = _packed_path(dev, rank, cfg.scale, True, None)
    o_sh = [torch.full_like(t, 3.0) for t in dev["q"]]
    lse = U.attn_fwd_shards(dev["q"], dev["k"], dev["v"], o_sh, rank, cfg.scale, True)
    torch.cuda.synchronize()
    Hl = cfg.Hq_l
    for a, b in zip(o_sh, want_o):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(lse, want_lse)


@pytest.mark.timeout(300)
def test_bwd_shards_qwen_64k_share():
    """Backward of the 64K headline share (rank 2): bitwise equal to the packed path."""
    cfg = W.WORKLOADS["qwen_64k"]
    rank = 2
    print("generating qwen_64k shards", flush=True)
    dev = {n: [to_dev(W.gen_rows(cfg, n, p * cfg.s_l, (p + 1) * cfg.s_l), "bf16") for p in range(cfg.P)]
           for n in ("q", "k", "v", "do")}
    o_sh, lse, o_lo = _packed_path(dev, rank, cfg.scale, True, None, True)
    want = _packed_bwd(dev, o_sh, lse, rank, cfg.scale, True, None, o_lo)
    got = {n: [torch.full_like(t, 3.0) for t in want[n]] for n in want}
    U.attn_bwd_shards(dev["q"], dev["k"], dev["v"], o_sh, lse, dev["do"], got["dq"], got["dk"], got["dv"], rank,
                      cfg.scale, True, o_lo=o_lo)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv"):
        for a, b in zip(got[n], want[n]):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
