"""GPU parity of the headwise-chunked (UPipe) forward, attn_fwd_chunked.

Chunking changes only which heads are resident at once, so on the GPU every chunk runs
the same kernels on the same rows as the unchunked pack -> attn_fwd -> unpack: the
outputs must be bitwise equal to it, and both are held to the oracle (the chunked
oracle at small sizes; sampled rows at the full 256K share). Heads of other ranks in
the output shards must be left untouched."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from oracle import chunked as OC
from tests.helpers import LSE_ABS, compare, dev_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _unchunked(qs, ks, vs, rank, scale, causal, cu_dev):
    q, k, v = (U.ulysses_pack(x, rank) for x in (qs, ks, vs))
    o, lse = U.attn_fwd(q, k, v, scale, causal, cu_dev)
    o_sh = [torch.zeros_like(t) for t in qs]
    U.ulysses_unpack(o, rank, o_sh)
    return o_sh, lse


def _sentinel_like(shards):
    """Output shards pre-filled with a recognisable pattern (not zeros)."""
    return [torch.full_like(t, 3.0) for t in shards]


def _check_rank_heads(got, want, untouched, rank, Hl):
    for a, b, c in zip(got, want, untouched):
        sl = slice(rank * Hl, (rank + 1) * Hl)
        assert torch.equal(a[:, sl].view(torch.int16), b[:, sl].view(torch.int16))
        rest = torch.cat([a[:, :rank * Hl], a[:, (rank + 1) * Hl:]], dim=1)
        rest_c = torch.cat([c[:, :rank * Hl], c[:, (rank + 1) * Hl:]], dim=1)
        assert torch.equal(rest, rest_c)


SMALL = [
    # P, s_l, Hq, Hkv, u, rank, cu
    (4, 300, 24, 8, 1, 0, None),
    (4, 300, 24, 8, 2, 3, None),
    (4, 300, 24, 8, 4, 1, None),        # u does not divide H_q/P = 6: last chunk has 2 heads
    (4, 300, 24, 8, 6, 2, None),        # one chunk = unchunked
    (4, 300, 24, 8, 9, 0, None),        # u beyond H_q/P is clamped to one chunk
    (2, 257, 8, 2, 3, 1, [0, 1, 40, 300, 514]),
    (8, 64, 64, 8, 2, 5, None),         # the UPipe head counts (8 q / 1 kv per rank) at small s
]


@pytest.mark.parametrize("P,s_l,Hq,Hkv,u,rank,cu", SMALL)
def test_chunked_small(P, s_l, Hq, Hkv, u, rank, cu):
    print(f"case P={P} s_l={s_l} Hq={Hq} Hkv={Hkv} u={u} rank={rank} cu={cu is not None}", flush=True)
    cfg = W.Config("chunk_small", P=P, s_l=s_l, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16")
    bits = {n: W.shards_of(W.gen_global(cfg, n, seed=11), P) for n in ("q", "k", "v")}
    dev = {n: [to_dev(b, "bf16") for b in bits[n]] for n in bits}
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    want_o, want_lse = _unchunked(dev["q"], dev["k"], dev["v"], rank, cfg.scale, True, cu_dev)
    o_sh = _sentinel_like(dev["q"])
    keep = [t.clone() for t in o_sh]
    lse = U.attn_fwd_chunked(dev["q"], dev["k"], dev["v"], o_sh, rank, u, cfg.scale, True, cu_dev)
    torch.cuda.synchronize()
    Hl = Hq // P
    _check_rank_heads(o_sh, want_o, keep, rank, Hl)
    assert torch.equal(lse, want_lse)

    to64 = lambda b: W.bits_to_f64(b, "bf16")
    zeros = [np.zeros(b.shape) for b in bits["q"]]
    oo, ol = OC.forward(bits["q"], bits["k"], bits["v"], zeros, rank, u, cfg.scale, True, cu,
                        to_f64=to64, from_f64=lambda x: x)
    got = torch.cat(o_sh, 0)[:, rank * Hl:(rank + 1) * Hl]
    want = np.concatenate(oo, 0)[:, rank * Hl:(rank + 1) * Hl]
    compare("chunked O", dev_to_f64(got), want, bf16=True)
    compare("chunked LSE", lse.cpu().numpy(), ol, max_abs=LSE_ABS, rel_fro=1e-4)


def test_chunked_workspace_matches_query():
    """A workspace one byte short is rejected before any launch; the exact size works."""
    cfg = W.Config("chunk_ws", P=4, s_l=64, Hq=16, Hkv=4, d=128, dtype="bf16")
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(W.gen_global(cfg, n, seed=2), cfg.P)]
           for n in ("q", "k", "v")}
    need = U.attn_fwd_chunked_workspace_bytes(cfg.P, cfg.s_l, cfg.Hq, cfg.Hkv, cfg.d, torch.bfloat16, 2)
    o_sh = [torch.zeros_like(t) for t in dev["q"]]
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(U.UlyssesError):
        U.attn_fwd_chunked(dev["q"], dev["k"], dev["v"], o_sh, 0, 2, workspace=short)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    U.attn_fwd_chunked(dev["q"], dev["k"], dev["v"], o_sh, 0, 2, workspace=ws)
    torch.cuda.synchronize()
    assert o_sh[0][:, :4].float().abs().sum().item() > 0


@pytest.mark.timeout(600)
def test_chunked_full_upipe_share():
    """The 256K UPipe share (8 ranks x 32768 tokens, 64 q / 8 kv heads, rank 0) at u = 1
    and u = 2: bitwise equal to the unchunked path, sampled rows of two heads against
    the oracle, and the workspace (peak intermediate bytes) as the analysis predicts."""
    cfg = W.CONFIGS["upipe_256k"]
    rank, P, s_l, Hl = 0, cfg.P, cfg.s_l, cfg.Hq_l
    heads = (0, Hl - 1)            # local q heads checked against the oracle (both read kv head 0)
    print("generating upipe_256k inputs", flush=True)
    dev, f = {n: [] for n in ("q", "k", "v")}, {}
    qh = np.zeros((cfg.s, len(heads), cfg.d))
    kh = np.zeros((cfg.s, 1, cfg.d))
    vh = np.zeros((cfg.s, 1, cfg.d))
    for p in range(P):
        r0, r1 = p * s_l, (p + 1) * s_l
        for n in ("q", "k", "v"):
            b = W.gen_rows(cfg, n, r0, r1)
            dev[n].append(to_dev(b, "bf16"))
            if n == "q":
                qh[r0:r1] = W.bits_to_f64(b[:, [rank * Hl + h for h in heads]], "bf16")
            else:
                (kh if n == "k" else vh)[r0:r1] = W.bits_to_f64(b[:, rank * cfg.Hkv_l:rank * cfg.Hkv_l + 1], "bf16")
        print(f"  shard {p} on device", flush=True)
    want_o, want_lse = _unchunked(dev["q"], dev["k"], dev["v"], rank, cfg.scale, True, None)
    torch.cuda.synchronize()
    print("unchunked done", flush=True)
    for u in (1, 2):
        need = U.attn_fwd_chunked_workspace_bytes(P, s_l, cfg.Hq, cfg.Hkv, cfg.d, torch.bfloat16, u)
        assert need == {1: 256, 2: 384}[u] * 2 ** 20
        o_sh = _sentinel_like(dev["q"])
        keep = [t.clone() for t in o_sh]
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        lse = U.attn_fwd_chunked(dev["q"], dev["k"], dev["v"], o_sh, rank, u, cfg.scale, True)
        torch.cuda.synchronize()
        # peak intermediate memory: the workspace plus the LSE output, nothing else
        peak = torch.cuda.max_memory_allocated() - base
        assert peak <= need + lse.numel() * 4 + (1 << 20), (u, peak, need)
        _check_rank_heads(o_sh, want_o, keep, rank, Hl)
        assert torch.equal(lse, want_lse)
        del keep, o_sh
        print(f"u={u} bitwise equal to unchunked", flush=True)

    rows = sample_rows(cfg.s)
    wo, wl = OA.forward(qh, kh, vh, cfg.scale, True, None, rows=rows)
    got = torch.stack([torch.stack([t[:, rank * Hl + h] for h in heads], 1) for t in want_o], 0)
    got = got.reshape(cfg.s, len(heads), cfg.d)[torch.as_tensor(rows, device="cuda")]
    compare("upipe O sampled", dev_to_f64(got), wo, bf16=True)
    compare("upipe LSE sampled", want_lse[list(heads)][:, torch.as_tensor(rows, device="cuda")].cpu().numpy(),
            wl, max_abs=LSE_ABS, rel_fro=1e-4)
