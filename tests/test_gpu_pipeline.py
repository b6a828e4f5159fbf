"""The whole share end to end on the GPU: pack Q/K/V -> attention forward -> unpack O;
pack dO -> attention backward -> unpack dQ/dK/dV, against the oracle run on the
unsharded global tensors (sharded-then-permuted must equal unsharded attention)."""
import dataclasses

import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from tests.helpers import LSE_ABS, compare, dev_to_f64, gen_shards

pytestmark = pytest.mark.gpu


def run_share(cfg, rank, shards, cu_dev):
    """One rank's forward and backward through the C ABI, as the bench runs them (bf16: with
    O's rounding residual handed from the forward to the backward); returns device outputs."""
    q = U.ulysses_pack(shards["q"], rank)
    k = U.ulysses_pack(shards["k"], rank)
    v = U.ulysses_pack(shards["v"], rank)
    o_lo = U.new_o_lo(q) if cfg.dtype == "bf16" else None
    o, lse = U.attn_fwd(q, k, v, cfg.scale, cfg.causal, cu_dev, o_lo=o_lo)
    o_sh = [torch.zeros_like(t) for t in shards["q"]]
    U.ulysses_unpack(o, rank, o_sh)
    do = U.ulysses_pack(shards["do"], rank)
    dq, dk, dv = U.attn_bwd(q, k, v, o, lse, do, cfg.scale, cfg.causal, cu_dev, o_lo=o_lo)
    dq_sh = [torch.zeros_like(t) for t in shards["q"]]
    dk_sh = [torch.zeros_like(t) for t in shards["k"]]
    dv_sh = [torch.zeros_like(t) for t in shards["v"]]
    U.ulysses_unpack(dq, rank, dq_sh)
    U.ulysses_unpack(dk, rank, dk_sh)
    U.ulysses_unpack(dv, rank, dv_sh)
    return dict(o=o_sh, lse=lse, dq=dq_sh, dk=dk_sh, dv=dv_sh)


def _cat_heads(sh, rank, P):
    x = torch.cat(sh, dim=0)
    Hl = x.shape[1] // P
    return dev_to_f64(x[:, rank * Hl:(rank + 1) * Hl])


# the tiny shape also in bf16, so that its size runs through the MFMA kernels
TINY_BF16 = dataclasses.replace(W.WORKLOADS["tiny_f32"], name="tiny_bf16", dtype="bf16")


@pytest.mark.parametrize("name,ranks", [("tiny_f32", (0, 1)), ("tiny_bf16", (0, 1)), ("qwen_8k", (0, 3))])
def test_share_matches_unsharded_oracle(name, ranks):
    cfg = TINY_BF16 if name == "tiny_bf16" else W.WORKLOADS[name]
    print(f"case {name} ranks {ranks}", flush=True)
    glob, shards = {}, {}
    for n in ("q", "k", "v", "do"):
        glob[n], shards[n] = gen_shards(cfg, n)
    f = {n: W.bits_to_f64(b, cfg.dtype) for n, b in glob.items()}
    for r in ranks:
        out = run_share(cfg, r, shards, None)
        torch.cuda.synchronize()
        sl = lambda a, H: a[:, r * (H // cfg.P):(r + 1) * (H // cfg.P)]
        q, k, v, do = sl(f["q"], cfg.Hq), sl(f["k"], cfg.Hkv), sl(f["v"], cfg.Hkv), sl(f["do"], cfg.Hq)
        wo, wl = OA.forward(q, k, v, cfg.scale, cfg.causal)
        wq, wk, wv = OA.backward(q, k, v, do, cfg.scale, cfg.causal)
        compare(f"{name} r{r} O", _cat_heads(out["o"], r, cfg.P), wo, bf16=(cfg.dtype == "bf16"))
        compare(f"{name} r{r} LSE", out["lse"].cpu().numpy(), wl, max_abs=LSE_ABS, rel_fro=1e-4)
        compare(f"{name} r{r} dQ", _cat_heads(out["dq"], r, cfg.P), wq, bf16=(cfg.dtype == "bf16"))
        compare(f"{name} r{r} dK", _cat_heads(out["dk"], r, cfg.P), wk, bf16=(cfg.dtype == "bf16"))
        compare(f"{name} r{r} dV", _cat_heads(out["dv"], r, cfg.P), wv, bf16=(cfg.dtype == "bf16"))
        # heads of other ranks are untouched by this rank's unpack
        Hl = cfg.Hq // cfg.P
        for t in out["o"]:
            rest = torch.cat([t[:, :r * Hl], t[:, (r + 1) * Hl:]], dim=1)
            assert not rest.float().abs().sum().item()
