"""GPU parity of Ring Attention (ring_attn_fwd / ring_attn_bwd), the pages' comparison
workload: every rank's forward (per-hop attention on the existing kernels, LSE merge in fp32)
and the backward run in rank order (dQ summed over hops, dK/dV sums travelling with the K/V
blocks) against the oracle on the unsharded tensors, which the ring oracle equals; and the
whole ring bitwise reproducible."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from tests.helpers import LSE_ABS, compare, dev_to_f64, to_dev

pytestmark = pytest.mark.gpu


def _run_ring(dev, P, causal, scale):
    s_l, Hq, d = dev["q"][0].shape
    Hkv = dev["k"][0].shape[1]
    outs = []
    for r in range(P):
        o_lo = torch.empty((s_l, Hq, d), dtype=torch.bfloat16, device="cuda")
        o, lse = U.ring_attn_fwd(dev["q"], dev["k"], dev["v"], r, scale, causal, o_lo=o_lo)
        outs.append((o, lse, o_lo))
    dk_acc = torch.full((P, s_l, Hkv, d), 123.0, dtype=torch.float32, device="cuda")   # no zeroing needed
    dv_acc = torch.full_like(dk_acc, -7.0)
    dk = [torch.full_like(t, 3.0) for t in dev["k"]]
    dv = [torch.full_like(t, 3.0) for t in dev["v"]]
    dqs = []
    for r in range(P):
        o, lse, o_lo = outs[r]
        dqs.append(U.ring_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"][r], r, dk_acc, dv_acc, dk, dv,
                                   scale, causal, o_lo=o_lo))
    torch.cuda.synchronize()
    return outs, dqs, dk, dv


@pytest.mark.parametrize("P,s_l,Hq,Hkv,d,causal", [
    (4, 200, 8, 2, 128, True), (3, 130, 4, 4, 64, False), (2, 256, 8, 1, 128, True), (1, 100, 2, 1, 128, True),
    (8, 64, 4, 2, 128, True),
])
def test_ring_matches_unsharded_oracle(P, s_l, Hq, Hkv, d, causal):
    print(f"case ring P={P} s_l={s_l} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
    cfg = W.Config("ring", P=P, s_l=s_l, Hq=Hq, Hkv=Hkv, d=d, dtype="bf16", causal=causal)
    glob = {n: W.gen_global(cfg, n, seed=17) for n in ("q", "k", "v", "do")}
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(g, P)] for n, g in glob.items()}
    outs, dqs, dk, dv = _run_ring(dev, P, causal, cfg.scale)
    f = {n: W.bits_to_f64(g, "bf16") for n, g in glob.items()}
    wo, wl = OA.forward(f["q"], f["k"], f["v"], cfg.scale, causal)
    wq, wk, wv = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, causal)
    compare("ring O", dev_to_f64(torch.cat([o for o, _, _ in outs])), wo, bf16=True)
    compare("ring LSE", torch.cat([l for _, l, _ in outs], dim=1).cpu().numpy(), wl, max_abs=LSE_ABS, rel_fro=1e-4)
    compare("ring dQ", dev_to_f64(torch.cat(dqs)), wq, bf16=True)
    compare("ring dK", dev_to_f64(torch.cat(dk)), wk, bf16=True)
    compare("ring dV", dev_to_f64(torch.cat(dv)), wv, bf16=True)


def test_ring_deterministic():
    cfg = W.Config("ring_det", P=4, s_l=192, Hq=8, Hkv=2, d=128, dtype="bf16")
    dev = {n: [to_dev(b, "bf16") for b in W.shards_of(W.gen_global(cfg, n, seed=2), cfg.P)]
           for n in ("q", "k", "v", "do")}
    runs = []
    for _ in range(2):
        outs, dqs, dk, dv = _run_ring(dev, cfg.P, True, cfg.scale)
        runs.append([t.clone() for t in [x for o in outs for x in o] + dqs + dk + dv])
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
