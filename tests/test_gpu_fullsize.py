"""Parity at the full size of the 64K headline share and of the packed 96K share (rank 0),
through the same calls and launch configuration the bench times.

The oracle cannot afford every element at these sizes, so it checks what it can compute
exactly one by one:
  * O, LSE and dQ on sampled rows -- each is a function of its own row: rows 0-63, both
    sides of tile boundaries at a stride, the last 64, and (packed) both sides of every
    document boundary;
  * dK and dV on keys whose attending rows are few: the last keys of the sequence, keys
    at tile boundaries of its last 1024 tokens, and (packed) the last keys of every
    document and the two shortest documents whole;
and, over every key, a property that holds at any size: rows of softmax weights sum to
one, so per kv head g (and per document) sum_j dV_j equals the sum over the group's q
heads of sum_i dO_i. On the GPU the bf16 rounding of P (relative 2^-8 per weight) and
of the stored dV (2^-8 per element) perturb both sides by independent roundings; the
test allows more than 8 standard deviations of that noise, 8 * 2^-8 * (||dV||_2 + ||dO||_2)
taken over the summed elements, which a lost or doubled tile or head would exceed."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from tests.helpers import LSE_ABS, compare, dev_to_f64, sample_rows, to_dev
from tests.test_gpu_pipeline import run_share

pytestmark = pytest.mark.gpu


def _inputs(cfg, rank):
    """Device shards of every rank and float64 head slices of rank `rank`."""
    shards, f = {}, {}
    for n in ("q", "k", "v", "do"):
        Hl = (cfg.Hq if n in ("q", "do") else cfg.Hkv) // cfg.P
        parts, sl = [], []
        for p in range(cfg.P):
            b = W.gen_rows(cfg, n, p * cfg.s_l, (p + 1) * cfg.s_l)
            parts.append(to_dev(b, cfg.dtype))
            sl.append(W.bits_to_f64(b[:, rank * Hl:(rank + 1) * Hl], cfg.dtype))
        shards[n], f[n] = parts, np.concatenate(sl, 0)
    return shards, f


def _rank_heads(sh, rank, P, idx):
    """Rows `idx` of this rank's heads, gathered from the P output shards, as float64."""
    x = torch.cat(sh, dim=0)
    Hl = x.shape[1] // P
    return dev_to_f64(x[torch.as_tensor(idx, device=x.device), rank * Hl:(rank + 1) * Hl])


def _dv_column_sums(dv, do, G, segments):
    """Check sum_j dV_j = sum_{h in g} sum_i dO_i over each segment [a, b)."""
    for a, b in segments:
        for g in range(dv.shape[1]):
            lhs = dv[a:b, g].sum(0)
            grp = do[a:b, g * G:(g + 1) * G]
            rhs = grp.sum((0, 1))
            tol = 8 * 2.0 ** -8 * (np.sqrt((dv[a:b, g] ** 2).sum(0)) + np.sqrt((grp ** 2).sum((0, 1))))
            err = np.abs(lhs - rhs)
            assert (err <= tol).all(), f"dV column sum [{a},{b}) g={g}: err {err.max():.3e} tol {tol.min():.3e}"


def _run(cfg, rank, extra_rows, keys, segments):
    print(f"case {cfg.name} rank {rank}: generating", flush=True)
    shards, f = _inputs(cfg, rank)
    cu = W.cu_seqlens_for(cfg)
    cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
    out = run_share(cfg, rank, shards, cu_dev)
    torch.cuda.synchronize()
    print("  GPU share done", flush=True)
    rows = sample_rows(cfg.s, extra=extra_rows)
    wo, wl = OA.forward(f["q"], f["k"], f["v"], cfg.scale, cfg.causal, cu, rows=rows)
    compare(f"{cfg.name} O rows", _rank_heads(out["o"], rank, cfg.P, rows), wo, bf16=True)
    compare(f"{cfg.name} LSE rows", out["lse"][:, torch.as_tensor(rows, device="cuda")].cpu().numpy(), wl,
            max_abs=LSE_ABS, rel_fro=1e-4)
    wq, _, _ = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, cfg.causal, cu, q_rows=rows, kv_cols=np.zeros(0, int))
    compare(f"{cfg.name} dQ rows", _rank_heads(out["dq"], rank, cfg.P, rows), wq, bf16=True)
    print("  sampled rows ok", flush=True)
    _, wk, wv = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, cfg.causal, cu, q_rows=np.zeros(0, int), kv_cols=keys)
    compare(f"{cfg.name} dK keys", _rank_heads(out["dk"], rank, cfg.P, keys), wk, bf16=True)
    compare(f"{cfg.name} dV keys", _rank_heads(out["dv"], rank, cfg.P, keys), wv, bf16=True)
    print("  sampled keys ok", flush=True)
    dv = _rank_heads(out["dv"], rank, cfg.P, np.arange(cfg.s))
    _dv_column_sums(dv, f["do"], cfg.G, segments)


@pytest.mark.timeout(600)
def test_qwen_64k_share():
    cfg = W.WORKLOADS["qwen_64k"]
    s = cfg.s
    keys = set(range(s - 64, s))
    for b in range(s - 1024, s, 128):
        keys |= {b - 1, b}
    _run(cfg, 0, (), np.array(sorted(keys)), [(0, s)])


@pytest.mark.timeout(600)
def test_packed_96k_share():
    cfg = W.WORKLOADS["packed_96k"]
    cu = [int(x) for x in W.cu_seqlens_for(cfg)]
    extra = {r for c in cu[1:-1] for r in (c - 1, c, c + 1)}
    keys = set()
    for a, b in zip(cu[:-1], cu[1:]):
        keys |= set(range(max(a, b - 64), b))
        if b - a <= 200:
            keys |= set(range(a, b))
    _run(cfg, 0, extra, np.array(sorted(keys)), list(zip(cu[:-1], cu[1:])))


@pytest.mark.timeout(300)
def test_qwen_64k_deterministic():
    """The 64K share's forward and backward, run three times on the same inputs, give the
    same bits every time (no atomics; every LDS tile published by a barrier after its DMA
    landed). The race this guards against showed at this size and not at small ones."""
    cfg = W.WORKLOADS["qwen_64k"]
    gen = torch.Generator(device="cuda").manual_seed(5)
    mk = lambda H: torch.randn((cfg.s, H, cfg.d), device="cuda", generator=gen).to(torch.bfloat16)
    q, k, v, do = mk(cfg.Hq_l), mk(cfg.Hkv_l), mk(cfg.Hkv_l), mk(cfg.Hq_l)
    runs = []
    for _ in range(3):
        o, lse = U.attn_fwd(q, k, v, cfg.scale, True)
        dq, dk, dv = U.attn_bwd(q, k, v, o, lse, do, cfg.scale, True)
        torch.cuda.synchronize()
        runs.append((o.view(torch.int16).clone(), lse.clone(), dq.view(torch.int16).clone(),
                     dk.view(torch.int16).clone(), dv.view(torch.int16).clone()))
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
