"""Parity at the full size of the 64K headline share and of the packed 96K share (rank 0),
and of a one-rank share of a million-token sequence, through the same calls and launch
configuration the bench times.

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
taken over the summed elements, which a lost or doubled tile or head would exceed.
Likewise rows of dS sum to zero (sum_j P_ij (dP_ij - delta_i) = delta_i - delta_i), so per kv
head (and per document) sum_j dK_j = 0; the bf16 roundings of dS and of the stored dK leave
a noise whose size an fp64 emulation of that rounding puts at 0.6 (mean) to 2.2 (max over
columns) times 2^-8 ||dK||_2 per column, and the test allows 8 * 2^-8 ||dK||_2.
Finally the keys with the longest accumulations (key 0 sums every row of every q head of
its group) are checked exactly at 64K: dK and dV of keys 0, 1, 63, 64, 127, 128, s/2 and
s/2 + 1 of kv head 0 against the oracle."""
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


def _dk_column_sums(dk, segments):
    """Check sum_j dK_j = 0 per kv head over each segment [a, b)."""
    for a, b in segments:
        for g in range(dk.shape[1]):
            lhs = np.abs(dk[a:b, g].sum(0))
            tol = 8 * 2.0 ** -8 * np.sqrt((dk[a:b, g] ** 2).sum(0))
            assert (lhs <= tol).all(), f"dK column sum [{a},{b}) g={g}: |sum| {lhs.max():.3e} tol {tol.min():.3e}"


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
    _dk_column_sums(_rank_heads(out["dk"], rank, cfg.P, np.arange(cfg.s)), segments)
    return out, f


@pytest.mark.timeout(600)
def test_qwen_64k_share():
    cfg = W.WORKLOADS["qwen_64k"]
    s = cfg.s
    keys = set(range(s - 64, s))
    for b in range(s - 1024, s, 128):
        keys |= {b - 1, b}
    _run(cfg, 0, (), np.array(sorted(keys)), [(0, s)])


@pytest.mark.timeout(900)
def test_million_token_share():
    """One rank's share of a 1,048,576-token sequence, the context length in the title of the
    first page: 8 ranks of 131072 tokens, 16 q / 8 kv heads, so 2 q / 1 kv heads per rank after
    the exchange. The checks of the 64K share at sixteen times its length: sampled rows of O,
    LSE and dQ, the last keys' dK and dV, and the column sums of dV and dK over all 2^20
    keys."""
    cfg = W.WORKLOADS["million"]
    s = cfg.s
    keys = set(range(s - 64, s))
    for b in range(s - 512, s, 128):
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


def _oracle_head_keys(f, h, g, scale, keys):
    """dK, dV of `keys` of kv head g from q head h alone (the oracle; numpy releases the GIL
    in its large kernels, so heads run in threads)."""
    sl = lambda a, i: a[:, i:i + 1]
    _, dk, dv = OA.backward(sl(f["q"], h), sl(f["k"], g), sl(f["v"], g), sl(f["do"], h), scale, True, None,
                            q_rows=np.zeros(0, int), kv_cols=keys)
    print(f"  oracle: q head {h} done", flush=True)
    return dk[:, 0], dv[:, 0]


@pytest.mark.timeout(900)
def test_qwen_64k_early_keys_exact():
    """The keys with the most rows: dK and dV of kv head 0 at keys 0, 1, 63, 64, 127, 128, s/2,
    s/2 + 1 against the oracle, whose forward pass covers the whole 64K causal sequence for
    each of the group's q heads (the GQA sum of per-head gradients)."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = W.WORKLOADS["qwen_64k"]
    s = cfg.s
    keys = np.array([0, 1, 63, 64, 127, 128, s // 2, s // 2 + 1])
    print("case qwen_64k early keys: generating", flush=True)
    shards, f = _inputs(cfg, 0)
    out = run_share(cfg, 0, shards, None)
    torch.cuda.synchronize()
    got_k = _rank_heads(out["dk"], 0, cfg.P, keys)[:, 0]
    got_v = _rank_heads(out["dv"], 0, cfg.P, keys)[:, 0]
    del out, shards
    print("  GPU share done; oracle over the 4 q heads of kv head 0", flush=True)
    with ThreadPoolExecutor(cfg.G) as ex:
        parts = list(ex.map(lambda h: _oracle_head_keys(f, h, 0, cfg.scale, keys), range(cfg.G)))
    wk = sum(p[0] for p in parts)
    wv = sum(p[1] for p in parts)
    compare("64K early keys dK", got_k, wk, bf16=True)
    compare("64K early keys dV", got_v, wv, bf16=True)


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
    o_lo = U.new_o_lo(q)
    for _ in range(3):
        o, lse = U.attn_fwd(q, k, v, cfg.scale, True, o_lo=o_lo)
        dq, dk, dv = U.attn_bwd(q, k, v, o, lse, do, cfg.scale, True, o_lo=o_lo)
        torch.cuda.synchronize()
        runs.append((o.view(torch.int16).clone(), lse.clone(), dq.view(torch.int16).clone(),
                     dk.view(torch.int16).clone(), dv.view(torch.int16).clone()))
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(a, b)
