#!/usr/bin/env python3
"""Benchmark one GPU's share of a Ulysses sequence-parallel attention layer on MI355X.

One step = the whole hot path for one rank over one batch of synthetic input:
  pack Q, K, V (sequence shards -> head shard) -> attention forward -> unpack O
  -> pack dO -> attention backward (delta, dK/dV, dQ) -> unpack dQ, dK, dV.
Default workload: the 64K-token Qwen3-4B-shaped SP=4 share (4 shards of 16384 tokens,
32 q / 8 kv heads -> 8 q / 2 kv heads after the exchange, head dim 128, bf16, causal).

Metric: causal attention TFLOP/s, fwd+bwd counted FLOPs (4 d N fwd + 10 d N bwd per q
head, N = s^2/2 visible pairs, or sum of l^2/2 over packed documents) divided by the
time of the whole step (permutes included). Prints ONE JSON line.

The UPipe workload (--workload upipe_256k) times the headwise-chunked schedule instead:
attn_fwd_chunked then attn_bwd_chunked (--forward-only: the forward alone) with
--heads-per-chunk q heads per chunk, and reports the workspace bytes beside the unchunked
intermediates; --unchunked runs the same share without chunking (every local head packed,
attended and unpacked at once) for comparison. `memory` gives the intermediates' device bytes
as torch's allocator counts them and the peak the library's calls added (none: they never
allocate).

--forward-only times the forward half alone (pack Q/K/V, forward, unpack O); --fused
replaces the permutes and head-shard buffers by attn_fwd_shards / attn_bwd_shards, which
read and write the sequence shards directly.

The forward writes O's bf16 rounding residual (o_lo) and the backward forms delta from
O + o_lo, as the library's tests do.

Besides the step, the permutes are timed cold: each permute of the step is run alone after a
512 MiB write that evicts the 256 MB Infinity Cache and the L2s, several times, and reported
with median, min and max; their rate against the 8 TB/s HBM peak is `permute_roofline`.

--ring times Ring Attention, the pages' comparison workload, over the whole layer on one GPU
(every rank's ring forward, then every rank's ring backward in rank order), with P times the
Ulysses rank share of the same layer beside it. --exchange times one rank's send-side and
receive-side permutes of a training step (what a real all-to-all needs around it), cold, on
the workload and with its kv heads replicated to two ranks each; it prints its own line.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                       [--heads-per-chunk U] [--unchunked] [--forward-only [--fused]] [--ring]
                       [--exchange]
"""
import argparse
import contextlib
import gc
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ulysses_sequence_parallelism_rank_amd as U  # noqa: E402
import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
METRIC = "fwd+bwd causal attention TFLOP/s @64K (8q/2kv heads, d128); % MFMA peak"
# the sources each timed kernel is built from: a stored counter reading is used only while they
# are unchanged
KERNEL_SOURCES = {
    "attn_fwd": ["attn_fwd.hip", "uly_device.h"],
    "bwd_dkdv": ["attn_bwd.hip", "uly_device.h"],
    "bwd_dq": ["attn_bwd.hip", "uly_device.h"],
    "bwd_preprocess": ["attn_bwd.hip", "uly_device.h"],
    "permute": ["permute.hip", "uly_device.h"],
}
ALL_SOURCES = ["attn_fwd.hip", "attn_bwd.hip", "permute.hip", "uly_device.h"]


def counted_pairs(cfg, cu):
    if cu is not None:
        lens = np.diff(np.asarray(cu, dtype=np.float64))
        return float((lens * lens).sum() / 2)
    return float(cfg.s) ** 2 / 2


def training_work(cfg, pairs):
    """Per phase of the training step: (bound, algorithmic work per launch). FLOPs count the
    visible pairs (4 d N forward, 8 d N dK/dV, 2 d N dQ per q head, 14 d N in all); bytes are
    the read + write of exactly the moved elements (2 s H_l d e per permuted tensor)."""
    d, Hq_l, Hkv_l, e, s = cfg.d, cfg.Hq_l, cfg.Hkv_l, cfg.esize, cfg.s
    return {
        "attn_fwd": ("mfma", 4.0 * d * pairs * Hq_l),
        "bwd_dkdv": ("mfma", 8.0 * d * pairs * Hq_l),
        "bwd_dq": ("mfma", 2.0 * d * pairs * Hq_l),
        "pack_qkv": ("hbm", 2.0 * s * (Hq_l + 2 * Hkv_l) * d * e),
        "unpack_o": ("hbm", 2.0 * s * Hq_l * d * e),
        "pack_do": ("hbm", 2.0 * s * Hq_l * d * e),
        # O, its residual and dO read, delta written
        "bwd_preprocess": ("hbm", (3.0 if cfg.dtype == "bf16" else 2.0) * s * Hq_l * d * e + 4.0 * s * Hq_l),
        "unpack_grads": ("hbm", 2.0 * s * (Hq_l + 2 * Hkv_l) * d * e),
        # the fused calls, timed whole (attn_bwd_shards: preprocess, dK/dV and dQ)
        "attn_fwd_shards": ("mfma", 4.0 * d * pairs * Hq_l),
        "attn_bwd_shards": ("mfma", 10.0 * d * pairs * Hq_l),
    }


def ring_work(cfg):
    """Ring Attention on the whole layer (every rank's token block of all Hq heads): per rank
    call, (bound, counted FLOPs). Rank r's rows see r earlier blocks whole and its own block
    causally (s_l^2 (r + 1/2) pairs per head; every block whole without the causal mask); the
    forward counts 4 d N and the backward 10 d N per head, as the training step does."""
    s_l, P, d, Hq = float(cfg.s_l), cfg.P, cfg.d, cfg.Hq
    out = {}
    for r in range(P):
        pairs = s_l * s_l * (r + 0.5) if cfg.causal else s_l * s_l * P
        out[f"ring_fwd_r{r}"] = ("mfma", 4.0 * d * pairs * Hq)
        out[f"ring_bwd_r{r}"] = ("mfma", 10.0 * d * pairs * Hq)
    return out


def exchange_shapes(cfg):
    """The send-side and receive-side permutes of one rank per training step, as (name, H, kind):
    send_pack of Q, K, V (forward) and dO (backward) from its sequence shards, recv_unpack of O
    (forward) and dQ, dK, dV (backward) into them."""
    return [("send_q", cfg.Hq, "send"), ("send_k", cfg.Hkv, "send"), ("send_v", cfg.Hkv, "send"),
            ("send_do", cfg.Hq, "send"), ("recv_o", cfg.Hq, "recv"), ("recv_dq", cfg.Hq, "recv"),
            ("recv_dk", cfg.Hkv, "recv"), ("recv_dv", cfg.Hkv, "recv")]


def exchange_bytes(cfg, H):
    """Bytes one send_pack or recv_unpack moves (read + write) for H heads: the shard
    [s_l, H, d] and the P blocks [P, s_l, H_l, d], H_l = H/P, or one replicated head each
    when H < P (a send then writes, and a receive reads, P/H copies of each head)."""
    e = cfg.esize
    hl = H // cfg.P if H % cfg.P == 0 else 1
    return float(cfg.s_l * H * cfg.d * e + cfg.P * cfg.s_l * hl * cfg.d * e)


def replicated_variant(cfg):
    """The same model and sequence over twice as many ranks as kv heads: each kv head then goes
    to two ranks (send_pack writes it twice, recv_unpack sums its two gradient partials)."""
    P = 2 * cfg.Hkv
    return W.Config(f"{cfg.name}_sp{P}", P=P, s_l=cfg.s // P, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d, dtype=cfg.dtype)


def source_hash(kernel=None):
    """Hash of the sources `kernel` is built from (all kernel sources when None)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, ALL_SOURCES):
        with open(os.path.join(ROOT, "ulysses_sequence_parallelism_rank_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(cfg, seed=0):
    glob = {n: W.gen_global(cfg, n, seed) for n in ("q", "k", "v", "do")}
    shards = {n: [W.torch_from_bits(x, cfg.dtype, "cuda") for x in W.shards_of(g, cfg.P)]
              for n, g in glob.items()}
    return glob, shards


@contextlib.contextmanager
def no_gc():
    """Python's cyclic garbage collector off for a timed region (collected just before): a
    collection pass stalls the host thread for milliseconds while the GPU waits for its next
    launch. All the work still runs inside the region."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def alloc_bytes(fn):
    """Device bytes `fn` leaves allocated (torch's caching allocator, so the intermediates the
    caller holds), and the peak above the starting point while it ran."""
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    r = fn()
    torch.cuda.synchronize()
    return r, torch.cuda.memory_allocated() - base, torch.cuda.max_memory_allocated() - base


class Phases:
    """HIP events around every phase of every timed step, on the stream the library uses."""

    def __init__(self):
        self.marks = []   # (name, start_event, end_event)

    def run(self, name, fn, record):
        if not record:
            return fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        self.marks.append((name, a, b))
        return r

    def summary(self, steps):
        """Per phase: the mean over the timed steps, and the median, min and max. The first timed
        step starts on an idle GPU (the region opens with a synchronize), so its first phase also
        holds the host's time to issue that call; the median is free of it."""
        per = {}
        for name, a, b in self.marks:
            per.setdefault(name, []).append(a.elapsed_time(b))
        mean = {k: sum(v) / steps for k, v in per.items()}
        spread = {k: {"median": float(statistics.median(v)), "min": min(v), "max": max(v)} for k, v in per.items()}
        return mean, spread


def run_training_share(cfg, steps, warmup, cu_dev, fused=False):
    _, sh = make_inputs(cfg)
    rank = 0
    s, Hq_l, Hkv_l, d = cfg.s, cfg.Hq_l, cfg.Hkv_l, cfg.d
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = "cuda"
    o_lo = torch.empty((s, Hq_l, d), dtype=torch.bfloat16, device=dev) if cfg.dtype == "bf16" else None
    lse = torch.empty((Hq_l, s), dtype=torch.float32, device=dev)

    def heads():  # the head-shard intermediates and the backward's delta, allocated once
        if fused:  # the shard-reading kernels need no head shards
            # the backward's delta with room for its split runs' partials (short sequences), and
            # the forward's partials
            ws = torch.empty(U.attn_bwd_workspace_bytes(s, Hq_l, Hkv_l, d), dtype=torch.uint8, device=dev)
            need = U.attn_fwd_workspace_bytes(s, Hq_l, d)
            return (None,) * 8 + (ws, torch.empty(need, dtype=torch.uint8, device=dev) if need else None)
        ws = torch.empty(U.delta_bytes(s, Hq_l), dtype=torch.uint8, device=dev)
        q = torch.empty((s, Hq_l, d), dtype=dt, device=dev)
        k = torch.empty((s, Hkv_l, d), dtype=dt, device=dev)
        # room for the partial results of the split runs on short sequences (none at 64K): the
        # forward's row blocks, dK/dV's key blocks, dQ's row blocks; the three run in turn on one
        # stream, each consuming its partials before the next starts, so they share it
        part_need = max(U.attn_fwd_workspace_bytes(s, Hq_l, d), U.attn_bwd_dkdv_workspace_bytes(s, Hkv_l, d),
                        U.attn_bwd_dq_workspace_bytes(s, Hq_l, d))
        part = torch.empty(part_need, dtype=torch.uint8, device=dev) if part_need else None
        return (q, k, torch.empty_like(k), torch.empty_like(q), torch.empty_like(q), torch.empty_like(q),
                torch.empty_like(k), torch.empty_like(k), ws, part)
    (q, k, v, o, do, dq, dk, dv, ws, part_ws), inter, _ = alloc_bytes(heads)
    delta = ws.view(torch.float32)[: Hq_l * s].view(Hq_l, s)
    o_sh = [torch.empty_like(t) for t in sh["q"]]
    dq_sh = [torch.empty_like(t) for t in sh["q"]]
    dk_sh = [torch.empty_like(t) for t in sh["k"]]
    dv_sh = [torch.empty_like(t) for t in sh["v"]]
    ph = Phases()

    def step_fused(rec):
        ph.run("attn_fwd_shards", lambda: U.attn_fwd_shards(sh["q"], sh["k"], sh["v"], o_sh, rank, cfg.scale,
                                                            cfg.causal, cu_dev, lse=lse, o_lo=o_lo,
                                                            workspace=part_ws), rec)
        ph.run("attn_bwd_shards", lambda: U.attn_bwd_shards(sh["q"], sh["k"], sh["v"], o_sh, lse, sh["do"], dq_sh,
                                                            dk_sh, dv_sh, rank, cfg.scale, cfg.causal, cu_dev,
                                                            workspace=ws, o_lo=o_lo), rec)

    def step(rec):
        if fused:
            return step_fused(rec)
        ph.run("pack_qkv", lambda: U.ulysses_pack_group([sh["q"], sh["k"], sh["v"]], rank, [q, k, v]), rec)
        ph.run("attn_fwd", lambda: U.attn_fwd(q, k, v, cfg.scale, cfg.causal, cu_dev, out=o, lse=lse, o_lo=o_lo,
                                              workspace=part_ws), rec)
        ph.run("unpack_o", lambda: U.ulysses_unpack(o, rank, o_sh), rec)
        ph.run("pack_do", lambda: U.ulysses_pack(sh["do"], rank, do), rec)
        ph.run("bwd_preprocess", lambda: U.attn_bwd_preprocess(o, do, delta, o_lo=o_lo), rec)
        ph.run("bwd_dkdv", lambda: U.attn_bwd_dkdv(q, k, v, lse, do, delta, cfg.scale, cfg.causal, cu_dev,
                                                   dk=dk, dv=dv, workspace=part_ws), rec)
        ph.run("bwd_dq", lambda: U.attn_bwd_dq(q, k, v, lse, do, delta, cfg.scale, cfg.causal, cu_dev, dq=dq,
                                               workspace=part_ws), rec)
        ph.run("unpack_grads", lambda: U.ulysses_unpack_group([dq, dk, dv], rank, [dq_sh, dk_sh, dv_sh]), rec)

    for _ in range(warmup):
        step(False)
    with no_gc():
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        call_peak = torch.cuda.max_memory_allocated() - base
    mem = {"intermediate_bytes": int(inter), "calls_peak_alloc_bytes": int(call_peak)}
    cold = None
    if not fused:
        cold = cold_permutes({
            "pack_qkv": lambda: U.ulysses_pack_group([sh["q"], sh["k"], sh["v"]], rank, [q, k, v]),
            "unpack_o": lambda: U.ulysses_unpack(o, rank, o_sh),
            "pack_do": lambda: U.ulysses_pack(sh["do"], rank, do),
            "unpack_grads": lambda: U.ulysses_unpack_group([dq, dk, dv], rank, [dq_sh, dk_sh, dv_sh]),
        })
    return (wall,) + ph.summary(steps) + (cold, mem)


def cold_permutes(calls, reps=7):
    """Each permute alone, `reps` times, each time after a 512 MiB write that evicts the 256 MB
    Infinity Cache and the L2s: per phase the median, min and max in ms."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for name, fn in calls.items():
        ts = []
        for _ in range(reps):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        out[name] = {"median": float(statistics.median(ts)), "min": min(ts), "max": max(ts)}
    del flush
    return out


def run_forward_share(cfg, steps, warmup, cu_dev, fused):
    """The forward half of the path for rank 0: pack Q/K/V -> attn_fwd -> unpack O, or (fused)
    attn_fwd_shards reading the sequence shards and writing O into them directly."""
    _, sh = make_inputs(cfg)
    rank = 0
    s, Hq_l, Hkv_l, d = cfg.s, cfg.Hq_l, cfg.Hkv_l, cfg.d
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    o_sh = [torch.empty_like(t) for t in sh["q"]]
    lse = torch.empty((Hq_l, s), dtype=torch.float32, device="cuda")

    def heads():  # the head-shard intermediates of the unchunked forward (not needed fused)
        need = U.attn_fwd_workspace_bytes(s, Hq_l, d)  # the split forward's partials (short sequences)
        part = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        if fused:
            return None, None, None, None, part
        q = torch.empty((s, Hq_l, d), dtype=dt, device="cuda")
        k = torch.empty((s, Hkv_l, d), dtype=dt, device="cuda")
        return q, k, torch.empty_like(k), torch.empty_like(q), part
    (q, k, v, o, part_ws), inter, _ = alloc_bytes(heads)
    ph = Phases()

    o_lo = torch.empty((s, Hq_l, d), dtype=torch.bfloat16, device="cuda") if cfg.dtype == "bf16" else None

    def step(rec):
        if fused:
            ph.run("attn_fwd_shards", lambda: U.attn_fwd_shards(sh["q"], sh["k"], sh["v"], o_sh, rank, cfg.scale,
                                                                cfg.causal, cu_dev, lse=lse, o_lo=o_lo,
                                                                workspace=part_ws), rec)
            return
        ph.run("pack_qkv", lambda: U.ulysses_pack_group([sh["q"], sh["k"], sh["v"]], rank, [q, k, v]), rec)
        ph.run("attn_fwd", lambda: U.attn_fwd(q, k, v, cfg.scale, cfg.causal, cu_dev, out=o, lse=lse, o_lo=o_lo,
                                              workspace=part_ws), rec)
        ph.run("unpack_o", lambda: U.ulysses_unpack(o, rank, o_sh), rec)

    for _ in range(warmup):
        step(False)
    with no_gc():
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        call_peak = torch.cuda.max_memory_allocated() - base
    return (wall,) + ph.summary(steps) + ({"intermediate_bytes": int(inter), "calls_peak_alloc_bytes": int(call_peak)},)


def run_upipe(cfg, steps, warmup, u, forward_only):
    """The UPipe schedule on the rank-0 share: attn_fwd_chunked, then (unless forward_only)
    attn_bwd_chunked, both on one workspace of the larger queried size."""
    _, sh = make_inputs(cfg)
    o_sh = [torch.empty_like(t) for t in sh["q"]]
    dq_sh = [torch.empty_like(t) for t in sh["q"]]
    dk_sh = [torch.empty_like(t) for t in sh["k"]]
    dv_sh = [torch.empty_like(t) for t in sh["v"]]
    lse = torch.empty((cfg.Hq_l, cfg.s), dtype=torch.float32, device="cuda")
    o_lo = torch.empty((cfg.s, cfg.Hq_l, cfg.d), dtype=torch.bfloat16, device="cuda")
    args = (cfg.P, cfg.s_l, cfg.Hq, cfg.Hkv, cfg.d, torch.bfloat16, u)
    need = {"fwd": U.attn_fwd_chunked_workspace_bytes(*args)}
    if not forward_only:
        need["bwd"] = U.attn_bwd_chunked_workspace_bytes(*args)
    ws = torch.empty(max(need.values()), dtype=torch.uint8, device="cuda")
    ph = Phases()
    with no_gc():
        for i in range(warmup + steps):
            if i == warmup:
                torch.cuda.synchronize()
                torch.cuda.reset_peak_memory_stats()
                base = torch.cuda.memory_allocated()
                t0 = time.perf_counter()
            ph.run("attn_fwd_chunked", lambda: U.attn_fwd_chunked(sh["q"], sh["k"], sh["v"], o_sh, 0, u, cfg.scale,
                                                                  cfg.causal, None, ws, lse, o_lo=o_lo), i >= warmup)
            if not forward_only:
                ph.run("attn_bwd_chunked", lambda: U.attn_bwd_chunked(sh["q"], sh["k"], sh["v"], o_sh, lse, sh["do"],
                                                                      dq_sh, dk_sh, dv_sh, 0, u, cfg.scale,
                                                                      cfg.causal, None, ws, o_lo=o_lo), i >= warmup)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        need["calls_peak_alloc_bytes"] = int(torch.cuda.max_memory_allocated() - base)
    return (wall,) + ph.summary(steps) + (need,)


def run_ring(cfg, steps, warmup):
    """Ring Attention over the whole layer on one GPU (the pages' comparison workload): every
    rank's ring forward, then every rank's ring backward in rank order (the order in which the
    dK/dV sums travel round the ring), each call timed; the ranks' buffers are separate
    allocations, as in the tests."""
    _, sh = make_inputs(cfg)
    P, s_l, Hq, Hkv, d = cfg.P, cfg.s_l, cfg.Hq, cfg.Hkv, cfg.d
    L = U.lib()

    def bufs():
        o = [torch.empty_like(x) for x in sh["q"]]
        lo = [torch.empty(x.shape, dtype=torch.bfloat16, device="cuda") for x in sh["q"]]
        lse = [torch.empty((Hq, s_l), dtype=torch.float32, device="cuda") for _ in range(P)]
        dq = [torch.empty_like(x) for x in sh["q"]]
        dk = [torch.empty_like(x) for x in sh["k"]]
        dv = [torch.empty_like(x) for x in sh["v"]]
        acc = [torch.empty((P, s_l, Hkv, d), dtype=torch.float32, device="cuda") for _ in range(2)]
        ws = [torch.empty(int(L.ring_attn_fwd_workspace_bytes(s_l, Hq, d)), dtype=torch.uint8, device="cuda"),
              torch.empty(int(L.ring_attn_bwd_workspace_bytes(s_l, Hq, d)), dtype=torch.uint8, device="cuda")]
        return o, lo, lse, dq, dk, dv, acc, ws
    (o, lo, lse, dq, dk, dv, acc, ws), inter, _ = alloc_bytes(bufs)
    ph = Phases()

    def step(rec):
        for r in range(P):
            ph.run(f"ring_fwd_r{r}", lambda: U.ring_attn_fwd(sh["q"], sh["k"], sh["v"], r, cfg.scale, cfg.causal,
                                                             out=o[r], lse=lse[r], o_lo=lo[r], workspace=ws[0]), rec)
        for r in range(P):
            ph.run(f"ring_bwd_r{r}", lambda: U.ring_attn_bwd(sh["q"], sh["k"], sh["v"], o[r], lse[r], sh["do"][r], r,
                                                             acc[0], acc[1], dk, dv, cfg.scale, cfg.causal, dq=dq[r],
                                                             o_lo=lo[r], workspace=ws[1]), rec)

    for _ in range(warmup):
        step(False)
    with no_gc():
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        t0 = time.perf_counter()
        for _ in range(steps):
            step(True)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
        call_peak = torch.cuda.max_memory_allocated() - base
    return (wall,) + ph.summary(steps) + ({"intermediate_bytes": int(inter), "calls_peak_alloc_bytes": int(call_peak)},)


def run_exchange(cfg, reps=7):
    """One rank's send-side and receive-side permutes of a training step, each alone on a cold
    cache (after a 512 MiB cache-evicting write, as the step's permutes are timed cold):
    ulysses_send_pack of its Q, K, V and dO sequence shards into P per-destination blocks and
    ulysses_recv_unpack of P received blocks of O, dQ, dK and dV into its sequence shards
    (replicated kv heads summed). Returns per-phase median / min / max ms and bytes."""
    P, s_l, d = cfg.P, cfg.s_l, cfg.d
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    src = {n: W.torch_from_bits(W.gen_rows(cfg, n, 0, s_l), cfg.dtype, "cuda") for n in ("q", "k", "v", "do")}
    calls, nbytes = {}, {}
    for name, H, kind in exchange_shapes(cfg):
        hl = U.rank_heads(0, P, H)[1]
        blocks = torch.zeros((P, s_l, hl, d), dtype=dt, device="cuda")
        if kind == "send":
            shard = src[name.split("_", 1)[1]]
            calls[name] = (lambda x=shard, b=blocks: U.ulysses_send_pack(x, P, b))
        else:
            shard = torch.empty((s_l, H, d), dtype=dt, device="cuda")
            calls[name] = (lambda b=blocks, x=shard, h=H: U.ulysses_recv_unpack(b, h, x))
        nbytes[name] = exchange_bytes(cfg, H)
    for fn in calls.values():
        fn()
    torch.cuda.synchronize()
    return cold_permutes(calls, reps), nbytes


def exchange_line(cfg, spread, nbytes):
    ms = sum(v["median"] for v in spread.values())
    total = sum(nbytes.values())
    gbs = total / (ms * 1e-3) / 1e9
    return {"config": {"P": cfg.P, "s_l": cfg.s_l, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv, "head_dim": cfg.d,
                       "kv_replicated_to": cfg.P // cfg.Hkv if cfg.Hkv < cfg.P else 1},
            "ms_per_step": round(ms, 4), "bytes_per_step": int(total),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4)},
            "phase_ms_median": {k: round(v["median"], 4) for k, v in spread.items()},
            "phase_ms_min": {k: round(v["min"], 4) for k, v in spread.items()},
            "phase_ms_max": {k: round(v["max"], 4) for k, v in spread.items()},
            "phase_bytes": {k: int(v) for k, v in nbytes.items()}}


def measured_ceilings():
    """Practical ceilings on this GPU, beside the published peaks: back-to-back bf16 MFMAs on
    every SIMD (uly_mfma_probe, with the sustained shader clock), the attention kernels'
    inner-loop instruction mix at 2 and 3 waves per SIMD (uly_mix_probe), and a plain 1 GiB
    device copy (ulysses_pack with one rank) for HBM."""
    tf, clk = U.mfma_probe()
    n = 1 << 30
    src = torch.empty((n // 256, 1, 128), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    U.ulysses_pack([src], 0, dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        U.ulysses_pack([src], 0, dst)
    b.record()
    torch.cuda.synchronize()
    gbs = 3 * 2.0 * n / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    # the kernels' inner-loop instruction mix (an LDS operand per product, plus the softmax's VALU
    # work) at the occupancies they run: 2 waves per SIMD (backward kernels) and 3 (forward)
    mix = {f"{U.MIX_KINDS[k]} @{w} waves/SIMD": round(U.mix_probe(k, w), 1) for k in (0, 1, 2) for w in (2, 3)}
    return {"mfma_bf16_tflops": round(tf, 1), "sustained_clock_mhz": round(clk, 0) if clk else None,
            "copy_gbs": round(gbs, 1), "mix_tflops": mix,
            "how": "uly_mfma_probe: 512 workgroups x 4 waves x 20000 x 4 back-to-back 32x32x16 bf16 MFMAs; "
                   "uly_mix_probe: 256 x W workgroups of 4 waves, 4000 rounds of 16 MFMAs each with its "
                   "first operand read from LDS and the listed fp32 FMAs / exp2 after it; "
                   "copy: 1 GiB read + 1 GiB written by ulysses_pack with one rank"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg):
    """The oracle, untuned, on a bounded sample of the same workload: one q head (and its kv
    head) over the first `prefix` tokens of the sequence, causal forward + backward. `cores`
    is the host cores this process may run on; the BLAS threads numpy used are listed too."""
    from threadpoolctl import threadpool_info

    from oracle import attention as OA
    prefix = min(cfg.s, 32768)
    f = {n: W.bits_to_f64(W.gen_rows(cfg, n, 0, prefix)[:, :1], cfg.dtype) for n in ("q", "k", "v", "do")}
    t0 = time.perf_counter()
    OA.forward(f["q"], f["k"], f["v"], cfg.scale, cfg.causal)
    OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, cfg.causal)
    dt = time.perf_counter() - t0
    flops = 14.0 * cfg.d * prefix * prefix / 2
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    # the permute oracle (a Python loop over rows and heads) on the Q pack of rank 0, the first
    # rows of each shard, as the algorithmic bytes it moves per second
    from oracle import permute as OP
    rows = min(cfg.s_l, 4096)
    shards = [W.gen_rows(cfg, "q", p * cfg.s_l, p * cfg.s_l + rows) for p in range(cfg.P)]
    t1 = time.perf_counter()
    y = OP.pack(shards, 0)
    dtp = time.perf_counter() - t1
    moved = 2 * y.nbytes
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "blas_threads": int(threads), "kind": "oracle",
            "sample": f"numpy fp64 oracle, causal fwd+bwd of 1 q head (+ its kv head) over the first {prefix} "
                      f"tokens, d={cfg.d}; {dt:.1f} s; FLOPs counted as in the metric",
            "permute": {"value": round(moved / dtp / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                        "sample": f"oracle pack of Q for rank 0 from the first {rows} rows of each of the {cfg.P} "
                                  f"shards ({moved / 2**20:.1f} MiB read + written, one thread); {dtp:.2f} s"}}


def main_exchange(args, cfg):
    """--exchange: one JSON line for one rank's send/recv permutes of a training step on the
    workload, with the kv-replicated variant beside it."""
    spread, nbytes = run_exchange(cfg)
    line = exchange_line(cfg, spread, nbytes)
    rcfg = replicated_variant(cfg)
    rep_line = None
    if rcfg.Hq % rcfg.P == 0 and cfg.dtype == "bf16":
        rs, rb = run_exchange(rcfg)
        rep_line = exchange_line(rcfg, rs, rb)
    ceil = measured_ceilings()
    roof = dict(line["roofline"], kernel="ulysses_send_pack + ulysses_recv_unpack", avg_ms=line["ms_per_step"],
                traffic=None)
    roof["frac_of_measured"] = round(roof["achieved"] / ceil["copy_gbs"], 4)
    out = {"metric": f"send/recv exchange permutes GB/s [workload {args.workload}: one rank's per-step send_pack "
                     "of Q, K, V, dO and recv_unpack of O, dQ, dK, dV, each alone on a cold cache]",
           "value": roof["achieved"], "unit": "GB/s", "n_gpus": 1, "steps": 7, "warmup": 1,
           "ms_per_step": line["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": cfg.dtype, "data": "synthetic",
           "config": dict(line["config"], workload=f"{args.workload}: one rank's all-to-all buffers"),
           "roofline": roof, "bytes_per_step": line["bytes_per_step"],
           "phase_ms_median": line["phase_ms_median"], "phase_ms_min": line["phase_ms_min"],
           "phase_ms_max": line["phase_ms_max"], "phase_bytes": line["phase_bytes"],
           "replicated_kv": rep_line, "measured_ceilings": ceil}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen_64k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--heads-per-chunk", type=int, default=1)
    ap.add_argument("--forward-only", action="store_true",
                    help="time the forward half of the path alone (UPipe workload: the chunked forward)")
    ap.add_argument("--unchunked", action="store_true",
                    help="UPipe workload: the same share without chunking (pack, attention and unpack of every "
                         "local head at once), for comparison")
    ap.add_argument("--fused", action="store_true",
                    help="attn_fwd_shards / attn_bwd_shards, reading and writing the sequence shards directly "
                         "(no head-shard buffers, no separate permutes)")
    ap.add_argument("--ring", action="store_true",
                    help="Ring Attention over the whole layer (every rank's token block of all heads, forward then "
                         "backward in rank order), beside the Ulysses ranks' shares of the same layer")
    ap.add_argument("--exchange", action="store_true",
                    help="one rank's send-side and receive-side permutes of a training step (send_pack of Q, K, V, "
                         "dO; recv_unpack of O, dQ, dK, dV), cold cache, and the same with each kv head "
                         "replicated to two ranks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy (ulysses_pack with one rank) and exit; "
                         "its FETCH_SIZE/WRITE_SIZE counters scale the traffic of other kernels")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the layer and runs on one GPU only (the P ranks are "
              "simulated as buffers on one device).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    U.lib()
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.empty((n // 256, 1, 128), dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        U.ulysses_pack([src], 0, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n}), flush=True)
        return
    cfg = W.WORKLOADS[args.workload]
    if args.exchange:
        return main_exchange(args, cfg)
    cu = W.cu_seqlens_for(cfg)
    cu_dev = None if cu is None else torch.from_numpy(cu).to("cuda")
    pairs = counted_pairs(cfg, cu)
    d, Hq_l, Hkv_l, e = cfg.d, cfg.Hq_l, cfg.Hkv_l, cfg.esize

    chunked = bool(cfg.chunk_heads) and not args.unchunked and not args.ring
    cold = mem = ring_cmp = None
    if args.ring:
        if cu is not None or cfg.dtype != "bf16":
            print("--ring runs bf16 workloads without packed documents", file=sys.stderr)
            sys.exit(2)
        wall, ph, spread, mem = run_ring(cfg, args.steps, args.warmup)
        kern = ring_work(cfg)
        flops = sum(w for _, w in kern.values())
        # the same layer as the Ulysses ranks split it, on this machine: the ranks' shares are equal
        # (every position of H/P heads each), so P times rank 0's training step
        u_steps = max(2, args.steps // 2)
        u_wall = run_training_share(cfg, u_steps, 1, cu_dev)[0]
        # per rank: a P-GPU job waits for its slowest rank, and the causal ring's ranks do unequal
        # work (rank r attends r + 1 blocks); the Ulysses ranks' shares are equal
        rank_ms = [ph[f"ring_fwd_r{r}"] + ph[f"ring_bwd_r{r}"] for r in range(cfg.P)]
        ring_cmp = {"ring_layer_ms": round(wall * 1e3, 3), "ulysses_layer_ms": round(cfg.P * u_wall * 1e3, 3),
                    "ring_over_ulysses": round(wall / (cfg.P * u_wall), 4),
                    "ring_rank_ms": [round(x, 3) for x in rank_ms], "ulysses_rank_ms": round(u_wall * 1e3, 3),
                    "slowest_ring_rank_over_ulysses_rank": round(max(rank_ms) / (u_wall * 1e3), 4),
                    "how": f"Ulysses: {cfg.P} x rank 0's training step (permutes, forward, backward), "
                           f"{u_steps} steps; ring: every rank's ring_attn_fwd then ring_attn_bwd; attention work "
                           "only, one GPU, no collective"}
    elif not chunked and args.forward_only:
        wall, ph, spread, mem = run_forward_share(cfg, args.steps, args.warmup, cu_dev, args.fused)
        fw = 4.0 * d * pairs * Hq_l
        kern = {"attn_fwd": ("mfma", fw), "attn_fwd_shards": ("mfma", fw),
                "pack_qkv": ("hbm", 2.0 * cfg.s * (Hq_l + 2 * Hkv_l) * d * e),
                "unpack_o": ("hbm", 2.0 * cfg.s * Hq_l * d * e)}
        flops = fw
    elif not chunked:
        wall, ph, spread, cold, mem = run_training_share(cfg, args.steps, args.warmup, cu_dev, args.fused)
        flops = 14.0 * d * pairs * Hq_l
        kern = training_work(cfg, pairs)
    else:
        wall, ph, spread, ws_bytes = run_upipe(cfg, args.steps, args.warmup, args.heads_per_chunk, args.forward_only)
        # each call is timed whole (per chunk: permutes and attention kernels)
        kern = {"attn_fwd_chunked": ("mfma", 4.0 * d * pairs * Hq_l)}
        if not args.forward_only:
            kern["attn_bwd_chunked"] = ("mfma", 10.0 * d * pairs * Hq_l)
        flops = sum(w for _, w in kern.values())

    step_ms = wall * 1e3
    dom = max(ph, key=ph.get)
    bound, work = kern[dom]
    ms = ph[dom]
    if bound == "mfma":
        achieved = work / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = work / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["kernel"] = dom
    roof["avg_ms"] = round(ms, 4)
    roof["traffic"] = read_traffic(dom, args.workload)

    attn_ms = sum(v for k, v in ph.items() if k.startswith("ring_") or k in (
        "attn_fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "attn_fwd_chunked", "attn_bwd_chunked", "attn_fwd_shards",
        "attn_bwd_shards"))
    # the permutes' rate inside the step from the per-phase medians (see Phases.summary: the first
    # phase of the first timed step also holds a host launch latency)
    perm_names = ("pack_qkv", "unpack_o", "pack_do", "unpack_grads")
    perm_ms = sum(spread[k]["median"] for k in perm_names if k in spread)
    perm_bytes = sum(kern[k][1] for k in perm_names if k in ph)
    value = flops / wall / 1e12
    out = {
        "metric": METRIC if args.workload == "qwen_64k" and not (args.forward_only or args.fused or args.ring) else
        f"{METRIC} [workload {args.workload}{', unchunked' if args.unchunked else ''}"
        f"{', forward only' if args.forward_only else ''}{', fused exchange' if args.fused else ''}"
        f"{f', Ring Attention over all {cfg.P} ranks and {cfg.Hq} heads' if args.ring else ''}]",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": {"qwen_64k": "Qwen3-4B-shaped SP=4 rank share at 65536 tokens",
                         "qwen_8k": "Qwen3-4B-shaped SP=4 rank share at 8192 tokens",
                         "qwen_16k": "Qwen3-4B-shaped SP=4 rank share at 16384 tokens",
                         "qwen_32k": "Qwen3-4B-shaped SP=4 rank share at 32768 tokens",
                         "packed_96k": "packed SFT batch at 98304 tokens (documents ~ geometric, mean 6000)",
                         "million": "one rank's share of a 1048576-token sequence (SP=8, 16 q / 8 kv heads)",
                         "upipe_256k": (f"UPipe headwise-chunked {'forward' if args.forward_only else 'forward+backward'}, "
                                        f"32B-shaped SP=8 share at 262144 tokens, {args.heads_per_chunk} q heads per "
                                        "chunk") if chunked else
                         (f"unchunked {'forward' if args.forward_only else 'forward+backward'} of the 32B-shaped "
                          "SP=8 share at 262144 tokens (every local head at once)"),
                         "tiny_f32": "tiny fp32 case"}[args.workload],
            "seq_len": cfg.s, "ranks_simulated": cfg.P, "rank": "all" if args.ring else 0,
            "q_heads": cfg.Hq if args.ring else Hq_l, "kv_heads": cfg.Hkv if args.ring else Hkv_l,
            "head_dim": d, "causal": cfg.causal, "packed_docs": None if cu is None else int(len(cu) - 1),
            "global_batch": 1, "parallelism": f"sp{cfg.P} (one rank's share, ranks as buffers)",
        },
        "roofline": roof,
        "mfma_frac_of_step": round(value / PEAK_BF16_TFLOPS, 4),
        "attention_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 2) if attn_ms else None,
        "permute_gbs": round(perm_bytes / (perm_ms * 1e-3) / 1e9, 1) if perm_ms else None,
        "permute_frac_of_step": round(perm_ms / step_ms, 4) if perm_ms and step_ms else None,
        "phase_ms": {k: round(v, 4) for k, v in ph.items()},
        "phase_ms_median": {k: round(v["median"], 4) for k, v in spread.items()},
        "phase_ms_min": {k: round(v["min"], 4) for k, v in spread.items()},
        "phase_ms_max": {k: round(v["max"], 4) for k, v in spread.items()},
    }
    if cold:
        # the permutes alone on a cold cache: HBM rate of their algorithmic bytes
        cold_ms = sum(v["median"] for v in cold.values())
        cold_bytes = sum(kern[k][1] for k in cold)
        gbs = cold_bytes / (cold_ms * 1e-3) / 1e9
        out["permute_roofline"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": cold_bytes, "ms": round(cold_ms, 4),
            "how": "each permute of the step alone after a 512 MiB cache-evicting write, 7 runs, medians",
            "phases": {k: {m: round(x, 4) for m, x in v.items()} for k, v in cold.items()}}
    if ring_cmp:
        out["ring_vs_ulysses"] = ring_cmp
    if mem is not None:
        # device memory of the share's intermediates (head shards, delta), measured with torch's
        # allocator, and the peak the library's calls added (they allocate nothing)
        out["memory"] = mem
    if chunked:
        # peak intermediate bytes: the chunked calls' workspaces (the chunks read the shards, so
        # the forward needs none and the backward delta and fp32 dK/dV sums), and the buffers a
        # multi-GPU all-to-all would have to deliver -- staged per chunk (Q/O of u heads, K/V of
        # their kv heads) against unchunked (every local head): the UPipe accounting
        out["memory"] = {"workspace_bytes": int(max(v for k, v in ws_bytes.items() if k != "calls_peak_alloc_bytes")),
                         "calls_peak_alloc_bytes": ws_bytes["calls_peak_alloc_bytes"]}
        out["workspace_bytes"] = {k: v for k, v in ws_bytes.items() if k != "calls_peak_alloc_bytes"}
        u = min(args.heads_per_chunk, Hq_l)
        span = max((min(c0 + u, Hq_l) - 1) // cfg.G - c0 // cfg.G + 1 for c0 in range(0, Hq_l, u))
        staged = 2 * cfg.s * u * d * e + 2 * cfg.s * span * d * e
        fwd_b = 2 * cfg.s * Hq_l * d * e + 2 * cfg.s * Hkv_l * d * e
        out["staged_chunk_bytes"] = int(staged)
        out["unchunked_intermediate_bytes"] = int(fwd_b if args.forward_only else 2 * fwd_b + 4 * cfg.s * Hq_l)
        out["staged_reduction_q_shaped"] = round(1 - u / Hq_l, 4)
    ceil = measured_ceilings()
    out["measured_ceilings"] = ceil
    roof["frac_of_measured"] = round(roof["achieved"] / (ceil["mfma_bf16_tflops"] if bound == "mfma"
                                                         else ceil["copy_gbs"]), 4)
    if "permute_roofline" in out:
        out["permute_roofline"]["frac_of_measured"] = round(out["permute_roofline"]["achieved"] / ceil["copy_gbs"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
