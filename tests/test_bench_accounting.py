"""The bench's work accounting, on the CPU: the counted FLOPs and moved bytes per phase for
the workloads it times, against the figures derived by hand from the shapes (causal pairs
s^2/2, or the sum of l^2/2 over packed documents; 14 d N FLOPs per q head in a training step;
2 s H_l d e bytes per permuted tensor)."""
import importlib.util
import os

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_64k_share_flops_and_bytes(bench):
    cfg = W.WORKLOADS["qwen_64k"]
    pairs = bench.counted_pairs(cfg, W.cu_seqlens_for(cfg))
    assert pairs == 65536.0 ** 2 / 2
    k = bench.training_work(cfg, pairs)
    # 8 q heads, d 128: forward 4 d N H = 8.796e12, backward 2.5x, step 3.079e13
    assert k["attn_fwd"][1] == pytest.approx(8.796e12, rel=1e-3)
    assert k["bwd_dkdv"][1] + k["bwd_dq"][1] == pytest.approx(2.199e13, rel=1e-3)
    assert sum(k[n][1] for n in ("attn_fwd", "bwd_dkdv", "bwd_dq")) == pytest.approx(3.079e13, rel=1e-3)
    assert k["attn_fwd_shards"][1] + k["attn_bwd_shards"][1] == pytest.approx(3.079e13, rel=1e-3)
    mib = 1 << 20
    # Q/K/V pack and dQ/dK/dV unpack: (128 + 32 + 32) MiB read and written; O, dO: 128 MiB each way
    assert k["pack_qkv"][1] == 384 * mib and k["unpack_grads"][1] == 384 * mib
    assert k["unpack_o"][1] == 256 * mib and k["pack_do"][1] == 256 * mib
    assert sum(k[n][1] for n in ("pack_qkv", "unpack_o", "pack_do", "unpack_grads")) == 1280 * mib
    assert all(k[n][0] == "mfma" for n in ("attn_fwd", "bwd_dkdv", "bwd_dq"))
    assert all(k[n][0] == "hbm" for n in ("pack_qkv", "unpack_o", "pack_do", "unpack_grads", "bwd_preprocess"))


def test_packed_pairs_are_within_documents(bench):
    cfg = W.WORKLOADS["packed_96k"]
    cu = W.cu_seqlens_for(cfg)
    pairs = bench.counted_pairs(cfg, cu)
    lens = np.diff(cu).astype(np.float64)
    assert pairs == pytest.approx((lens ** 2).sum() / 2)
    # seed-0 documents: 11 of them, 20.4% of the dense causal pairs, forward 4.045e12 FLOPs
    assert len(lens) == 11
    assert pairs / (cfg.s ** 2 / 2) == pytest.approx(0.204, abs=5e-4)
    assert bench.training_work(cfg, pairs)["attn_fwd"][1] == pytest.approx(4.045e12, rel=1e-3)


def test_counter_readings_are_keyed_to_their_own_kernel(bench):
    # a stored dK/dV counter reading stays valid when only the permutes or the forward change
    assert "permute.hip" not in bench.KERNEL_SOURCES["bwd_dkdv"]
    assert "attn_fwd.hip" not in bench.KERNEL_SOURCES["bwd_dkdv"]
    assert bench.source_hash("bwd_dkdv") == bench.source_hash("bwd_dq")
    assert bench.source_hash("bwd_dkdv") != bench.source_hash("attn_fwd")


def test_ring_work_sums_to_the_layer(bench):
    """Ring Attention's per-rank calls cover the whole causal layer once: rank r's rows see r
    earlier blocks whole and their own block causally, s_l^2 (r + 1/2) pairs per head, summing to
    s^2/2; 14 d N FLOPs per head over all 32 heads at 64K."""
    cfg = W.WORKLOADS["qwen_64k"]
    k = bench.ring_work(cfg)
    s_l = float(cfg.s_l)
    assert sorted(k) == sorted([f"ring_fwd_r{r}" for r in range(4)] + [f"ring_bwd_r{r}" for r in range(4)])
    for r in range(4):
        assert k[f"ring_fwd_r{r}"][1] == 4.0 * cfg.d * s_l * s_l * (r + 0.5) * cfg.Hq
        assert k[f"ring_bwd_r{r}"][1] == 2.5 * k[f"ring_fwd_r{r}"][1]
    total = sum(w for _, w in k.values())
    assert total == pytest.approx(14.0 * cfg.d * cfg.s ** 2 / 2 * cfg.Hq, rel=1e-12)
    assert total == pytest.approx(4 * 3.079e13, rel=1e-3)   # the 4 Ulysses ranks' shares together


def test_exchange_bytes(bench):
    """send_pack / recv_unpack move the shard [s_l, H, d] and the P blocks [P, s_l, H/P, d]; with
    a kv head replicated to two ranks the blocks hold one head each, twice the shard's kv bytes."""
    cfg = W.WORKLOADS["qwen_64k"]
    mib = 1 << 20
    names = [n for n, _, _ in bench.exchange_shapes(cfg)]
    assert names == ["send_q", "send_k", "send_v", "send_do", "recv_o", "recv_dq", "recv_dk", "recv_dv"]
    assert bench.exchange_bytes(cfg, cfg.Hq) == 256 * mib      # 128 MiB shard + 128 MiB of blocks
    assert bench.exchange_bytes(cfg, cfg.Hkv) == 64 * mib
    rcfg = bench.replicated_variant(cfg)
    assert (rcfg.P, rcfg.s_l, rcfg.s) == (16, 4096, cfg.s)
    assert bench.exchange_bytes(rcfg, rcfg.Hkv) == 8 * mib + 16 * mib    # shard 8 MiB, 16 blocks of one head
    assert bench.exchange_bytes(rcfg, rcfg.Hq) == 64 * mib     # 32 MiB shard + 32 MiB of blocks
