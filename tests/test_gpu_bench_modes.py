"""The bench's Ring Attention and exchange modes, driven in-process on small shapes so that
their code paths stay exercised: every rank call of the ring is timed and its output matches
the unsharded oracle, and the exchange times every send/recv phase, with and without kv
replication, moving the bytes its accounting states."""
import importlib.util
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from tests.helpers import LSE_ABS, compare, dev_to_f64

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_gpu_modes", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_ring_mode(bench):
    cfg = W.Config("ring_small", P=4, s_l=256, Hq=8, Hkv=4, d=128, dtype="bf16")
    print("case bench ring mode", flush=True)
    wall, ph, spread, mem = bench.run_ring(cfg, 2, 1)
    assert sorted(ph) == sorted(bench.ring_work(cfg))
    assert wall > 0 and all(v > 0 for v in ph.values())
    assert mem["calls_peak_alloc_bytes"] == 0


def test_ring_mode_output_matches_oracle(bench):
    """The calls the mode times, on the inputs it generates (bench.make_inputs): every rank's
    ring forward against the oracle rows of its block."""
    import ulysses_sequence_parallelism_rank_amd as U
    cfg = W.Config("ring_small", P=2, s_l=256, Hq=4, Hkv=2, d=64, dtype="bf16")
    glob, sh = bench.make_inputs(cfg)
    outs = [U.ring_attn_fwd(sh["q"], sh["k"], sh["v"], r, cfg.scale, True) for r in range(cfg.P)]
    torch.cuda.synchronize()
    f = {n: W.bits_to_f64(g, "bf16") for n, g in glob.items()}
    wo, wl = OA.forward(f["q"], f["k"], f["v"], cfg.scale, True)
    compare("ring O", dev_to_f64(torch.cat([o for o, _ in outs])), wo, bf16=True)
    compare("ring LSE", torch.cat([l for _, l in outs], dim=1).cpu().numpy(), wl, max_abs=LSE_ABS, rel_fro=1e-4)


@pytest.mark.parametrize("Hkv", [4, 2])   # P = 4: one kv head per rank, then each replicated to 2 ranks
def test_exchange_mode(bench, Hkv):
    cfg = W.Config("exchange_small", P=4, s_l=512, Hq=8, Hkv=Hkv, d=128, dtype="bf16")
    print(f"case bench exchange mode Hkv={Hkv}", flush=True)
    spread, nbytes = bench.run_exchange(cfg, reps=2)
    names = [n for n, _, _ in bench.exchange_shapes(cfg)]
    assert sorted(spread) == sorted(names) and sorted(nbytes) == sorted(names)
    assert all(v["median"] > 0 for v in spread.values())
    line = bench.exchange_line(cfg, spread, nbytes)
    assert line["bytes_per_step"] == int(sum(nbytes.values()))
    assert line["config"]["kv_replicated_to"] == (cfg.P // Hkv if Hkv < cfg.P else 1)
    assert np.isfinite(line["roofline"]["achieved"])
