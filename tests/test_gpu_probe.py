"""The measurement helpers uly_mfma_probe (a plausible practical MFMA ceiling and sustained
clock) and uly_mix_probe (the inner-loop instruction mix), and their argument checks."""
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U

pytestmark = pytest.mark.gpu


def test_mfma_probe_plausible():
    tf, clk = U.mfma_probe(iters=4000, blocks=512)
    # MI355X: 2.5 PFLOP/s dense bf16 at 2.4 GHz; the probe cannot exceed it by much
    assert 200.0 < tf < 2700.0, tf
    assert clk is not None and 500.0 < clk < 3000.0, clk


def test_mfma_probe_rejects_bad_arguments():
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    with pytest.raises(U.UlyssesError):
        U._call("uly_mfma_probe", 0, 4, U._dev(sink), U._dev(clocks), U._stream())
    with pytest.raises(U.UlyssesError):
        U._call("uly_mfma_probe", 4, 4, None, U._dev(clocks), U._stream())


def test_mix_probe_plausible():
    r = {(k, w): U.mix_probe(k, w, iters=1000) for k in (0, 2) for w in (2, 3)}
    for key, tf in r.items():
        assert 100.0 < tf < 2700.0, (key, tf)
    # the VALU work per product costs rate at a fixed occupancy
    assert r[(2, 2)] < r[(0, 2)], r
    with pytest.raises(ValueError):
        U.mix_probe(3, 2)
    with pytest.raises(ValueError):
        U.mix_probe(0, 5)
