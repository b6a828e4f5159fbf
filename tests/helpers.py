"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run the
oracle on the same bytes, and compare with the tolerances the tests state.

Tolerance for floating-point outputs (O, dQ, dK, dV), computed over the compared
elements in float64 against the fp64 oracle: max |gpu - oracle| <= 2e-2 and
||gpu - oracle||_F / ||oracle||_F <= 5e-3. LSE: max |gpu - oracle| <= 1e-3.
Permutes: bit-exact.

A bf16 output cannot hold the exact value: storing it costs up to half a bf16 ulp,
2^(e-8) for |x| in [2^e, 2^(e+1)), which is 0.03125 already for |x| in [8, 16) (dV of
the first keys of a long causal sequence reaches that range). For bf16 outputs the
max-abs bar therefore applies to the error beyond that storage rounding:
|gpu - oracle| - ulp_bf16(oracle)/2 <= 2e-2, element by element. The relative
Frobenius bar is applied unchanged."""
import numpy as np
import torch

import workloads as W

MAX_ABS = 2e-2
REL_FRO = 5e-3
LSE_ABS = 1e-3


def to_dev(bits, dtype, device="cuda"):
    return W.torch_from_bits(bits, dtype, device)


def dev_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.detach().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    """Half the bf16 spacing at |x| (bf16 keeps 8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def compare(name, got, want, max_abs=MAX_ABS, rel_fro=REL_FRO, bf16=False, allow=None):
    """`allow`: per-element storage-rounding allowance replacing half a bf16 ulp of `want`
    (for values assembled from several separately rounded bf16 parts)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - want)
    if allow is not None:
        err = np.maximum(err - allow, 0.0)
    elif bf16:
        err = np.maximum(err - half_ulp_bf16(want), 0.0)
    mx = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want)) / den if den > 0 else float(np.linalg.norm(got - want))
    assert mx <= max_abs, f"{name}: max abs err {mx:.3e} > {max_abs:.1e} (rel fro {rel:.3e})"
    assert rel <= rel_fro, f"{name}: rel fro err {rel:.3e} > {rel_fro:.1e} (max abs {mx:.3e})"
    return mx, rel


def sample_rows(s, tile=128, extra=()):
    """Rows that cover the start, every tile boundary (both sides) at a stride, and the end."""
    rows = set(range(min(64, s)))
    rows |= set(range(max(0, s - 64), s))
    stride = max(tile, (s // 48) // tile * tile)
    for b in range(tile, s, stride):
        rows |= {b - 1, b, b + 1}
    rows |= {r for r in extra if 0 <= r < s}
    return np.array(sorted(r for r in rows if r < s))


def gen_shards(cfg, name, seed=0, device="cuda"):
    """Global tensor bits and the P device shards of it."""
    g = W.gen_global(cfg, name, seed)
    return g, [to_dev(x, cfg.dtype, device) for x in W.shards_of(g, cfg.P)]
