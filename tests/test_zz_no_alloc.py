"""attn_bwd_noalloc, the backward for callers that cannot allocate, against attn_bwd (same
kernels, delta in the library's static device array instead of a caller workspace, dK/dV
unsplit): bitwise equal to attn_bwd run unsplit and within the parity tolerance of attn_bwd's
default (split on these short sequences) on two calls in a row, the second smaller than the
first; and a size beyond the array rejected with nothing written."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
from tests.helpers import compare, dev_to_f64

pytestmark = pytest.mark.gpu


def _case(s, Hq, Hkv, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    mk = lambda H: torch.randn((s, H, d), device="cuda", generator=g).to(torch.bfloat16)
    return mk(Hq), mk(Hkv), mk(Hkv), mk(Hq)


@pytest.mark.parametrize("cases", [[(1500, 8, 2, 128, None), (333, 4, 2, 64, [0, 50, 51, 200, 333])]])
def test_noalloc_equals_attn_bwd_twice(cases):
    for i, (s, Hq, Hkv, d, cu) in enumerate(cases):
        print(f"case {i}: s={s} Hq={Hq} Hkv={Hkv} d={d} cu={cu is not None}", flush=True)
        q, k, v, do = _case(s, Hq, Hkv, d, 40 + i)
        cu_dev = None if cu is None else torch.tensor(cu, dtype=torch.int32, device="cuda")
        o_lo = U.new_o_lo(q)
        o, lse = U.attn_fwd(q, k, v, causal=True, cu_seqlens=cu_dev, o_lo=o_lo)
        want = U.attn_bwd(q, k, v, o, lse, do, causal=True, cu_seqlens=cu_dev, o_lo=o_lo, split=False)
        split = U.attn_bwd(q, k, v, o, lse, do, causal=True, cu_seqlens=cu_dev, o_lo=o_lo)
        got = [torch.full_like(t, 7.0) for t in want]
        U.attn_bwd_noalloc(q, k, v, o, lse, do, causal=True, cu_seqlens=cu_dev, dq=got[0], dk=got[1], dv=got[2],
                           o_lo=o_lo)
        torch.cuda.synchronize()
        for name, a, b, c in zip(("dq", "dk", "dv"), got, want, split):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (i, name)
            compare(f"noalloc {name} vs attn_bwd", dev_to_f64(a), dev_to_f64(c), bf16=True)


def test_noalloc_rejects_beyond_the_array():
    s, Hq = U.NOALLOC_MAX_DELTA // 4 + 128, 4
    q = torch.zeros((s, Hq, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((s, 1, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((Hq, s), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(k, 7.0)
    with pytest.raises(U.UlyssesError):
        U.attn_bwd_noalloc(q, k, k, q, lse, q, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool((dq == 7.0).all()) and bool((dk == 7.0).all()) and bool((dv == 7.0).all())
