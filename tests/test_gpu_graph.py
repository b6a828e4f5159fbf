"""The share's forward and backward captured in a HIP graph (torch.cuda.graph) and replayed.

The C ABI neither allocates nor synchronises, so its calls can be captured as they are. The
graph is replayed several times on new inputs copied into its static buffers, with eager work
and synchronisations between the replays, and every replay must give the bits an eager run on
the same inputs gives (the library records no memset, which has misbehaved on replays after
the first on these GPUs). Two graphs: attn_fwd + attn_bwd with a caller workspace, and
attn_fwd + attn_bwd_noalloc (its static delta array), on a causal packed batch short enough
that the forward, given its workspace, splits its row blocks' keys and merges them in a
second kernel, as the backward's dK/dV and dQ do with theirs."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def _bits(s, H, d, seed):
    rng = np.random.default_rng(seed)
    return W.to_bf16_bits(rng.standard_normal((s, H, d), dtype=np.float32))


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager(noalloc):
    s, Hq, Hkv, d = 1536, 8, 2, 128
    print(f"case graph replay noalloc={noalloc} s={s}", flush=True)
    cu = torch.tensor([0, 300, 301, 1000, 1536], dtype=torch.int32, device="cuda")
    q = torch.empty((s, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((s, Hkv, d), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    do = torch.empty_like(q)
    o, lse, o_lo = torch.empty_like(q), torch.empty((Hq, s), dtype=torch.float32, device="cuda"), U.new_o_lo(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(U.attn_bwd_workspace_bytes(s, Hq, Hkv, d), dtype=torch.uint8, device="cuda")
    fws = torch.empty(U.attn_fwd_workspace_bytes(s, Hq, d), dtype=torch.uint8, device="cuda")  # split forward
    assert fws.numel() > 0

    def step():
        U.attn_fwd(q, k, v, None, True, cu, out=o, lse=lse, o_lo=o_lo, workspace=fws)
        if noalloc:
            U.attn_bwd_noalloc(q, k, v, o, lse, do, None, True, cu, dq=dq, dk=dk, dv=dv, o_lo=o_lo)
        else:
            U.attn_bwd(q, k, v, o, lse, do, None, True, cu, workspace=ws, dq=dq, dk=dk, dv=dv, o_lo=o_lo)

    def load(seed):
        for t, H, off in ((q, Hq, 0), (k, Hkv, 1), (v, Hkv, 2), (do, Hq, 3)):
            t.copy_(to_dev(_bits(s, H, d, 10 * seed + off), "bf16"))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream, as capture requires
        load(0)
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        load(seed)
        step()  # eager reference on the same inputs
        torch.cuda.synchronize()
        want = [t.clone() for t in (o, o_lo, lse, dq, dk, dv)]
        for t in (o, o_lo, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "o_lo", "LSE", "dQ", "dK", "dV"), (o, o_lo, lse, dq, dk, dv), want):
            assert _same(a, b), f"replay {seed}: {name} differs from the eager run"
