"""GPU parity of the stored-dS backward (attn_bwd_dkdv_store_ds + attn_bwd_dq_stored_ds):
dQ, dK and dV against the fp64 oracle at small sizes (every element; causal and not, both
head dims, ragged lengths), dK/dV bit-identical to attn_bwd_dkdv (the stored dS is the
operand its dK product already uses), and dQ on sampled rows of the 64K share."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from tests.helpers import compare, dev_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _bits16(t):
    return t.view(torch.int16)


def _stored_ds_bwd(q, k, v, do, scale, causal):
    o, lse = U.attn_fwd(q, k, v, scale, causal)
    delta = U.attn_bwd_preprocess(o, do)
    s, Hq, _ = q.shape
    ds = torch.empty(U.attn_bwd_stored_ds_bytes(s, Hq, causal), dtype=torch.uint8, device="cuda")
    dk, dv = U.attn_bwd_dkdv_store_ds(q, k, v, lse, do, delta, ds, scale, causal)
    dq = U.attn_bwd_dq_stored_ds(k, ds, torch.empty_like(q), scale, causal)
    ref_dk, ref_dv = U.attn_bwd_dkdv(q, k, v, lse, do, delta, scale, causal)
    return dq, dk, dv, ref_dk, ref_dv


@pytest.mark.parametrize("s,Hq,Hkv,d,causal", [
    (1, 2, 1, 128, True),
    (129, 2, 1, 64, True),      # one key block and a 1-row tail
    (257, 8, 2, 128, True),
    (600, 4, 2, 64, False),
    (333, 4, 4, 128, False),
    (1024, 8, 2, 128, True),
])
def test_stored_ds_matches_oracle(s, Hq, Hkv, d, causal):
    print(f"case stored dS s={s} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
    rng = np.random.default_rng(s + 7 * Hq)
    mk = lambda H: W.to_bf16_bits(rng.standard_normal((s, H, d), dtype=np.float32))
    bits = {"q": mk(Hq), "k": mk(Hkv), "v": mk(Hkv), "do": mk(Hq)}
    f = {n: W.bits_to_f64(b, "bf16") for n, b in bits.items()}
    g = {n: to_dev(b, "bf16") for n, b in bits.items()}
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv, ref_dk, ref_dv = _stored_ds_bwd(g["q"], g["k"], g["v"], g["do"], scale, causal)
    torch.cuda.synchronize()
    assert torch.equal(_bits16(dk), _bits16(ref_dk)) and torch.equal(_bits16(dv), _bits16(ref_dv))
    wq, wk, wv = OA.backward(f["q"], f["k"], f["v"], f["do"], scale, causal)
    compare("dQ", dev_to_f64(dq), wq, bf16=True)
    compare("dK", dev_to_f64(dk), wk, bf16=True)
    compare("dV", dev_to_f64(dv), wv, bf16=True)


def test_stored_ds_rejects():
    q = torch.zeros((64, 2, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    small = torch.empty(U.attn_bwd_stored_ds_bytes(64, 2, True) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(U.UlyssesError) as e:
        U.attn_bwd_dkdv_store_ds(q, k, k, lse, q, lse, small)
    assert e.value.status == 5
    with pytest.raises(U.UlyssesError) as e:
        U.attn_bwd_dq_stored_ds(k, small, torch.empty_like(q))
    assert e.value.status == 5
    qf = q.float()
    big = torch.empty(U.attn_bwd_stored_ds_bytes(64, 2, True), dtype=torch.uint8, device="cuda")
    with pytest.raises(U.UlyssesError) as e:
        U.attn_bwd_dq_stored_ds(k.float(), big, qf)
    assert e.value.status == 3


@pytest.mark.timeout(600)
def test_stored_ds_qwen_64k_share():
    """The 64K share's rank 0 (8 q / 2 kv heads, causal): dQ on sampled rows against the oracle,
    dK/dV bit-identical to attn_bwd_dkdv (34.4 GB of stored dS)."""
    from tests.test_gpu_fullsize import _inputs
    cfg = W.WORKLOADS["qwen_64k"]
    print("case stored dS qwen_64k rank 0: generating", flush=True)
    shards, f = _inputs(cfg, 0)
    q, k, v, do = U.ulysses_pack_group([shards["q"], shards["k"], shards["v"]], 0) + [U.ulysses_pack(shards["do"], 0)]
    del shards
    dq, dk, dv, ref_dk, ref_dv = _stored_ds_bwd(q, k, v, do, cfg.scale, True)
    torch.cuda.synchronize()
    print("  GPU done", flush=True)
    assert torch.equal(_bits16(dk), _bits16(ref_dk)) and torch.equal(_bits16(dv), _bits16(ref_dv))
    rows = sample_rows(cfg.s)
    wq, _, _ = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, True, None, q_rows=rows,
                           kv_cols=np.zeros(0, int))
    compare("qwen_64k stored-dS dQ rows", dev_to_f64(dq[torch.as_tensor(rows, device="cuda")]), wq, bf16=True)
