"""GPU parity of the send-side and receive-side permutes of a real all-to-all
(ulysses_send_pack / ulysses_recv_unpack), including kv heads replicated when there are fewer
than ranks.

The collective between them (block r of rank p's send buffer -> block p of rank r's receive
buffer) is played by the test with device copies. Checked: bit-exact equality with the oracle's
index loops (and its fp32 replica sums), the send + exchange path equal to ulysses_pack, and a
whole share with replicated kv heads -- every rank's attention forward and backward between the
permutes -- against the oracle on the unsharded tensors."""
import numpy as np
import pytest
import torch

import ulysses_sequence_parallelism_rank_amd as U
import workloads as W
from oracle import attention as OA
from oracle import permute as OP
from tests.helpers import LSE_ABS, compare, dev_to_f64, half_ulp_bf16, to_dev

pytestmark = pytest.mark.gpu


def _bits(rng, shape, dt):
    x = rng.standard_normal(shape).astype(np.float32)
    return W.to_bf16_bits(x) if dt == "bf16" else x.view(np.uint32)


def _host_bits(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy().view(
        np.uint16 if t.dtype == torch.bfloat16 else np.uint32)


def _exchange(bufs):
    P = len(bufs)
    return [torch.stack([bufs[p][r] for p in range(P)]) for r in range(P)]


@pytest.mark.parametrize("P,s_l,H,d,dt", [
    (4, 37, 8, 128, "bf16"), (4, 50, 2, 128, "bf16"), (8, 33, 1, 64, "bf16"), (8, 21, 2, 128, "bf16"),
    (2, 19, 4, 64, "f32"), (8, 16, 2, 64, "f32"), (1, 5, 3, 64, "bf16"), (64, 3, 8, 64, "bf16"),
])
def test_send_recv_bit_exact(P, s_l, H, d, dt):
    print(f"case P={P} s_l={s_l} H={H} d={d} {dt}", flush=True)
    rng = np.random.default_rng(P * 100 + H)
    shard = _bits(rng, (s_l, H, d), dt)
    got = U.ulysses_send_pack(to_dev(shard, dt), P)
    nh = OP.rank_heads(0, P, H)[1]
    blocks = _bits(rng, (P, s_l, nh, d), dt)
    back = U.ulysses_recv_unpack(to_dev(blocks, dt), H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host_bits(got), OP.send_pack(shard, P))
    np.testing.assert_array_equal(_host_bits(back), OP.recv_unpack(blocks, P, H))


@pytest.mark.parametrize("P,H", [(4, 32), (4, 8), (8, 64), (2, 2)])
def test_send_and_exchange_equal_pack(P, H):
    cfg = W.Config("exch", P=P, s_l=129, Hq=H, Hkv=H, d=128, dtype="bf16")
    shards = [to_dev(b, "bf16") for b in W.shards_of(W.gen_global(cfg, "q", seed=3), P)]
    recv = _exchange([U.ulysses_send_pack(x, P) for x in shards])
    for r in range(P):
        want = U.ulysses_pack(shards, r)
        assert torch.equal(recv[r].reshape(want.shape).view(torch.int16), want.view(torch.int16))
    # and the receive side inverts it: every rank's head shard back to the token owners
    heads = [U.ulysses_pack(shards, r).reshape(P, cfg.s_l, H // P, 128) for r in range(P)]
    back = _exchange(heads)
    for p in range(P):
        assert torch.equal(U.ulysses_recv_unpack(back[p], H).view(torch.int16), shards[p].view(torch.int16))
    torch.cuda.synchronize()


@pytest.mark.parametrize("P,s_l,Hq,Hkv", [(8, 96, 16, 2), (4, 160, 8, 2)])
def test_replicated_kv_share_matches_unsharded_oracle(P, s_l, Hq, Hkv):
    """Fewer kv heads than ranks: each rank receives its q heads and the one kv head they read,
    runs attention forward and backward (O's residual handed to the backward), and the
    gradients of a kv head held by P / Hkv ranks are summed on the way back."""
    print(f"case replicated kv P={P} s_l={s_l} Hq={Hq} Hkv={Hkv}", flush=True)
    cfg = W.Config("rep", P=P, s_l=s_l, Hq=Hq, Hkv=Hkv, d=128, dtype="bf16")
    glob = {n: W.gen_global(cfg, n, seed=9) for n in ("q", "k", "v", "do")}
    sh = {n: [to_dev(b, "bf16") for b in W.shards_of(g, P)] for n, g in glob.items()}
    recv = {n: _exchange([U.ulysses_send_pack(x, P) for x in sh[n]]) for n in sh}
    s, d = cfg.s, cfg.d
    outs = {n: [] for n in ("o", "dq", "dk", "dv")}
    lses = []
    for r in range(P):
        q, k, v, do = (recv[n][r].reshape(s, -1, d) for n in ("q", "k", "v", "do"))
        assert k.shape[1] == 1
        o_lo = U.new_o_lo(q)
        o, lse = U.attn_fwd(q, k, v, cfg.scale, True, o_lo=o_lo)
        dq, dk, dv = U.attn_bwd(q, k, v, o, lse, do, cfg.scale, True, o_lo=o_lo)
        for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
            outs[n].append(t.reshape(P, s_l, t.shape[1], d))
        lses.append(lse)
    back = {n: torch.cat([U.ulysses_recv_unpack(b, Hq if n in ("o", "dq") else Hkv)
                          for b in _exchange(outs[n])]) for n in outs}
    torch.cuda.synchronize()
    f = {n: W.bits_to_f64(g, "bf16") for n, g in glob.items()}
    wo, wl = OA.forward(f["q"], f["k"], f["v"], cfg.scale, True)
    wq, wk, wv = OA.backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, True)
    compare("replicated O", dev_to_f64(back["o"]), wo, bf16=True)
    compare("replicated LSE", torch.cat(lses).cpu().numpy(), wl, max_abs=LSE_ABS, rel_fro=1e-4)
    compare("replicated dQ", dev_to_f64(back["dq"]), wq, bf16=True)
    # a replicated kv head's gradient is the sum of P / Hkv partials, each rounded to bf16 by its
    # rank before the exchange: the storage allowance is half an ulp of each partial (from the
    # oracle's per-rank gradients) plus half an ulp of the rounded sum
    allow = {n: half_ulp_bf16(w) for n, w in (("dk", wk), ("dv", wv))}
    Hq_l, R = Hq // P, P // Hkv
    for r in range(P):
        g = r // R
        sl = lambda a, h0, n: a[:, h0:h0 + n]
        _, pk, pv = OA.backward(sl(f["q"], r * Hq_l, Hq_l), sl(f["k"], g, 1), sl(f["v"], g, 1),
                                sl(f["do"], r * Hq_l, Hq_l), cfg.scale, True)
        allow["dk"][:, g:g + 1] += half_ulp_bf16(pk)
        allow["dv"][:, g:g + 1] += half_ulp_bf16(pv)
    compare("replicated dK", dev_to_f64(back["dk"]), wk, allow=allow["dk"])
    compare("replicated dV", dev_to_f64(back["dv"]), wv, allow=allow["dv"])
