"""Oracle for the local permutes on either side of Ulysses' two all-to-alls.

Test infrastructure only (see the package docstring).

Source: "Ulysses Sequence Parallelism: Training with Million-Token Contexts"
(agentlenshq.com), section "how Ulysses works", steps 1, 3 and 5: each of P GPUs
holds a local chunk of tokens with every head; the first all-to-all leaves each GPU
with every sequence position for a subset of heads; the second returns the output
to the sequence-sharded form. The tilnote.io commentary (section on what Ulysses
changes) describes the same swap: each GPU goes from a short piece of the sequence
with every head to the whole sequence with a slice of the heads.

Readings taken where the pages are silent:
  * rank p holds tokens [p*s_l, (p+1)*s_l) (contiguous local chunks);
  * rank r receives heads [r*H_l, (r+1)*H_l), H_l = H / P (contiguous head groups),
    which needs H divisible by P (the commentary's divisibility condition).

The permutes only move bits, so they work on raw element bits (uint16 for bf16,
uint32 for fp32) and a comparison against them is exact.
"""
import numpy as np


def pack(shards, rank, h0=None, nh=None):
    """Sequence shards -> one head shard (forward half of the first all-to-all).

    shards: list of P arrays [s_l, H, d]. Returns Y [P*s_l, nh, d] with
    Y[p*s_l + t, j, :] = shards[p][t, h0 + j, :].  By default h0 = rank*H/P and
    nh = H/P, the rank's own head slice; h0/nh select a sub-range of it (used by
    the headwise-chunked schedule)."""
    P = len(shards)
    s_l, H, d = shards[0].shape
    if H % P != 0:
        raise ValueError("head count must be divisible by the number of ranks")
    Hl = H // P
    if h0 is None:
        h0, nh = rank * Hl, Hl
    out = np.empty((P * s_l, nh, d), dtype=shards[0].dtype)
    for p in range(P):
        src = shards[p]
        for t in range(s_l):
            for j in range(nh):
                out[p * s_l + t, j, :] = src[t, h0 + j, :]
    return out


def unpack(y, rank, shards, h0=None):
    """Head shard -> sequence shards (the second all-to-all, and the backward of the first).

    y: [P*s_l, nh, d]. Returns copies of `shards` in which
    X_p[t, h0 + j, :] = y[p*s_l + t, j, :]; every other head is left as it was."""
    P = len(shards)
    s_l, H, d = shards[0].shape
    Hl = H // P
    nh = y.shape[1]
    if h0 is None:
        h0 = rank * Hl
    out = [np.array(x, copy=True) for x in shards]
    for p in range(P):
        for t in range(s_l):
            for j in range(nh):
                out[p][t, h0 + j, :] = y[p * s_l + t, j, :]
    return out


# ---------------------------------------------------------------------------------------
# The same exchange as a real all-to-all performs it: a send-side permute on every source
# rank and a receive-side permute on every destination rank, with the collective itself in
# between (it moves block r of rank p's send buffer to block p of rank r's receive buffer).
# Same sources as above; the comparison table on the first page also allows
# num_heads >= sp_size only, so a head count below P (the kv heads of a GQA model at large
# SP) is read as replication: rank r receives the one head floor(r * H / P), i.e. each head
# goes to P / H consecutive ranks (P divisible by H), and on the way back the gradient of a
# replicated head is the sum of its replicas' gradients (the chain rule over the ranks that
# read it), taken in float32 in rank order and rounded once to the element type.

def rank_heads(r, P, H):
    """(first head, head count) that rank r receives of H heads over P ranks."""
    if H % P == 0:
        return r * (H // P), H // P
    if P % H == 0:
        return r // (P // H), 1
    raise ValueError("head count must divide or be divisible by the number of ranks")


def send_pack(shard, P):
    """One source rank's sequence shard [s_l, H, d] -> its send buffer [P, s_l, H_l, d]:
    out[r, t, j, :] = shard[t, first(r) + j, :]."""
    s_l, H, d = shard.shape
    nh = rank_heads(0, P, H)[1]
    out = np.empty((P, s_l, nh, d), dtype=shard.dtype)
    for r in range(P):
        h0, _ = rank_heads(r, P, H)
        for t in range(s_l):
            for j in range(nh):
                out[r, t, j, :] = shard[t, h0 + j, :]
    return out


def _bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values; float32 bits (uint32) -> float32."""
    if bits.dtype == np.uint16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits.view(np.float32)


def f32_to_bf16_bits(x):
    """float32 values -> bf16 bit patterns, rounding to nearest, ties to even (finite inputs):
    add 0x7fff plus the lowest kept bit to the 32-bit pattern, then keep its upper half."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def recv_unpack(blocks, P, H):
    """One destination rank's receive buffer [P, s_l, H_l, d] (block p from source rank p)
    -> its sequence shard [s_l, H, d]: shard[t, h, :] = sum over the ranks r holding head h
    of blocks[r, t, h - first(r), :]. On raw bits: one holder is a copy of the bits; several
    (replicated heads) are summed in float32 in rank order and rounded once (bf16 bits:
    nearest even). Float64 values (not bits) are summed in float64."""
    _, s_l, nh, d = blocks.shape
    out = np.zeros((s_l, H, d), dtype=blocks.dtype)
    holders = [[r for r in range(P) if rank_heads(r, P, H)[0] <= h < sum(rank_heads(r, P, H))] for h in range(H)]
    for h in range(H):
        rs = holders[h]
        for t in range(s_l):
            if len(rs) == 1:
                r = rs[0]
                out[t, h, :] = blocks[r, t, h - rank_heads(r, P, H)[0], :]
                continue
            if blocks.dtype == np.float64:
                out[t, h, :] = sum(blocks[r, t, h - rank_heads(r, P, H)[0], :] for r in rs)
                continue
            acc = np.zeros(d, dtype=np.float32)
            for r in rs:
                acc = (acc + _bits_to_f32(blocks[r, t, h - rank_heads(r, P, H)[0], :])).astype(np.float32)
            out[t, h, :] = f32_to_bf16_bits(acc) if blocks.dtype == np.uint16 else acc.view(np.uint32)
    return out
