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
