"""Oracle for Ring Attention over P ranks, the comparison workload of the pages.

Test infrastructure only (see the package docstring).

Source: "Ulysses Sequence Parallelism: Training with Million-Token Contexts"
(agentlenshq.com), sections on communication complexity and on Ulysses compared with Ring
Attention: Ring Attention keeps every rank's query block in place and passes the key/value
blocks from rank to rank around a ring (point-to-point), each rank attending to each block as
it arrives; the partial results are combined, so the output equals attention over the whole
sequence.

Readings taken where the pages are silent:
  * rank p holds tokens [p*s_l, (p+1)*s_l) of Q, K and V with every head (the same
    contiguous chunks as for Ulysses);
  * at hop i rank p holds the K/V block of rank (p - i) mod P;
  * causal: a block from a later rank is entirely masked and skipped, the rank's own block
    (hop 0) is causal inside the block, earlier blocks are fully visible;
  * the partial outputs are combined by their log-sum-exps: with per-hop (O_i, LSE_i),
    LSE = log sum_i exp(LSE_i) and O = sum_i exp(LSE_i - LSE) O_i (the softmax over the
    union of the key blocks, regrouped by block);
  * the backward runs the same hops with the merged LSE and delta = dO . O: rank p's dQ is the
    sum over its hops, and the dK/dV of block b is the sum of the contributions of every rank
    that attended to it (in a real ring they travel with the K/V block).

Arithmetic is float64, on the attention oracle (oracle.attention), which is pinned on its own.
"""
import numpy as np

from . import attention


def hops(P, rank, causal=True):
    """Source blocks rank `rank` attends to, in ring order: (p - i) mod P for hop i, skipping
    blocks a causal mask hides entirely."""
    out = []
    for i in range(P):
        src = (rank - i) % P
        if causal and src > rank:
            continue
        out.append(src)
    return out


def partial(q, k, v, scale, diagonal, causal=True):
    """Attention of a query block against one key/value block: (O_i, LSE_i). The diagonal
    block is causal inside the block when `causal`; other visible blocks are unmasked."""
    return attention.forward(q, k, v, scale, causal=(causal and diagonal))


def merge(parts):
    """Combine [(O_i [s_l, H, d], LSE_i [H, s_l]), ...] into (O, LSE)."""
    lses = np.stack([l for _, l in parts])                 # [n, H, s_l]
    m = lses.max(axis=0)
    w = np.exp(lses - m)                                   # [n, H, s_l]
    tot = w.sum(axis=0)
    lse = m + np.log(tot)
    o = sum(o_i * (w_i / tot).T[:, :, None] for (o_i, _), w_i in zip(parts, w))
    return o, lse


def forward(q_shards, k_shards, v_shards, rank, scale, causal=True):
    """Rank `rank`'s output block O_p [s_l, Hq, d] and LSE_p [Hq, s_l]."""
    P = len(q_shards)
    parts = [partial(q_shards[rank], k_shards[src], v_shards[src], scale, src == rank, causal)
             for src in hops(P, rank, causal)]
    return merge(parts)


def backward(q_shards, k_shards, v_shards, do_shards, rank, scale, causal=True):
    """Rank `rank`'s dQ_p and its contributions to every block's dK/dV: (dq [s_l, Hq, d],
    {src: (dk_src, dv_src)}), each contribution the gradient of rank p's rows against block src,
    with P from the merged LSE and delta from the merged O."""
    P = len(q_shards)
    o, lse = forward(q_shards, k_shards, v_shards, rank, scale, causal)
    q, do = q_shards[rank], do_shards[rank]
    s_l, Hq, d = q.shape
    G = Hq // k_shards[0].shape[1]
    delta = (do * o).sum(axis=2).T                         # [Hq, s_l]
    dq = np.zeros_like(q)
    contrib = {}
    rows = np.arange(s_l)
    for src in hops(P, rank, causal):
        k, v = k_shards[src], v_shards[src]
        diag = src == rank
        mask = attention.allowed(rows, rows, causal and diag, None)
        dk, dv = np.zeros_like(k), np.zeros_like(v)
        for h in range(Hq):
            g = h // G
            S = scale * (q[:, h] @ k[:, g].T)
            Pm = np.where(mask, np.exp(np.where(mask, S, 0.0) - lse[h][:, None]), 0.0)
            dS = Pm * (do[:, h] @ v[:, g].T - delta[h][:, None])
            dq[:, h] += scale * (dS @ k[:, g])
            dk[:, g] += scale * (dS.T @ q[:, h])
            dv[:, g] += Pm.T @ do[:, h]
        contrib[src] = (dk, dv)
    return dq, contrib
