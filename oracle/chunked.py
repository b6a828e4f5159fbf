"""Oracle for the headwise-chunked (UPipe-style) forward and backward.

Test infrastructure only (see the package docstring).

Source: tilnote.io commentary, section on activation memory past a million tokens:
Untied Ulysses (UPipe) processes only some attention heads at a time to cut the
memory held by attention intermediates. The result per head is unchanged; only
which heads are resident at once differs. So each chunk runs the same three steps
as the unchunked layer (pack, attention, unpack) restricted to its heads.

Readings: chunks cover the rank's q heads in order, u heads
each, the last one smaller when u does not divide H_q/P; a chunk's kv heads are
those its q heads read (h // G). In the backward, the gradient of a kv head read by
several chunks is the sum of the chunks' contributions (the chain rule over the heads
that read it, exactly as in the unchunked GQA backward).
"""
import numpy as np

from . import attention, permute


def forward(q_shards, k_shards, v_shards, o_shards, rank, heads_per_chunk, scale,
            causal=True, cu_seqlens=None, to_f64=None, from_f64=None):
    """Chunked forward for rank `rank`.

    *_shards: lists of P raw-bit arrays [s_l, H, d]. to_f64 converts raw bits to
    float64 values; from_f64 converts float64 outputs back to raw bits of the
    element type. Returns (new o_shards, lse [Hq/P, s])."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    Hq_l, Hkv_l = Hq // P, Hkv // P
    G = Hq // Hkv
    s = P * s_l
    lse = np.zeros((Hq_l, s))
    out = [np.array(x, copy=True) for x in o_shards]
    for c0 in range(0, Hq_l, heads_per_chunk):
        c1 = min(c0 + heads_per_chunk, Hq_l)
        g0, g1 = c0 // G, (c1 - 1) // G + 1
        qc = permute.pack(q_shards, rank, h0=rank * Hq_l + c0, nh=c1 - c0)
        kc = permute.pack(k_shards, rank, h0=rank * Hkv_l + g0, nh=g1 - g0)
        vc = permute.pack(v_shards, rank, h0=rank * Hkv_l + g0, nh=g1 - g0)
        qf, kf, vf = to_f64(qc), to_f64(kc), to_f64(vc)
        oc = np.zeros((s, c1 - c0, d))
        for j in range(c1 - c0):
            g = (c0 + j) // G - g0
            o1, l1 = attention.forward(qf[:, j:j + 1], kf[:, g:g + 1], vf[:, g:g + 1], scale,
                                       causal, cu_seqlens)
            oc[:, j] = o1[:, 0]
            lse[c0 + j] = l1[0]
        out = permute.unpack(from_f64(oc), rank, out, h0=rank * Hq_l + c0)
    return out, lse


def workspace_elems(s, Hq_l, G, d, heads_per_chunk):
    """Elements of the chunk buffers: Q and O chunks [s, u, d] plus K and V chunks
    [s, n_kv, d], n_kv = the most kv heads any chunk spans."""
    u = min(heads_per_chunk, Hq_l)
    n_kv = 0
    for c0 in range(0, Hq_l, u):
        c1 = min(c0 + u, Hq_l)
        n_kv = max(n_kv, (c1 - 1) // G - c0 // G + 1)
    return 2 * s * u * d + 2 * s * n_kv * d


def backward(q_shards, k_shards, v_shards, do_shards, rank, heads_per_chunk, scale, causal=True,
             cu_seqlens=None, to_f64=None):
    """Chunked backward for rank `rank` (the UPipe schedule applied to training).

    Same readings as forward(): chunks of u local q heads in order, each with the kv heads
    its q heads read. Per chunk, each q head's gradients come from the plain backward of
    that head with its kv head; the dK/dV of a kv head are summed over the chunks (and
    heads) that read it. Returns float64 (dq [s, Hq/P, d], dk [s, Hkv/P, d], dv)."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    Hq_l, Hkv_l = Hq // P, Hkv // P
    G = Hq // Hkv
    s = P * s_l
    dq = np.zeros((s, Hq_l, d))
    dk = np.zeros((s, Hkv_l, d))
    dv = np.zeros((s, Hkv_l, d))
    for c0 in range(0, Hq_l, heads_per_chunk):
        c1 = min(c0 + heads_per_chunk, Hq_l)
        g0, g1 = c0 // G, (c1 - 1) // G + 1
        qc = to_f64(permute.pack(q_shards, rank, h0=rank * Hq_l + c0, nh=c1 - c0))
        gc = to_f64(permute.pack(do_shards, rank, h0=rank * Hq_l + c0, nh=c1 - c0))
        kc = to_f64(permute.pack(k_shards, rank, h0=rank * Hkv_l + g0, nh=g1 - g0))
        vc = to_f64(permute.pack(v_shards, rank, h0=rank * Hkv_l + g0, nh=g1 - g0))
        for j in range(c1 - c0):
            g = (c0 + j) // G - g0
            q1, k1, v1 = attention.backward(qc[:, j:j + 1], kc[:, g:g + 1], vc[:, g:g + 1], gc[:, j:j + 1],
                                            scale, causal, cu_seqlens)
            dq[:, c0 + j] = q1[:, 0]
            dk[:, g0 + g] += k1[:, 0]
            dv[:, g0 + g] += v1[:, 0]
    return dq, dk, dv
