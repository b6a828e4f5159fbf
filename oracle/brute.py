"""Scalar-loop attention for tiny inputs: an independent check of oracle.attention.

Test infrastructure only (see the package docstring).

This is the textbook definition written one score at a time with math.exp, no
matrix routines and no -inf arithmetic: for each row, gather the visible keys
(causal j <= i; packed: same document), take the softmax of their scaled dot
products and average the values. It follows the same pages as oracle.attention
("how Ulysses works", step 4: dense attention over the full sequence per head).
Intended for s <= ~16, d <= ~8.
"""
import math


def _visible(i, j, causal, cu):
    if causal and j > i:
        return False
    if cu is not None:
        for a, b in zip(cu[:-1], cu[1:]):
            if a <= i < b:
                return a <= j < b
    return True


def forward(q, k, v, scale, causal=True, cu=None):
    """q: nested lists/arrays [s][Hq][d]; k, v [s][Hkv][d]. Returns (o[s][Hq][d], lse[Hq][s])."""
    s, Hq, d = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    o = [[[0.0] * d for _ in range(Hq)] for _ in range(s)]
    lse = [[0.0] * s for _ in range(Hq)]
    for h in range(Hq):
        g = h // G
        for i in range(s):
            keys = [j for j in range(s) if _visible(i, j, causal, cu)]
            sc = []
            for j in keys:
                dot = 0.0
                for x in range(d):
                    dot += float(q[i][h][x]) * float(k[j][g][x])
                sc.append(scale * dot)
            mx = max(sc)
            w = [math.exp(t - mx) for t in sc]
            tot = sum(w)
            for x in range(d):
                acc = 0.0
                for wj, j in zip(w, keys):
                    acc += wj * float(v[j][g][x])
                o[i][h][x] = acc / tot
            lse[h][i] = mx + math.log(tot)
    return o, lse


def loss(q, k, v, do, scale, causal=True, cu=None):
    """L = sum over rows, heads and dims of dO * O; its gradient is the attention backward."""
    o, _ = forward(q, k, v, scale, causal, cu)
    s, Hq, d = len(o), len(o[0]), len(o[0][0])
    return sum(float(do[i][h][x]) * o[i][h][x] for i in range(s) for h in range(Hq) for x in range(d))


def finite_diff_grads(q, k, v, do, scale, causal=True, cu=None, step=1e-5):
    """Central differences of loss() w.r.t. every element of q, k and v (numpy float64 arrays)."""
    import numpy as np
    grads = []
    for arr in (q, k, v):
        g = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + step
            lp = loss(q, k, v, do, scale, causal, cu)
            arr[idx] = old - step
            lm = loss(q, k, v, do, scale, causal, cu)
            arr[idx] = old
            g[idx] = (lp - lm) / (2 * step)
        grads.append(g)
    return grads
