"""Oracle for the local attention of one head shard: plain masked softmax attention.

Test infrastructure only (see the package docstring).

What is computed, and where the pages fix it:
  * After the first all-to-all each GPU runs ordinary dense attention over the whole
    sequence for its heads ("Ulysses Sequence Parallelism: Training with
    Million-Token Contexts", section "how Ulysses works", step 4; tilnote.io
    commentary, section on what Ulysses changes: each GPU attends densely over the
    full sequence for its slice of heads).
  * FlashAttention computes the same attention with O(n) memory (same page,
    section on the long-sequence challenge), so the exact softmax result is the
    reference; no tiling or online softmax appears here.
  * Packing for SFT (same page, TRL SFTTrainer section) concatenates documents; the
    mask keeps attention inside each document.

Readings taken where the pages are silent:
  * S = scale * Q K^T with scale passed in (1/sqrt(d) in every workload);
  * causal self-attention over one sequence: key j is visible to row i iff j <= i;
  * packed documents: additionally lo(i) <= j, where lo(i) is the start of the
    document holding row i (cu_seqlens, block-diagonal causal);
  * grouped-query attention: q head h reads kv head h // G, G = Hq / Hkv;
  * LSE is the natural-log log-sum-exp of each row's visible scores;
  * the backward is the exact gradient of O w.r.t. Q, K, V contracted with dO.

All arithmetic is float64. Inputs are taken as given values (the callers pass the
bf16- or fp32-rounded inputs, upcast). Blocking over query rows only bounds memory:
every row is computed over its full key range.
"""
import numpy as np

ROW_BLOCK = 512


def doc_start(rows, cu_seqlens):
    """lo(i): first token of the document holding row i (0 when unpacked)."""
    rows = np.asarray(rows)
    if cu_seqlens is None:
        return np.zeros_like(rows)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    k = np.searchsorted(cu, rows, side="right") - 1
    return cu[k]


def allowed(rows, cols, causal, cu_seqlens):
    """Boolean [len(rows), len(cols)] visibility mask."""
    rows = np.asarray(rows)[:, None]
    cols = np.asarray(cols)[None, :]
    ok = np.ones((rows.shape[0], cols.shape[1]), dtype=bool)
    if causal:
        ok &= cols <= rows
    if cu_seqlens is not None:
        lo = doc_start(rows[:, 0], cu_seqlens)[:, None]
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        hi = cu[np.searchsorted(cu, rows[:, 0], side="right")][:, None]
        ok &= (cols >= lo) & (cols < hi)
    return ok


def _row_blocks(rows):
    for a in range(0, len(rows), ROW_BLOCK):
        yield rows[a:a + ROW_BLOCK]


def _key_range(block_rows, s, causal):
    # keys past the last row of a causal block are all masked; skipping them leaves
    # every visible score in place.
    return np.arange(int(block_rows.max()) + 1 if causal else s)


def forward(q, k, v, scale, causal=True, cu_seqlens=None, rows=None):
    """O and LSE of softmax attention.

    q [s, Hq, d], k, v [s, Hkv, d] (float64). Returns (o, lse) where o is
    [len(rows), Hq, d] and lse [Hq, len(rows)] for the requested rows (all rows by
    default), each computed exactly over its visible keys."""
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("q heads must be a multiple of kv heads")
    G = Hq // Hkv
    rows = np.arange(s) if rows is None else np.asarray(rows)
    o = np.zeros((len(rows), Hq, d))
    lse = np.zeros((Hq, len(rows)))
    for h in range(Hq):
        g = h // G
        pos = 0
        for br in _row_blocks(rows):
            keys = _key_range(br, s, causal)
            S = scale * (q[br, h, :] @ k[keys, g, :].T)
            S[~allowed(br, keys, causal, cu_seqlens)] = -np.inf
            m = S.max(axis=1)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            o[pos:pos + len(br), h, :] = (E @ v[keys, g, :]) / l[:, None]
            lse[h, pos:pos + len(br)] = m + np.log(l)
            pos += len(br)
    return o, lse


def rows_attending(keys, s, causal, cu_seqlens):
    """Every row i that can see at least one key of `keys` (exactly those rows): per
    document holding a key, its rows from the smallest such key (causal) or from the
    document start (noncausal) to the document end."""
    keys = np.asarray(keys)
    if cu_seqlens is None:
        return np.arange(int(keys.min()) if causal else 0, s)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    kdoc = np.searchsorted(cu, keys, side="right") - 1
    parts = []
    for doc in np.unique(kdoc):
        lo = int(keys[kdoc == doc].min()) if causal else int(cu[doc])
        parts.append(np.arange(lo, int(cu[doc + 1])))
    return np.concatenate(parts)


def backward(q, k, v, do, scale, causal=True, cu_seqlens=None, q_rows=None, kv_cols=None):
    """Gradients of O = softmax(scale Q K^T, masked) V contracted with dO.

    Returns (dq, dk, dv): dq [len(q_rows), Hq, d]; dk, dv [len(kv_cols), Hkv, d].
    For GQA the gradient of a kv head sums over the G q heads that read it.
    By default all rows and all keys are returned. With subsets, each returned
    value is still exact: every row that sees a requested key is included. dK_j and
    dV_j use only column j of P and dS, so row blocks holding no requested dQ row
    compute those columns alone (the forward pass still covers every key).

    Per row i of q head h (kv head g = h // G), with O_i and LSE_i from forward():
      P_ij  = exp(S_ij - LSE_i)  (0 where masked)
      D_i   = dO_i . O_i
      dP_ij = dO_i . V_j
      dS_ij = P_ij (dP_ij - D_i)
      dQ_i  = scale sum_j dS_ij K_j
      dV_j += sum_i P_ij dO_i,   dK_j += scale sum_i dS_ij Q_i."""
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    q_rows = np.arange(s) if q_rows is None else np.asarray(q_rows)
    kv_cols = np.arange(s) if kv_cols is None else np.asarray(kv_cols)
    need = rows_attending(kv_cols, s, causal, cu_seqlens) if len(kv_cols) else np.arange(0)
    rows = np.union1d(q_rows, need)
    col_pos = np.full(s, -1)
    col_pos[kv_cols] = np.arange(len(kv_cols))
    q_pos = np.full(s, -1)
    q_pos[q_rows] = np.arange(len(q_rows))

    o, lse = forward(q, k, v, scale, causal, cu_seqlens, rows=rows)
    dq = np.zeros((len(q_rows), Hq, d))
    dk = np.zeros((len(kv_cols), Hkv, d))
    dv = np.zeros((len(kv_cols), Hkv, d))
    for h in range(Hq):
        g = h // G
        pos = 0
        for br in _row_blocks(rows):
            n = len(br)
            sel = q_pos[br] >= 0
            keys = _key_range(br, s, causal)
            if not sel.any():
                # no dQ row in this block: only the requested key columns of P and dS are used
                keys = kv_cols[kv_cols < len(keys)]
                if len(keys) == 0:
                    pos += n
                    continue
            S = scale * (q[br, h, :] @ k[keys, g, :].T)
            mask = allowed(br, keys, causal, cu_seqlens)
            Pm = np.where(mask, np.exp(np.where(mask, S, 0.0) - lse[h, pos:pos + n][:, None]), 0.0)
            Dv = np.sum(do[br, h, :] * o[pos:pos + n, h, :], axis=1)
            dP = do[br, h, :] @ v[keys, g, :].T
            dS = Pm * (dP - Dv[:, None])
            if sel.any():
                dq[q_pos[br][sel], h, :] = scale * (dS[sel] @ k[keys, g, :])
            cols = col_pos[keys]
            csel = cols >= 0
            if csel.any():
                dv[cols[csel], g, :] += Pm[:, csel].T @ do[br, h, :]
                dk[cols[csel], g, :] += scale * (dS[:, csel].T @ q[br, h, :])
            pos += n
    return dq, dk, dv
