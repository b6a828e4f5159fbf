"""Python binding of libulysses: one GPU's share of a Ulysses attention layer on MI355X.

Argument marshalling only. Every step runs in the HIP kernels of libulysses.so (built
in-tree by `_build.py`); torch supplies device memory and the current stream. If the
library is missing, every call raises: there is no fallback path.

The names follow the C ABI in include/ulysses.h:
  ulysses_pack, ulysses_unpack        -- local halves of the two all-to-alls
  ulysses_pack_group, ulysses_unpack_group -- the same for up to three tensors in one launch
  attn_fwd, attn_bwd                  -- attention of one head shard
  attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq -- the phases of attn_bwd
  attn_fwd_chunked                    -- the UPipe headwise-chunked forward
  attn_bwd_chunked                    -- its backward
  attn_fwd_shards, attn_bwd_shards    -- forward / backward reading and writing the sequence shards
  attn_bwd_dkdv_store_ds, attn_bwd_dq_stored_ds -- the backward with dS stored once (opt-in)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libulysses.so")

ULY_BF16, ULY_F32 = 0, 1
STATUS = {0: "ULY_OK", 1: "ULY_ERR_NULL", 2: "ULY_ERR_SHAPE", 3: "ULY_ERR_UNSUPPORTED",
          4: "ULY_ERR_ALIGN", 5: "ULY_ERR_WORKSPACE", 6: "ULY_ERR_HIP"}
MAX_RANKS = 64

_lib = None

_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_vpp = ctypes.POINTER(ctypes.c_void_p)
_szp = ctypes.POINTER(ctypes.c_size_t)
_i32p = ctypes.POINTER(ctypes.c_int)
PERM_GROUP_MAX = 3

SIGNATURES = {
    "uly_status_string": (ctypes.c_char_p, [_i32]),
    "uly_abi_version": (_i32, []),
    "ulysses_pack": (_i32, [_vpp, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp]),
    "ulysses_unpack": (_i32, [_vp, _i32, _i32, _i64, _i32, _i32, _i32, _vpp, _vp]),
    "ulysses_pack_group": (_i32, [_i32, _vpp, _i32p, _vpp, _i32, _i32, _i64, _i32, _i32, _vp]),
    "ulysses_unpack_group": (_i32, [_i32, _vpp, _i32p, _vpp, _i32, _i32, _i64, _i32, _i32, _vp]),
    "attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp]),
    "attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                        _vp, _i32, _vp, _szp, _vp]),
    "attn_bwd_workspace_bytes": (_sz, [_i64, _i32]),
    "attn_bwd_preprocess": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp]),
    "attn_bwd_dkdv": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                             _vp, _i32, _vp]),
    "attn_bwd_dq": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                           _vp, _i32, _vp]),
    "attn_fwd_chunked": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                _i32, _vp, _i32, _i32, _vp, _szp, _vp]),
    "attn_fwd_chunked_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "attn_bwd_chunked": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vpp, _vpp, _vpp, _vpp, _i32, _i32, _i64, _i32,
                                _i32, _i32, _i32, _f32, _i32, _vp, _i32, _i32, _vp, _szp, _vp]),
    "attn_bwd_chunked_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "attn_fwd_shards": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                               _i32, _vp, _i32, _vp]),
    "uly_mfma_probe": (_i32, [_i32, _i32, _vp, _vp, _vp]),
    "attn_bwd_stored_ds_bytes": (_sz, [_i64, _i32, _i32]),
    "attn_bwd_dkdv_store_ds": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i32, _i32, _i32,
                                      _i32, _f32, _i32, _vp]),
    "attn_bwd_dq_stored_ds": (_i32, [_vp, _vp, _sz, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "attn_bwd_shards": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vpp, _vpp, _vpp, _vpp, _i32, _i32, _i64, _i32,
                               _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _szp, _vp]),
}


class UlyssesError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def lib():
    """Load libulysses.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libulysses.so not built at {LIB_PATH}; run "
                               "`python -m ulysses_sequence_parallelism_rank_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise UlyssesError(name, st)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return ULY_BF16
    if t.dtype == torch.float32:
        return ULY_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _ptrs(ts):
    arr = (ctypes.c_void_p * len(ts))(*[_dev(t) for t in ts])
    return ctypes.cast(arr, _vpp), arr


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, 0
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    return _dev(cu_seqlens), cu_seqlens.numel() - 1


def ulysses_pack(shards, rank, out=None):
    """P sequence shards [s_l, H, d] -> this rank's head shard [P*s_l, H/P, d]."""
    P = len(shards)
    s_l, H, d = shards[0].shape
    if out is None:
        out = torch.empty((P * s_l, H // P, d), dtype=shards[0].dtype, device=shards[0].device)
    pp, _keep = _ptrs(shards)
    _call("ulysses_pack", pp, P, rank, s_l, H, d, _dtype(shards[0]), _dev(out), _stream())
    return out


def ulysses_unpack(y, rank, shards):
    """Head shard [P*s_l, H/P, d] -> head slice `rank` of the P shards [s_l, H, d] (in place)."""
    P = len(shards)
    s_l, H, d = shards[0].shape
    pp, _keep = _ptrs(shards)
    _call("ulysses_unpack", _dev(y), P, rank, s_l, H, d, _dtype(y), pp, _stream())
    return shards


def _group_args(tensor_lists):
    """Host arrays for the grouped permutes: one array of P device pointers per tensor, an
    array of those arrays, and the global head counts."""
    arrays = [_ptrs(ts) for ts in tensor_lists]
    outer = (ctypes.c_void_p * len(arrays))(*[ctypes.cast(a, ctypes.c_void_p).value for a, _ in arrays])
    heads = (ctypes.c_int * len(tensor_lists))(*[ts[0].shape[1] for ts in tensor_lists])
    return ctypes.cast(outer, _vpp), ctypes.cast(heads, _i32p), (arrays, outer, heads)


def ulysses_pack_group(shard_lists, rank, outs=None):
    """Several tensors' P sequence shards [s_l, H_i, d] -> their head shards [P*s_l, H_i/P, d],
    in one launch (the Q/K/V of the forward exchange)."""
    n = len(shard_lists)
    P = len(shard_lists[0])
    s_l, _, d = shard_lists[0][0].shape
    if outs is None:
        outs = [torch.empty((P * s_l, sh[0].shape[1] // P, d), dtype=sh[0].dtype, device=sh[0].device)
                for sh in shard_lists]
    pp, hh, _keep = _group_args(shard_lists)
    op, _keep2 = _ptrs(outs)
    _call("ulysses_pack_group", n, pp, hh, op, P, rank, s_l, d, _dtype(outs[0]), _stream())
    return outs


def ulysses_unpack_group(ys, rank, shard_lists):
    """Several head shards [P*s_l, H_i/P, d] -> head slice `rank` of their P shards, in one launch
    (the dQ/dK/dV of the backward exchange)."""
    n = len(ys)
    P = len(shard_lists[0])
    s_l, _, d = shard_lists[0][0].shape
    pp, hh, _keep = _group_args(shard_lists)
    yp, _keep2 = _ptrs(ys)
    _call("ulysses_unpack_group", n, yp, hh, pp, P, rank, s_l, d, _dtype(ys[0]), _stream())
    return shard_lists


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def attn_fwd(q, k, v, scale=None, causal=True, cu_seqlens=None, out=None, lse=None):
    """q [s, Hq, d], k, v [s, Hkv, d] -> (o [s, Hq, d], lse [Hq, s] fp32)."""
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((Hq, s), dtype=torch.float32, device=q.device)
    cu, nd = _cu(cu_seqlens)
    _call("attn_fwd", _dev(q), _dev(k), _dev(v), _dev(o), _dev(lse), s, Hq, Hkv, d, _dtype(q),
          _default_scale(d, scale), int(causal), cu, nd, _stream())
    return o, lse


def attn_bwd_workspace_bytes(s, Hq):
    return int(lib().attn_bwd_workspace_bytes(s, Hq))


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=True, cu_seqlens=None, workspace=None,
             dq=None, dk=None, dv=None):
    """Gradients (dq, dk, dv) of the attention forward, given its o and lse and dout."""
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_bytes(s, Hq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens)
    _call("attn_bwd", _dev(q), _dev(k), _dev(v), _dev(o), _dev(lse), _dev(dout), _dev(dq), _dev(dk), _dev(dv),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, _dev(workspace),
          ctypes.byref(cap), _stream())
    return dq, dk, dv


def attn_bwd_preprocess(o, dout, delta=None):
    s, Hq, d = o.shape
    if delta is None:
        delta = torch.empty((Hq, s), dtype=torch.float32, device=o.device)
    _call("attn_bwd_preprocess", _dev(o), _dev(dout), _dev(delta), s, Hq, d, _dtype(o), _stream())
    return delta


def attn_bwd_dkdv(q, k, v, lse, dout, delta, scale=None, causal=True, cu_seqlens=None, dk=None, dv=None):
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    cu, nd = _cu(cu_seqlens)
    _call("attn_bwd_dkdv", _dev(q), _dev(k), _dev(v), _dev(lse), _dev(dout), _dev(delta), _dev(dk), _dev(dv),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, _stream())
    return dk, dv


def attn_bwd_stored_ds_bytes(s, Hq, causal=True):
    """Bytes of the dS buffer the stored-dS backward needs (s tokens, Hq local q heads)."""
    return int(lib().attn_bwd_stored_ds_bytes(s, Hq, int(causal)))


def attn_bwd_dkdv_store_ds(q, k, v, lse, dout, delta, ds, scale=None, causal=True, dk=None, dv=None):
    """attn_bwd_dkdv that also writes dS into `ds` (a uint8 device tensor of at least
    attn_bwd_stored_ds_bytes bytes) for attn_bwd_dq_stored_ds."""
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _call("attn_bwd_dkdv_store_ds", _dev(q), _dev(k), _dev(v), _dev(lse), _dev(dout), _dev(delta), _dev(dk),
          _dev(dv), _dev(ds), ds.numel() * ds.element_size(), s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale),
          int(causal), _stream())
    return dk, dv


def attn_bwd_dq_stored_ds(k, ds, dq, scale=None, causal=True):
    """dQ [s, Hq, d] (written into dq) from the dS that attn_bwd_dkdv_store_ds stored."""
    s, Hq, d = dq.shape
    Hkv = k.shape[1]
    _call("attn_bwd_dq_stored_ds", _dev(k), _dev(ds), ds.numel() * ds.element_size(), _dev(dq), s, Hq, Hkv, d,
          _dtype(dq), _default_scale(d, scale), int(causal), _stream())
    return dq


def attn_bwd_dq(q, k, v, lse, dout, delta, scale=None, causal=True, cu_seqlens=None, dq=None):
    s, Hq, d = q.shape
    Hkv = k.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    cu, nd = _cu(cu_seqlens)
    _call("attn_bwd_dq", _dev(q), _dev(k), _dev(v), _dev(lse), _dev(dout), _dev(delta), _dev(dq),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, _stream())
    return dq


def attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk):
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    return int(lib().attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk))


def attn_fwd_chunked(q_shards, k_shards, v_shards, o_shards, rank, heads_per_chunk, scale=None,
                     causal=True, cu_seqlens=None, workspace=None, lse=None):
    """UPipe forward of rank `rank`: writes this rank's heads of o_shards; returns lse [Hq/P, s]."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    s = P * s_l
    if lse is None:
        lse = torch.empty((Hq // P, s), dtype=torch.float32, device=q_shards[0].device)
    need = attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, _dtype(q_shards[0]), heads_per_chunk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_shards[0].device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    qp, k1 = _ptrs(q_shards)
    kp, k2 = _ptrs(k_shards)
    vp, k3 = _ptrs(v_shards)
    op, k4 = _ptrs(o_shards)
    cu, nd = _cu(cu_seqlens)
    _call("attn_fwd_chunked", qp, kp, vp, op, _dev(lse), P, rank, s_l, Hq, Hkv, d, _dtype(q_shards[0]),
          _default_scale(d, scale), int(causal), cu, nd, heads_per_chunk, _dev(workspace), ctypes.byref(cap),
          _stream())
    return lse


def attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk):
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    return int(lib().attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk))


def attn_bwd_chunked(q_shards, k_shards, v_shards, o_shards, lse, do_shards, dq_shards, dk_shards, dv_shards,
                     rank, heads_per_chunk, scale=None, causal=True, cu_seqlens=None, workspace=None):
    """UPipe backward of rank `rank`: writes this rank's heads of dq_shards, dk_shards, dv_shards."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    dt = _dtype(q_shards[0])
    need = attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_shards[0].device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards, dk_shards, dv_shards)]
    qp, kp, vp, op, gp, dqp, dkp, dvp = (k[0] for k in keep)
    cu, nd = _cu(cu_seqlens)
    _call("attn_bwd_chunked", qp, kp, vp, op, _dev(lse), gp, dqp, dkp, dvp, P, rank, s_l, Hq, Hkv, d, dt,
          _default_scale(d, scale), int(causal), cu, nd, heads_per_chunk, _dev(workspace), ctypes.byref(cap),
          _stream())
    return dq_shards, dk_shards, dv_shards


def attn_fwd_shards(q_shards, k_shards, v_shards, o_shards, rank, scale=None, causal=True, cu_seqlens=None,
                    lse=None):
    """Forward of rank `rank` straight from the sequence shards into head slice `rank` of
    o_shards (no head-shard buffers); returns the LSE [Hq/P, s]."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    if lse is None:
        lse = torch.empty((Hq // P, P * s_l), dtype=torch.float32, device=q_shards[0].device)
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards)]
    qp, kp, vp, op = (k[0] for k in keep)
    cu, nd = _cu(cu_seqlens)
    _call("attn_fwd_shards", qp, kp, vp, op, _dev(lse), P, rank, s_l, Hq, Hkv, d, _dtype(q_shards[0]),
          _default_scale(d, scale), int(causal), cu, nd, _stream())
    return lse


def attn_bwd_shards(q_shards, k_shards, v_shards, o_shards, lse, do_shards, dq_shards, dk_shards, dv_shards,
                    rank, scale=None, causal=True, cu_seqlens=None, workspace=None):
    """Backward of rank `rank` straight from the sequence shards into head slice `rank` of
    the dq / dk / dv shards."""
    P = len(q_shards)
    s_l, Hq, d = q_shards[0].shape
    Hkv = k_shards[0].shape[1]
    need = attn_bwd_workspace_bytes(P * s_l, Hq // P)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_shards[0].device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards, dk_shards, dv_shards)]
    qp, kp, vp, op, gp, dqp, dkp, dvp = (k[0] for k in keep)
    cu, nd = _cu(cu_seqlens)
    _call("attn_bwd_shards", qp, kp, vp, op, _dev(lse), gp, dqp, dkp, dvp, P, rank, s_l, Hq, Hkv, d,
          _dtype(q_shards[0]), _default_scale(d, scale), int(causal), cu, nd, _dev(workspace), ctypes.byref(cap),
          _stream())
    return dq_shards, dk_shards, dv_shards


def mfma_probe(iters=20000, blocks=512):
    """Practical bf16 MFMA ceiling and sustained clock: returns (tflops, clock_mhz), timed
    with events on the current stream."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    _call("uly_mfma_probe", 2, blocks, _dev(sink), _dev(clocks), _stream())  # warm-up
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    _call("uly_mfma_probe", iters, blocks, _dev(sink), _dev(clocks), _stream())
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    cyc, ref = (int(x) for x in clocks.cpu())
    flops = float(blocks) * 4 * iters * 4 * 32768
    return flops / (ms * 1e-3) / 1e12, (cyc / ref * 100.0 if ref > 0 else None)
