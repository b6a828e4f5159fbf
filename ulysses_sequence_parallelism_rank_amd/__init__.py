"""Python binding of libulysses: one GPU's share of a Ulysses attention layer on MI355X.

Argument marshalling only. Every step runs in the HIP kernels of libulysses.so (built
in-tree by `_build.py`); torch supplies device memory and the current stream. If the
library is missing, every call raises: there is no fallback path.

The names follow the C ABI in include/ulysses.h:
  ulysses_pack, ulysses_unpack        -- local halves of the two all-to-alls
  ulysses_pack_group, ulysses_unpack_group -- the same for up to three tensors in one launch
  ulysses_send_pack, ulysses_recv_unpack -- one rank's send-side / receive-side permutes of a
                                        real all-to-all (kv heads replicated when fewer than ranks)
  attn_fwd, attn_bwd                  -- attention of one head shard
  attn_bwd_preprocess, attn_bwd_dkdv, attn_bwd_dq -- the phases of attn_bwd
  attn_fwd_chunked                    -- the UPipe headwise-chunked forward
  attn_bwd_chunked                    -- its backward
  attn_fwd_shards, attn_bwd_shards    -- forward / backward reading and writing the sequence shards
  ring_attn_fwd, ring_attn_bwd        -- Ring Attention over the P ranks (the comparison workload)

Every tensor's shape, dtype and device are checked here before the C call (the C side
checks sizes and alignment but cannot see a tensor's extent). `o_lo` arguments take the
forward's bf16 rounding residual of O ([s, Hq_l, d] bf16, see include/ulysses.h);
`new_o_lo(q)` allocates one.
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
    "ulysses_send_pack": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp]),
    "ulysses_recv_unpack": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp]),
    "ulysses_pack_group": (_i32, [_i32, _vpp, _i32p, _vpp, _i32, _i32, _i64, _i32, _i32, _vp]),
    "ulysses_unpack_group": (_i32, [_i32, _vpp, _i32p, _vpp, _i32, _i32, _i64, _i32, _i32, _vp]),
    "attn_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _sz,
                        _vp]),
    "attn_fwd_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "attn_bwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                        _vp, _i32, _vp, _szp, _vp]),
    "attn_bwd_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "attn_bwd_dkdv_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "attn_bwd_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32,
                                _i32, _vp, _i32, _vp]),
    "attn_bwd_preprocess": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp]),
    "attn_bwd_dkdv": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                             _vp, _i32, _vp, _sz, _vp]),
    "attn_bwd_dq": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                           _vp, _i32, _vp, _sz, _vp]),
    "attn_bwd_dq_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "attn_fwd_chunked": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                _i32, _vp, _i32, _i32, _vp, _szp, _vp]),
    "attn_fwd_chunked_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "attn_bwd_chunked": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vp, _vpp, _vpp, _vpp, _vpp, _i32, _i32, _i64, _i32,
                                _i32, _i32, _i32, _f32, _i32, _vp, _i32, _i32, _vp, _szp, _vp]),
    "attn_bwd_chunked_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "attn_fwd_shards": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _f32,
                               _i32, _vp, _i32, _vp, _sz, _vp]),
    "attn_bwd_shards": (_i32, [_vpp, _vpp, _vpp, _vpp, _vp, _vp, _vpp, _vpp, _vpp, _vpp, _i32, _i32, _i64, _i32,
                               _i32, _i32, _i32, _f32, _i32, _vp, _i32, _vp, _szp, _vp]),
    "ring_attn_fwd_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "ring_attn_bwd_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "ring_attn_fwd": (_i32, [_vpp, _vpp, _vpp, _vp, _vp, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _i32, _f32, _i32,
                             _vp, _szp, _vp]),
    "ring_attn_bwd": (_i32, [_vpp, _vpp, _vpp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vpp, _vpp, _i32, _i32, _i64, _i32,
                             _i32, _i32, _i32, _f32, _i32, _vp, _szp, _vp]),
    "uly_mfma_probe": (_i32, [_i32, _i32, _vp, _vp, _vp]),
    "uly_mix_probe": (_i32, [_i32, _i32, _i32, _vp, _vp]),
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


def _shape(t, name, shape, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _need(t, name, shape, dtype, device=None):
    """Check a tensor argument before its pointer crosses the boundary."""
    _shape(t, name, shape, dtype)
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    return _dev(t)


def _opt(t, name, shape, dtype, device=None):
    return None if t is None else _need(t, name, shape, dtype, device)


def _same(ts, name):
    """A list of shards: equal shapes, dtypes and devices; returns the first."""
    if len(ts) < 1:
        raise ValueError(f"{name}: no shards")
    for i, t in enumerate(ts):
        _shape(t, f"{name}[{i}]", ts[0].shape, ts[0].dtype)
    for i, t in enumerate(ts):
        _need(t, f"{name}[{i}]", ts[0].shape, ts[0].dtype, ts[0].device)
    return ts[0]


def _ptrs(ts):
    arr = (ctypes.c_void_p * len(ts))(*[_dev(t) for t in ts])
    return ctypes.cast(arr, _vpp), arr


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _cu(cu_seqlens, device=None):
    if cu_seqlens is None:
        return None, 0
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with at least two entries")
    if device is not None and cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be on the tensors' device")
    return _dev(cu_seqlens), cu_seqlens.numel() - 1


def new_o_lo(q, Hq_l=None):
    """An O-residual buffer for q [s, Hq, d] (or for Hq_l local heads of sequence shards)."""
    s, Hq, d = q.shape
    return torch.empty((s, Hq if Hq_l is None else Hq_l, d), dtype=torch.bfloat16, device=q.device)


def ulysses_pack(shards, rank, out=None):
    """P sequence shards [s_l, H, d] -> this rank's head shard [P*s_l, H/P, d]."""
    P = len(shards)
    x = _same(shards, "shards")
    s_l, H, d = x.shape
    if out is None:
        out = torch.empty((P * s_l, H // P, d), dtype=x.dtype, device=x.device)
    _need(out, "out", (P * s_l, H // P, d), x.dtype, x.device)
    pp, _keep = _ptrs(shards)
    _call("ulysses_pack", pp, P, rank, s_l, H, d, _dtype(x), _dev(out), _stream())
    return out


def ulysses_unpack(y, rank, shards):
    """Head shard [P*s_l, H/P, d] -> head slice `rank` of the P shards [s_l, H, d] (in place)."""
    P = len(shards)
    x = _same(shards, "shards")
    s_l, H, d = x.shape
    _need(y, "y", (P * s_l, H // P, d), x.dtype, x.device)
    pp, _keep = _ptrs(shards)
    _call("ulysses_unpack", _dev(y), P, rank, s_l, H, d, _dtype(y), pp, _stream())
    return shards


def rank_heads(r, P, H):
    """(first head, count) rank r receives of H heads over P ranks (replicated when H < P)."""
    return (r * H // P, H // P) if H % P == 0 else (r // (P // H), 1)


def ulysses_send_pack(shard, P, out=None):
    """One rank's sequence shard [s_l, H, d] -> its all-to-all send buffer [P, s_l, H_l, d]."""
    s_l, H, d = shard.shape
    nh = rank_heads(0, P, H)[1]
    if out is None:
        out = torch.empty((P, s_l, nh, d), dtype=shard.dtype, device=shard.device)
    _need(out, "out", (P, s_l, nh, d), shard.dtype, shard.device)
    _call("ulysses_send_pack", _dev(shard), P, s_l, H, d, _dtype(shard), _dev(out), _stream())
    return out


def ulysses_recv_unpack(buf, H, shard=None):
    """One rank's all-to-all receive buffer [P, s_l, H_l, d] -> its sequence shard [s_l, H, d]
    (replicated heads summed over their ranks)."""
    P, s_l, nh, d = buf.shape
    if shard is None:
        shard = torch.empty((s_l, H, d), dtype=buf.dtype, device=buf.device)
    _need(shard, "shard", (s_l, H, d), buf.dtype, buf.device)
    if H % P == 0 or P % H == 0:
        _shape(buf, "buf", (P, s_l, rank_heads(0, P, H)[1], d), buf.dtype)
    _call("ulysses_recv_unpack", _dev(buf), P, s_l, H, d, _dtype(buf), _dev(shard), _stream())
    return shard


def _group_args(tensor_lists):
    """Host arrays for the grouped permutes: one array of P device pointers per tensor, an
    array of those arrays, and the global head counts."""
    arrays = [_ptrs(ts) for ts in tensor_lists]
    outer = (ctypes.c_void_p * len(arrays))(*[ctypes.cast(a, ctypes.c_void_p).value for a, _ in arrays])
    heads = (ctypes.c_int * len(tensor_lists))(*[ts[0].shape[1] for ts in tensor_lists])
    return ctypes.cast(outer, _vpp), ctypes.cast(heads, _i32p), (arrays, outer, heads)


def _group_check(shard_lists, flats, what):
    P = len(shard_lists[0])
    x0 = _same(shard_lists[0], f"{what}[0]")
    s_l, _, d = x0.shape
    for i, (sh, f) in enumerate(zip(shard_lists, flats)):
        if len(sh) != P:
            raise ValueError(f"{what}[{i}]: {len(sh)} shards, expected {P}")
        x = _same(sh, f"{what}[{i}]")
        if x.shape[0] != s_l or x.shape[2] != d or x.dtype != x0.dtype or x.device != x0.device:
            raise ValueError(f"{what}[{i}]: shards {tuple(x.shape)} {x.dtype} do not match {what}[0]")
        _need(f, f"head shard {i}", (P * s_l, x.shape[1] // P, d), x0.dtype, x0.device)
    return P, s_l, d, x0


def ulysses_pack_group(shard_lists, rank, outs=None):
    """Several tensors' P sequence shards [s_l, H_i, d] -> their head shards [P*s_l, H_i/P, d],
    in one launch (the Q/K/V of the forward exchange)."""
    n = len(shard_lists)
    P = len(shard_lists[0])
    s_l, _, d = shard_lists[0][0].shape
    if outs is None:
        outs = [torch.empty((P * s_l, sh[0].shape[1] // P, d), dtype=sh[0].dtype, device=sh[0].device)
                for sh in shard_lists]
    if len(outs) != n:
        raise ValueError("one output per tensor")
    P, s_l, d, x0 = _group_check(shard_lists, outs, "shard_lists")
    pp, hh, _keep = _group_args(shard_lists)
    op, _keep2 = _ptrs(outs)
    _call("ulysses_pack_group", n, pp, hh, op, P, rank, s_l, d, _dtype(x0), _stream())
    return outs


def ulysses_unpack_group(ys, rank, shard_lists):
    """Several head shards [P*s_l, H_i/P, d] -> head slice `rank` of their P shards, in one launch
    (the dQ/dK/dV of the backward exchange)."""
    n = len(ys)
    if len(shard_lists) != n:
        raise ValueError("one shard list per tensor")
    P, s_l, d, x0 = _group_check(shard_lists, ys, "shard_lists")
    pp, hh, _keep = _group_args(shard_lists)
    yp, _keep2 = _ptrs(ys)
    _call("ulysses_unpack_group", n, yp, hh, pp, P, rank, s_l, d, _dtype(x0), _stream())
    return shard_lists


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _qkv(q, k, v):
    """Shapes of a head shard's q [s, Hq, d], k, v [s, Hkv, d] (checked)."""
    s, Hq, d = q.shape
    _dtype(q)
    Hkv = k.shape[1]
    _shape(k, "k", (s, Hkv, d), q.dtype)
    _shape(v, "v", (s, Hkv, d), q.dtype)
    _dev(q)
    _need(k, "k", (s, Hkv, d), q.dtype, q.device)
    _need(v, "v", (s, Hkv, d), q.dtype, q.device)
    return s, Hq, Hkv, d


def attn_fwd_workspace_bytes(s, Hq, d):
    return int(lib().attn_fwd_workspace_bytes(s, Hq, d))


def attn_fwd(q, k, v, scale=None, causal=True, cu_seqlens=None, out=None, lse=None, o_lo=None, workspace=None,
             split=True):
    """q [s, Hq, d], k, v [s, Hkv, d] -> (o [s, Hq, d], lse [Hq, s] fp32). When `o_lo` (bf16
    [s, Hq, d], e.g. new_o_lo(q)) is given, O's bf16 rounding residual is written into it. On
    short sequences each row block's keys split over several workgroups when a workspace of
    attn_fwd_workspace_bytes is given (allocated here unless split=False)."""
    s, Hq, Hkv, d = _qkv(q, k, v)
    o = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((Hq, s), dtype=torch.float32, device=q.device)
    _need(o, "out", (s, Hq, d), q.dtype, q.device)
    _need(lse, "lse", (Hq, s), torch.float32, q.device)
    lo = _opt(o_lo, "o_lo", (s, Hq, d), torch.bfloat16, q.device)
    if workspace is None and split:
        need = attn_fwd_workspace_bytes(s, Hq, d)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws, cap = (None, 0) if workspace is None or not split else (_dev(workspace),
                                                                 workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens, q.device)
    _call("attn_fwd", _dev(q), _dev(k), _dev(v), _dev(o), lo, _dev(lse), s, Hq, Hkv, d, _dtype(q),
          _default_scale(d, scale), int(causal), cu, nd, ws, cap, _stream())
    return o, lse


def attn_bwd_workspace_bytes(s, Hq, Hkv, d):
    return int(lib().attn_bwd_workspace_bytes(s, Hq, Hkv, d))


def attn_bwd_dkdv_workspace_bytes(s, Hkv, d):
    return int(lib().attn_bwd_dkdv_workspace_bytes(s, Hkv, d))


def attn_bwd_dq_workspace_bytes(s, Hq, d):
    return int(lib().attn_bwd_dq_workspace_bytes(s, Hq, d))


def delta_bytes(s, Hq):
    """Bytes of delta [Hq, s] fp32 rounded up to 256 (the shard-reading backward's workspace)."""
    return (s * Hq * 4 + 255) // 256 * 256


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=True, cu_seqlens=None, workspace=None,
             dq=None, dk=None, dv=None, o_lo=None, split=True):
    """Gradients (dq, dk, dv) of the attention forward, given its o and lse and dout (and the
    forward's o_lo, if it wrote one: delta then comes from O to about 16 bits). split=False
    allocates room for delta only, so dK/dV and dQ run unsplit on short sequences too."""
    s, Hq, Hkv, d = _qkv(q, k, v)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _need(t, n, (s, Hq, d), q.dtype, q.device)
    for t, n in ((dk, "dk"), (dv, "dv")):
        _need(t, n, (s, Hkv, d), q.dtype, q.device)
    _need(lse, "lse", (Hq, s), torch.float32, q.device)
    lo = _opt(o_lo, "o_lo", (s, Hq, d), torch.bfloat16, q.device)
    need = attn_bwd_workspace_bytes(s, Hq, Hkv, d) if split else delta_bytes(s, Hq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens, q.device)
    _call("attn_bwd", _dev(q), _dev(k), _dev(v), _dev(o), lo, _dev(lse), _dev(dout), _dev(dq), _dev(dk), _dev(dv),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, _dev(workspace),
          ctypes.byref(cap), _stream())
    return dq, dk, dv


NOALLOC_MAX_DELTA = 1 << 22


def attn_bwd_noalloc(q, k, v, o, lse, dout, scale=None, causal=True, cu_seqlens=None, dq=None, dk=None, dv=None,
                     o_lo=None):
    """attn_bwd without a workspace: delta lives in the library's static per-device array
    (s * Hq <= NOALLOC_MAX_DELTA). Calls that overlap on one GPU race."""
    s, Hq, Hkv, d = _qkv(q, k, v)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _need(t, n, (s, Hq, d), q.dtype, q.device)
    for t, n in ((dk, "dk"), (dv, "dv")):
        _need(t, n, (s, Hkv, d), q.dtype, q.device)
    _need(lse, "lse", (Hq, s), torch.float32, q.device)
    lo = _opt(o_lo, "o_lo", (s, Hq, d), torch.bfloat16, q.device)
    cu, nd = _cu(cu_seqlens, q.device)
    _call("attn_bwd_noalloc", _dev(q), _dev(k), _dev(v), _dev(o), lo, _dev(lse), _dev(dout), _dev(dq), _dev(dk),
          _dev(dv), s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, _stream())
    return dq, dk, dv


def attn_bwd_preprocess(o, dout, delta=None, o_lo=None):
    s, Hq, d = o.shape
    _dtype(o)
    _need(dout, "dout", (s, Hq, d), o.dtype, o.device)
    if delta is None:
        delta = torch.empty((Hq, s), dtype=torch.float32, device=o.device)
    _need(delta, "delta", (Hq, s), torch.float32, o.device)
    lo = _opt(o_lo, "o_lo", (s, Hq, d), torch.bfloat16, o.device)
    _call("attn_bwd_preprocess", _dev(o), lo, _dev(dout), _dev(delta), s, Hq, d, _dtype(o), _stream())
    return delta


def _bwd_phase_checks(q, lse, dout, delta):
    s, Hq, d = q.shape
    _need(dout, "dout", (s, Hq, d), q.dtype, q.device)
    _need(lse, "lse", (Hq, s), torch.float32, q.device)
    _need(delta, "delta", (Hq, s), torch.float32, q.device)


def attn_bwd_dkdv(q, k, v, lse, dout, delta, scale=None, causal=True, cu_seqlens=None, dk=None, dv=None,
                  workspace=None, split=True):
    """dK, dV. On short sequences the key blocks split over several workgroups when a workspace
    of attn_bwd_dkdv_workspace_bytes is given (allocated here unless split=False)."""
    s, Hq, Hkv, d = _qkv(q, k, v)
    _bwd_phase_checks(q, lse, dout, delta)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((dk, "dk"), (dv, "dv")):
        _need(t, n, (s, Hkv, d), q.dtype, q.device)
    if workspace is None and split:
        need = attn_bwd_dkdv_workspace_bytes(s, Hkv, d)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws, cap = (None, 0) if workspace is None or not split else (_dev(workspace),
                                                                 workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens, q.device)
    _call("attn_bwd_dkdv", _dev(q), _dev(k), _dev(v), _dev(lse), _dev(dout), _dev(delta), _dev(dk), _dev(dv),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, ws, cap, _stream())
    return dk, dv


def attn_bwd_dq(q, k, v, lse, dout, delta, scale=None, causal=True, cu_seqlens=None, dq=None,
                workspace=None, split=True):
    """dQ. On short sequences each row block's keys split over several workgroups when a
    workspace of attn_bwd_dq_workspace_bytes is given (allocated here unless split=False)."""
    s, Hq, Hkv, d = _qkv(q, k, v)
    _bwd_phase_checks(q, lse, dout, delta)
    dq = torch.empty_like(q) if dq is None else dq
    _need(dq, "dq", (s, Hq, d), q.dtype, q.device)
    if workspace is None and split:
        need = attn_bwd_dq_workspace_bytes(s, Hq, d)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws, cap = (None, 0) if workspace is None or not split else (_dev(workspace),
                                                                 workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens, q.device)
    _call("attn_bwd_dq", _dev(q), _dev(k), _dev(v), _dev(lse), _dev(dout), _dev(delta), _dev(dq),
          s, Hq, Hkv, d, _dtype(q), _default_scale(d, scale), int(causal), cu, nd, ws, cap, _stream())
    return dq


def _shard_sets(q_shards, k_shards, v_shards, *more_q, more_kv=()):
    """Checks the shard lists of a rank's call: q-shaped [s_l, Hq, d] and kv-shaped [s_l, Hkv, d]
    lists of P shards each, one dtype and device; returns (P, s_l, Hq, Hkv, d, q0)."""
    P = len(q_shards)
    q0 = _same(q_shards, "q_shards")
    s_l, Hq, d = q0.shape
    _dtype(q0)
    Hkv = k_shards[0].shape[1]
    for name, L, H in [("k_shards", k_shards, Hkv), ("v_shards", v_shards, Hkv)] + \
            [(f"q-shaped shards {i}", L, Hq) for i, L in enumerate(more_q)] + \
            [(f"kv-shaped shards {i}", L, Hkv) for i, L in enumerate(more_kv)]:
        if len(L) != P:
            raise ValueError(f"{name}: {len(L)} shards, expected {P}")
        for j, t in enumerate(L):
            _need(t, f"{name}[{j}]", (s_l, H, d), q0.dtype, q0.device)
    return P, s_l, Hq, Hkv, d, q0


def attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk):
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    return int(lib().attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk))


def attn_fwd_chunked(q_shards, k_shards, v_shards, o_shards, rank, heads_per_chunk, scale=None,
                     causal=True, cu_seqlens=None, workspace=None, lse=None, o_lo=None):
    """UPipe forward of rank `rank`: writes this rank's heads of o_shards (and, when given, O's
    rounding residual into o_lo [s, Hq/P, d]); returns lse [Hq/P, s]."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards, o_shards)
    s = P * s_l
    if lse is None:
        lse = torch.empty((Hq // P, s), dtype=torch.float32, device=q0.device)
    _need(lse, "lse", (Hq // P, s), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (s, Hq // P, d), torch.bfloat16, q0.device)
    need = attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, _dtype(q0), heads_per_chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q0.device)
    if workspace is None or workspace.numel() == 0:   # none needed: NULL workspace and size
        ws_ptr, cap_ref = None, None
    else:
        cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
        ws_ptr, cap_ref = _dev(workspace), ctypes.byref(cap)
    qp, k1 = _ptrs(q_shards)
    kp, k2 = _ptrs(k_shards)
    vp, k3 = _ptrs(v_shards)
    op, k4 = _ptrs(o_shards)
    cu, nd = _cu(cu_seqlens, q0.device)
    _call("attn_fwd_chunked", qp, kp, vp, op, lo, _dev(lse), P, rank, s_l, Hq, Hkv, d, _dtype(q0),
          _default_scale(d, scale), int(causal), cu, nd, heads_per_chunk, ws_ptr, cap_ref, _stream())
    return lse


def attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk):
    dt = dtype if isinstance(dtype, int) else _dtype(torch.empty(0, dtype=dtype))
    return int(lib().attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk))


def attn_bwd_chunked(q_shards, k_shards, v_shards, o_shards, lse, do_shards, dq_shards, dk_shards, dv_shards,
                     rank, heads_per_chunk, scale=None, causal=True, cu_seqlens=None, workspace=None, o_lo=None):
    """UPipe backward of rank `rank`: writes this rank's heads of dq_shards, dk_shards, dv_shards."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards,
                                         more_kv=(dk_shards, dv_shards))
    s = P * s_l
    _need(lse, "lse", (Hq // P, s), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (s, Hq // P, d), torch.bfloat16, q0.device)
    dt = _dtype(q0)
    need = attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dt, heads_per_chunk)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q0.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards, dk_shards, dv_shards)]
    qp, kp, vp, op, gp, dqp, dkp, dvp = (k[0] for k in keep)
    cu, nd = _cu(cu_seqlens, q0.device)
    _call("attn_bwd_chunked", qp, kp, vp, op, lo, _dev(lse), gp, dqp, dkp, dvp, P, rank, s_l, Hq, Hkv, d, dt,
          _default_scale(d, scale), int(causal), cu, nd, heads_per_chunk, _dev(workspace), ctypes.byref(cap),
          _stream())
    return dq_shards, dk_shards, dv_shards


def attn_fwd_shards(q_shards, k_shards, v_shards, o_shards, rank, scale=None, causal=True, cu_seqlens=None,
                    lse=None, o_lo=None, workspace=None, split=True):
    """Forward of rank `rank` straight from the sequence shards into head slice `rank` of
    o_shards (no head-shard buffers); returns the LSE [Hq/P, s]. Short and mid-size grids split
    their keys as attn_fwd does, given a workspace (allocated here unless split=False)."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards, o_shards)
    if lse is None:
        lse = torch.empty((Hq // P, P * s_l), dtype=torch.float32, device=q0.device)
    _need(lse, "lse", (Hq // P, P * s_l), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (P * s_l, Hq // P, d), torch.bfloat16, q0.device)
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards)]
    qp, kp, vp, op = (k[0] for k in keep)
    if workspace is None and split:
        need = attn_fwd_workspace_bytes(P * s_l, Hq // P, d)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q0.device)
    ws, cap = (None, 0) if workspace is None or not split else (_dev(workspace),
                                                                 workspace.numel() * workspace.element_size())
    cu, nd = _cu(cu_seqlens, q0.device)
    _call("attn_fwd_shards", qp, kp, vp, op, lo, _dev(lse), P, rank, s_l, Hq, Hkv, d, _dtype(q0),
          _default_scale(d, scale), int(causal), cu, nd, ws, cap, _stream())
    return lse


def attn_bwd_shards(q_shards, k_shards, v_shards, o_shards, lse, do_shards, dq_shards, dk_shards, dv_shards,
                    rank, scale=None, causal=True, cu_seqlens=None, workspace=None, o_lo=None, split=True):
    """Backward of rank `rank` straight from the sequence shards into head slice `rank` of
    the dq / dk / dv shards. The workspace holds delta and, if it has room (the queried size,
    which is allocated here unless split=False), the partial sums of the split dK/dV and dQ
    runs of short and mid-size grids."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards,
                                         more_kv=(dk_shards, dv_shards))
    _need(lse, "lse", (Hq // P, P * s_l), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (P * s_l, Hq // P, d), torch.bfloat16, q0.device)
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, o_shards, do_shards, dq_shards, dk_shards, dv_shards)]
    qp, kp, vp, op, gp, dqp, dkp, dvp = (k[0] for k in keep)
    cu, nd = _cu(cu_seqlens, q0.device)
    if workspace is None:
        need = ctypes.c_size_t(0)
        if split:
            _call("attn_bwd_shards", qp, kp, vp, op, lo, _dev(lse), gp, dqp, dkp, dvp, P, rank, s_l, Hq, Hkv, d,
                  _dtype(q0), _default_scale(d, scale), int(causal), cu, nd, None, ctypes.byref(need), _stream())
        workspace = torch.empty(need.value if split else delta_bytes(P * s_l, Hq // P), dtype=torch.uint8,
                                device=q0.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    _call("attn_bwd_shards", qp, kp, vp, op, lo, _dev(lse), gp, dqp, dkp, dvp, P, rank, s_l, Hq, Hkv, d,
          _dtype(q0), _default_scale(d, scale), int(causal), cu, nd, _dev(workspace), ctypes.byref(cap),
          _stream())
    return dq_shards, dk_shards, dv_shards


def ring_attn_fwd(q_shards, k_shards, v_shards, rank, scale=None, causal=True, out=None, lse=None, o_lo=None,
                  workspace=None):
    """Ring Attention forward of rank `rank` (its token block of every head): returns (o, lse),
    o [s_l, Hq, d], lse [Hq, s_l]; o_lo (bf16 [s_l, Hq, d]) receives O's residual when given."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards)
    o = torch.empty_like(q0) if out is None else out
    if lse is None:
        lse = torch.empty((Hq, s_l), dtype=torch.float32, device=q0.device)
    _need(o, "out", (s_l, Hq, d), q0.dtype, q0.device)
    _need(lse, "lse", (Hq, s_l), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (s_l, Hq, d), torch.bfloat16, q0.device)
    need = int(lib().ring_attn_fwd_workspace_bytes(s_l, Hq, d))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q0.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards)]
    qp, kp, vp = (k[0] for k in keep)
    _call("ring_attn_fwd", qp, kp, vp, _dev(o), lo, _dev(lse), P, rank, s_l, Hq, Hkv, d, _dtype(q0),
          _default_scale(d, scale), int(causal), _dev(workspace), ctypes.byref(cap), _stream())
    return o, lse


def ring_attn_bwd(q_shards, k_shards, v_shards, o, lse, dout, rank, dk_acc, dv_acc, dk_shards, dv_shards,
                  scale=None, causal=True, dq=None, o_lo=None, workspace=None):
    """Ring Attention backward of rank `rank`: returns its dq [s_l, Hq, d] and adds its share to
    the fp32 dK/dV sums dk_acc, dv_acc [P, s_l, Hkv, d]; the call of rank P - 1 rounds them into
    dk_shards / dv_shards. Ranks must be called in order on one stream."""
    P, s_l, Hq, Hkv, d, q0 = _shard_sets(q_shards, k_shards, v_shards, more_kv=(dk_shards, dv_shards))
    dq = torch.empty_like(q0) if dq is None else dq
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _need(t, n, (s_l, Hq, d), q0.dtype, q0.device)
    _need(lse, "lse", (Hq, s_l), torch.float32, q0.device)
    for t, n in ((dk_acc, "dk_acc"), (dv_acc, "dv_acc")):
        _need(t, n, (P, s_l, Hkv, d), torch.float32, q0.device)
    lo = _opt(o_lo, "o_lo", (s_l, Hq, d), torch.bfloat16, q0.device)
    need = int(lib().ring_attn_bwd_workspace_bytes(s_l, Hq, d))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q0.device)
    cap = ctypes.c_size_t(workspace.numel() * workspace.element_size())
    keep = [_ptrs(x) for x in (q_shards, k_shards, v_shards, dk_shards, dv_shards)]
    qp, kp, vp, dkp, dvp = (k[0] for k in keep)
    _call("ring_attn_bwd", qp, kp, vp, _dev(o), lo, _dev(lse), _dev(dout), _dev(dq), _dev(dk_acc), _dev(dv_acc),
          dkp, dvp, P, rank, s_l, Hq, Hkv, d, _dtype(q0), _default_scale(d, scale), int(causal), _dev(workspace),
          ctypes.byref(cap), _stream())
    return dq


MIX_KINDS = {0: "mfma+lds", 1: "mfma+lds+2fma+1exp", 2: "mfma+lds+4fma+1exp"}


def mix_probe(kind, waves_per_simd, iters=4000):
    """Rate (TFLOP/s) of the inner-loop instruction mix `kind` (MIX_KINDS) with
    `waves_per_simd` (1..4) waves on every SIMD, timed with events on the current stream."""
    if kind not in MIX_KINDS or not 1 <= waves_per_simd <= 4:
        raise ValueError("kind must be 0..2 and waves_per_simd 1..4")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    blocks = 256 * waves_per_simd
    _call("uly_mix_probe", kind, 2, blocks, _dev(sink), _stream())  # warm-up
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    _call("uly_mix_probe", kind, iters, blocks, _dev(sink), _stream())
    b.record()
    torch.cuda.synchronize()
    return float(blocks) * 4 * iters * 16 * 32768 / (a.elapsed_time(b) * 1e-3) / 1e12


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
