"""The C ABI without a GPU: the library loads, exports every entry point the header
declares, and rejects bad arguments on the host before touching the device.

Only calls that fail validation (or only report sizes) run here; nothing is launched."""
import ctypes
import os
import re

import pytest

import ulysses_sequence_parallelism_rank_amd as U

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses.h")

FAKE = 0x10000   # 16-byte aligned stand-in for a device pointer; never dereferenced
MIS = 0x10008    # misaligned stand-in


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**([a-z_][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_header_parses():
    names = declared_functions()
    for want in ("ulysses_pack", "ulysses_unpack", "attn_fwd", "attn_bwd", "attn_fwd_chunked"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(U.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(U.SIGNATURES)


def test_status_strings_and_version():
    L = U.lib()
    assert L.uly_abi_version() == 7
    for code, name in U.STATUS.items():
        assert L.uly_status_string(code).decode() == name


def _ptr_array(vals):
    arr = (ctypes.c_void_p * len(vals))(*vals)
    return ctypes.cast(arr, U._vpp), arr


@pytest.mark.parametrize("P,rank,s_l,H,d,dt,want", [
    (0, 0, 4, 4, 64, 0, 2), (65, 0, 4, 65, 64, 0, 2), (2, 2, 4, 4, 64, 0, 2), (2, -1, 4, 4, 64, 0, 2),
    (2, 0, 0, 4, 64, 0, 2), (3, 0, 4, 4, 64, 0, 2), (2, 0, 4, 4, 64, 7, 3), (2, 0, 4, 2, 4, 0, 4),
    (2, 0, 4, 4098, 64, 0, 2),   # more heads than ULY_MAX_HEADS
])
def test_pack_rejects(P, rank, s_l, H, d, dt, want):
    L = U.lib()
    pp, keep = _ptr_array([FAKE] * max(P, 1))
    assert L.ulysses_pack(pp, P, rank, s_l, H, d, dt, FAKE, None) == want
    assert L.ulysses_unpack(FAKE, P, rank, s_l, H, d, dt, pp, None) == want


def test_pack_null_and_alignment():
    L = U.lib()
    pp, keep = _ptr_array([FAKE, None])
    assert L.ulysses_pack(pp, 2, 0, 4, 4, 64, 0, FAKE, None) == 1
    assert L.ulysses_pack(None, 2, 0, 4, 4, 64, 0, FAKE, None) == 1
    pp, keep = _ptr_array([FAKE, MIS])
    assert L.ulysses_pack(pp, 2, 0, 4, 4, 64, 0, FAKE, None) == 4
    pp, keep = _ptr_array([FAKE, FAKE])
    assert L.ulysses_pack(pp, 2, 0, 4, 4, 64, 0, MIS, None) == 4


def _group(n, P, Hs, shard_vals=None, flat_vals=None, rank=0, s_l=4, d=64, dt=0):
    """Host arrays for ulysses_pack_group / ulysses_unpack_group with fake device pointers."""
    keep = []
    inner = []
    for i in range(len(Hs)):
        pp, arr = _ptr_array(shard_vals[i] if shard_vals else [FAKE] * P)
        keep.append(arr)
        inner.append(ctypes.cast(pp, ctypes.c_void_p).value)
    outer = (ctypes.c_void_p * max(len(inner), 1))(*inner)
    heads = (ctypes.c_int * max(len(Hs), 1))(*Hs)
    flat = (ctypes.c_void_p * max(len(Hs), 1))(*(flat_vals or [FAKE] * len(Hs)))
    keep += [outer, heads, flat]
    L = U.lib()
    a = (ctypes.cast(outer, U._vpp), ctypes.cast(heads, U._i32p), ctypes.cast(flat, U._vpp))
    got_pack = L.ulysses_pack_group(n, a[0], a[1], a[2], P, rank, s_l, d, dt, None)
    got_unpack = L.ulysses_unpack_group(n, a[2], a[1], a[0], P, rank, s_l, d, dt, None)
    return got_pack, got_unpack


@pytest.mark.parametrize("n,P,Hs,kw,want", [
    (0, 2, (4,), {}, 2),                       # no tensor
    (4, 2, (4, 4, 4, 4), {}, 2),               # more than ULY_PERM_GROUP_MAX
    (2, 2, (4, 3), {}, 2),                     # one head count not divisible by P
    (3, 2, (4, 4, 4), {"rank": 2}, 2),         # rank out of range
    (2, 2, (4, 4), {"dt": 7}, 3),              # dtype
    (2, 2, (2, 2), {"d": 4}, 4),               # a tensor's run not a multiple of 16 bytes
    (2, 2, (4, 4), {"s_l": 0}, 2),             # empty shards
])
def test_group_permute_rejects(n, P, Hs, kw, want):
    assert _group(n, P, Hs, **kw) == (want, want)


def test_group_permute_null_and_alignment():
    assert _group(2, 2, (4, 4), shard_vals=[[FAKE, FAKE], [FAKE, None]]) == (1, 1)
    assert _group(2, 2, (4, 4), flat_vals=[FAKE, None]) == (1, 1)
    assert _group(2, 2, (4, 4), shard_vals=[[FAKE, FAKE], [MIS, FAKE]]) == (4, 4)
    assert _group(3, 2, (4, 4, 4), flat_vals=[FAKE, FAKE, MIS]) == (4, 4)
    L = U.lib()
    heads = (ctypes.c_int * 1)(4)
    assert L.ulysses_pack_group(1, None, ctypes.cast(heads, U._i32p), None, 2, 0, 4, 64, 0, None) == 1
    assert L.ulysses_unpack_group(1, None, None, None, 2, 0, 4, 64, 0, None) == 1


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, o_lo=None, lse=FAKE, s=16, Hq=4, Hkv=2, d=128, dt=0, scale=0.1,
                causal=1, cu=None, nd=0)
    args.update(kw)
    a = args
    return U.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["o_lo"], a["lse"], a["s"], a["Hq"], a["Hkv"],
                            a["d"], a["dt"], a["scale"], a["causal"], a["cu"], a["nd"], a.get("ws"), a.get("cap", 0),
                            None)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(lse=None), 1),
    (dict(Hq=3, Hkv=2), 2), (dict(s=0), 2), (dict(Hkv=0), 2), (dict(cu=FAKE, nd=0), 2),
    (dict(Hq=4097 * 2, Hkv=2), 2),   # more heads than ULY_MAX_HEADS
    (dict(d=96), 3), (dict(dt=1, d=128), 3), (dict(dt=5), 3),
    (dict(k=MIS), 4), (dict(o=MIS), 4),
    (dict(o_lo=MIS), 4), (dict(dt=1, d=64, o_lo=FAKE), 3),   # the O residual: aligned, bf16 only
    (dict(ws=MIS, cap=1 << 20), 4),                          # a workspace must be 16-byte aligned
])
def test_attn_fwd_rejects(kw, want):
    assert _fwd(**kw) == want


def test_bwd_workspace_query_and_checks():
    L = U.lib()
    need = ctypes.c_size_t(0)
    z = [FAKE] * 10
    st = L.attn_bwd(*z, 1000, 8, 2, 128, 0, 0.1, 1, None, 0, None, ctypes.byref(need), None)
    assert st == 0 and need.value == L.attn_bwd_workspace_bytes(1000, 8, 2, 128) and need.value >= 1000 * 8 * 4
    small = ctypes.c_size_t(1000 * 8 * 4 - 1)   # less than delta
    assert L.attn_bwd(*z, 1000, 8, 2, 128, 0, 0.1, 1, None, 0, FAKE, ctypes.byref(small), None) == 5
    assert L.attn_bwd(*z, 1000, 8, 3, 128, 0, 0.1, 1, None, 0, None, ctypes.byref(need), None) == 2
    assert L.attn_bwd(*z, 1000, 8, 2, 128, 0, 0.1, 1, None, 0, None, None, None) == 1
    assert L.attn_bwd_preprocess(FAKE, None, None, FAKE, 10, 2, 128, 0, None) == 1
    assert L.attn_bwd_preprocess(FAKE, MIS, FAKE, FAKE, 10, 2, 128, 0, None) == 4
    assert L.attn_bwd_preprocess(FAKE, FAKE, FAKE, FAKE, 10, 2, 64, 1, None) == 3
    zl = [FAKE, FAKE, FAKE, FAKE, MIS] + [FAKE] * 5   # misaligned o_lo
    assert L.attn_bwd(*zl, 1000, 8, 2, 128, 0, 0.1, 1, None, 0, None, ctypes.byref(need), None) == 4
    assert L.attn_bwd_dkdv(*[FAKE] * 8, 10, 4, 3, 128, 0, 0.1, 1, None, 0, None, 0, None) == 2
    assert L.attn_bwd_dkdv(*[FAKE] * 8, 10, 4, 2, 128, 0, 0.1, 1, None, 0, MIS, 1 << 20, None) == 4
    assert L.attn_bwd_dq(*[FAKE] * 7, 10, 4, 2, 100, 0, 0.1, 1, None, 0, None, 0, None) == 3
    assert L.attn_bwd_dq(*[FAKE] * 7, 10, 4, 2, 128, 0, 0.1, 1, None, 0, MIS, 1 << 20, None) == 4


def test_chunked_workspace_matches_upipe_accounting():
    L = U.lib()
    MiB = 2 ** 20
    # 262144 tokens, 64 q / 8 kv heads, P = 8, d = 128, bf16: the chunks read the shards directly
    for u in (1, 2, 8):
        assert L.attn_fwd_chunked_workspace_bytes(8, 32768, 64, 8, 128, 0, u) == 0
    assert L.attn_fwd_chunked_workspace_bytes(8, 32768, 64, 8, 128, 0, 0) == 0
    # shards whose length is not a multiple of 128 stage each chunk: Q and O of u heads plus K and
    # V of the kv heads they read, [s, ., d] bf16 each (the UPipe accounting: 87.5% less than the
    # 8 q heads' Q and O at u = 1)
    s_l = 32760
    s = 8 * s_l
    r256 = lambda b: (b + 255) // 256 * 256
    for u, span in ((1, 1), (2, 1), (8, 1)):
        want = 2 * r256(s * u * 128 * 2) + 2 * r256(s * span * 128 * 2)
        assert L.attn_fwd_chunked_workspace_bytes(8, s_l, 64, 8, 128, 0, u) == want
    assert L.attn_fwd_chunked_workspace_bytes(8, s_l, 64, 8, 128, 0, 1) < 257 * MiB


def test_chunked_rejects():
    L = U.lib()
    pp, keep = _ptr_array([FAKE] * 2)
    need = ctypes.c_size_t(0)
    args = lambda **kw: dict(dict(P=2, rank=0, s_l=8, Hq=8, Hkv=4, d=64, dt=0, u=1), **kw)

    def call(ws=None, cap=None, **kw):
        a = args(**kw)
        return L.attn_fwd_chunked(pp, pp, pp, pp, None, FAKE, a["P"], a["rank"], a["s_l"], a["Hq"], a["Hkv"], a["d"],
                                  a["dt"], 0.1, 1, None, 0, a["u"], ws, cap, None)
    assert call(cap=ctypes.byref(need)) == 0 and need.value > 0
    assert call(cap=ctypes.byref(need), u=0) == 2
    assert call(cap=ctypes.byref(need), Hkv=3) == 2
    assert call(cap=ctypes.byref(need), Hq=6, Hkv=3) == 2    # Hkv % P
    assert call(cap=ctypes.byref(need), rank=2) == 2
    small = ctypes.c_size_t(need.value - 256)
    assert call(ws=FAKE, cap=ctypes.byref(small)) == 5


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        U.attn_fwd(x, x, x)


def test_bwd_chunked_workspace_and_rejects():
    L = U.lib()
    MiB = 2 ** 20
    # the 256K UPipe share read from the shards: delta of a one-head chunk (1 MiB) and the fp32
    # dK/dV sums of the rank's kv head (2 x 128 MiB)
    assert L.attn_bwd_chunked_workspace_bytes(8, 32768, 64, 8, 128, 0, 1) == 257 * MiB
    # staged chunks (shards not a multiple of 128): also Q, O, dO, dQ of the chunk, K/V and dK/dV
    s = 8 * 32760
    r256 = lambda b: (b + 255) // 256 * 256
    staged = 4 * r256(s * 256) + 2 * r256(s * 256) + r256(s * 4) + 2 * r256(s * 512) + 2 * r256(s * 256)
    assert L.attn_bwd_chunked_workspace_bytes(8, 32760, 64, 8, 128, 0, 1) == staged
    assert L.attn_bwd_chunked_workspace_bytes(8, 32768, 64, 8, 128, 0, 0) == 0
    pp, keep = _ptr_array([FAKE] * 2)
    need = ctypes.c_size_t(0)

    def call(ws=None, cap=None, P=2, rank=0, s_l=8, Hq=8, Hkv=4, d=64, dt=0, u=1, lse=FAKE):
        return L.attn_bwd_chunked(pp, pp, pp, pp, None, lse, pp, pp, pp, pp, P, rank, s_l, Hq, Hkv, d, dt, 0.1, 1,
                                  None, 0, u, ws, cap, None)
    assert call(cap=ctypes.byref(need)) == 0 and need.value == L.attn_bwd_chunked_workspace_bytes(2, 8, 8, 4, 64,
                                                                                                0, 1)
    assert call(cap=ctypes.byref(need), u=0) == 2
    assert call(cap=ctypes.byref(need), Hkv=3) == 2
    assert call(cap=ctypes.byref(need), rank=2) == 2
    assert call(cap=ctypes.byref(need), d=96) == 3
    small = ctypes.c_size_t(need.value - 256)
    assert call(ws=FAKE, cap=ctypes.byref(small)) == 5
    assert call(ws=FAKE, cap=ctypes.byref(need), lse=None) == 1
    assert call(ws=MIS, cap=ctypes.byref(need)) == 4


def test_shards_rejects():
    L = U.lib()
    pp, keep = _ptr_array([FAKE] * 2)
    mp, keep2 = _ptr_array([FAKE, MIS])

    def fwd(q=pp, s_l=128, Hq=8, Hkv=4, d=128, dt=0, rank=0, lse=FAKE, o_lo=None, ws=None, cap=0):
        return L.attn_fwd_shards(q, pp, pp, pp, o_lo, lse, 2, rank, s_l, Hq, Hkv, d, dt, 0.1, 1, None, 0, ws, cap,
                                 None)
    assert fwd(s_l=96) == 3          # a workgroup's rows must lie in one shard
    assert fwd(dt=1, d=64) == 3      # bf16 only
    assert fwd(d=96) == 3
    assert fwd(Hkv=3) == 2
    assert fwd(rank=2) == 2
    assert fwd(lse=None) == 1
    assert fwd(q=mp) == 4
    assert fwd(o_lo=MIS) == 4
    assert fwd(ws=MIS, cap=1 << 20) == 4
    need = ctypes.c_size_t(0)

    def bwd(ws=None, cap=None, s_l=128, dt=0, d=128):
        return L.attn_bwd_shards(pp, pp, pp, pp, None, FAKE, pp, pp, pp, pp, 2, 0, s_l, 8, 4, d, dt, 0.1, 1, None, 0,
                                 ws, cap, None)
    # the query: delta, then room for the split runs' partial sums (256 tokens: both split)
    part = max(L.attn_bwd_dkdv_workspace_bytes(256, 2, 128), L.attn_bwd_dq_workspace_bytes(256, 4, 128))
    assert part > 0
    assert bwd(cap=ctypes.byref(need)) == 0 and need.value == U.delta_bytes(256, 4) + part
    assert bwd(cap=ctypes.byref(need), s_l=64) == 3
    assert bwd(cap=ctypes.byref(need), dt=1, d=64) == 3
    small = ctypes.c_size_t(U.delta_bytes(256, 4) - 1)   # delta is required, the partials are not
    assert bwd(ws=FAKE, cap=ctypes.byref(small)) == 5
    assert bwd(ws=None, cap=None) == 1


def test_probe_rejects():
    L = U.lib()
    assert L.uly_mfma_probe(0, 4, FAKE, FAKE, None) == 2
    assert L.uly_mfma_probe(4, 0, FAKE, FAKE, None) == 2
    assert L.uly_mfma_probe(4, 4, None, FAKE, None) == 1
    assert L.uly_mix_probe(0, 0, 4, FAKE, None) == 2
    assert L.uly_mix_probe(0, 4, 0, FAKE, None) == 2
    assert L.uly_mix_probe(3, 4, 4, FAKE, None) == 3
    assert L.uly_mix_probe(-1, 4, 4, FAKE, None) == 3
    assert L.uly_mix_probe(1, 4, 4, None, None) == 1


def test_binding_checks_shapes_before_the_call():
    """The binding rejects a tensor whose shape or dtype does not match before any pointer
    reaches the library (the C side cannot see a tensor's extent)."""
    import torch
    q = torch.zeros(16, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k: shape"):
        U.attn_fwd(q, torch.zeros(15, 2, 64, dtype=torch.bfloat16), torch.zeros(16, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="v: dtype"):
        U.attn_fwd(q, torch.zeros(16, 2, 64, dtype=torch.bfloat16), torch.zeros(16, 2, 64, dtype=torch.float32))
    with pytest.raises(ValueError, match="shards\\[1\\]"):
        U.ulysses_pack([torch.zeros(8, 4, 64, dtype=torch.bfloat16), torch.zeros(8, 2, 64, dtype=torch.bfloat16)], 0)
    with pytest.raises(ValueError, match="cu_seqlens"):
        U._cu(torch.zeros(1, dtype=torch.int32))


def test_bwd_noalloc_rejects_on_the_host():
    """The allocation-free backward refuses a delta larger than its static array, and the usual
    argument errors, before touching the device."""
    L = U.lib()
    z = [FAKE] * 10
    too_big = (U.NOALLOC_MAX_DELTA // 8) + 1
    assert L.attn_bwd_noalloc(*z, too_big, 8, 2, 128, 0, 0.1, 1, None, 0, None) == 5
    assert L.attn_bwd_noalloc(*z, 1000, 8, 3, 128, 0, 0.1, 1, None, 0, None) == 2
    assert L.attn_bwd_noalloc(None, *z[1:], 1000, 8, 2, 128, 0, 0.1, 1, None, 0, None) == 1
    assert L.attn_bwd_noalloc(*z[:4], MIS, *z[5:], 1000, 8, 2, 128, 0, 0.1, 1, None, 0, None) == 4


@pytest.mark.parametrize("P,s_l,H,d,dt,want", [
    (0, 4, 4, 64, 0, 2), (65, 4, 4, 64, 0, 2), (4, 0, 4, 64, 0, 2), (4, 4, 3, 64, 0, 2), (3, 4, 2, 64, 0, 2),
    (4, 4, 4, 64, 7, 3), (4, 4, 2, 4, 0, 4), (4, 4, 4100, 64, 0, 2),
])
def test_send_recv_reject_on_the_host(P, s_l, H, d, dt, want):
    L = U.lib()
    assert L.ulysses_send_pack(FAKE, P, s_l, H, d, dt, FAKE, None) == want
    assert L.ulysses_recv_unpack(FAKE, P, s_l, H, d, dt, FAKE, None) == want


def test_send_recv_null_and_alignment():
    L = U.lib()
    assert L.ulysses_send_pack(None, 4, 4, 8, 64, 0, FAKE, None) == 1
    assert L.ulysses_recv_unpack(FAKE, 4, 4, 8, 64, 0, None, None) == 1
    assert L.ulysses_send_pack(MIS, 4, 4, 8, 64, 0, FAKE, None) == 4
    assert L.ulysses_recv_unpack(FAKE, 4, 4, 2, 64, 0, MIS, None) == 4


def test_ring_rejects_on_the_host():
    L = U.lib()
    pp, keep = _ptr_array([FAKE] * 4)
    need = ctypes.c_size_t(0)

    def fwd(P=4, rank=1, s_l=64, Hq=8, Hkv=2, d=128, dt=0, ws=None, cap=None, o=FAKE, q=pp):
        return L.ring_attn_fwd(q, pp, pp, o, None, FAKE, P, rank, s_l, Hq, Hkv, d, dt, 0.1, 1, ws, cap, None)
    assert fwd(cap=ctypes.byref(need)) == 0 and need.value == L.ring_attn_fwd_workspace_bytes(64, 8, 128)
    assert fwd(rank=4, cap=ctypes.byref(need)) == 2
    assert fwd(Hkv=3, cap=ctypes.byref(need)) == 2
    assert fwd(Hq=8192, cap=ctypes.byref(need)) == 2   # more heads than ULY_MAX_HEADS
    assert fwd(dt=1, d=64, cap=ctypes.byref(need)) == 3
    small = ctypes.c_size_t(need.value - 1)
    assert fwd(ws=FAKE, cap=ctypes.byref(small)) == 5
    assert fwd(ws=FAKE, cap=ctypes.byref(need), o=None) == 1
    mp, keep2 = _ptr_array([FAKE, FAKE, MIS, FAKE])
    assert fwd(q=mp, cap=ctypes.byref(need)) == 4

    def bwd(ws=FAKE, cap=None, acc=FAKE, rank=3):
        return L.ring_attn_bwd(pp, pp, pp, FAKE, None, FAKE, FAKE, FAKE, acc, FAKE, pp, pp, 4, rank, 64, 8, 2, 128, 0,
                               0.1, 1, ws, cap, None)
    nb = ctypes.c_size_t(0)
    assert bwd(ws=None, cap=ctypes.byref(nb)) == 0 and nb.value == L.ring_attn_bwd_workspace_bytes(64, 8, 128)
    assert bwd(cap=ctypes.byref(nb), acc=None) == 1
    assert bwd(cap=ctypes.byref(nb), acc=MIS) == 4
    assert bwd(cap=ctypes.byref(nb), rank=-1) == 2


def test_dkdv_split_accounting():
    """Key blocks split over workgroups while the grid is under two rounds (512 workgroups of
    one per CU): 8K share (2 kv heads) -> 4 splits and 64 MiB of fp32 partials; 16K share -> 2;
    64K share -> none."""
    L = U.lib()
    MiB = 2 ** 20
    assert L.attn_bwd_dkdv_workspace_bytes(8192, 2, 128) == 2 * 64 * 4 * 2 * 128 * 128 * 4 == 64 * MiB
    assert L.attn_bwd_dkdv_workspace_bytes(65536, 2, 128) == 0
    assert L.attn_bwd_dkdv_workspace_bytes(16384, 2, 128) == 2 * 128 * 2 * 2 * 128 * 128 * 4 == 64 * MiB
    assert L.attn_bwd_dkdv_workspace_bytes(32768, 1, 128) == 1 * 256 * 2 * 2 * 128 * 128 * 4   # 256 -> 2
    assert L.attn_bwd_dkdv_workspace_bytes(65536, 1, 128) == 0      # 512 blocks: two full rounds
    assert L.attn_bwd_dkdv_workspace_bytes(128, 1, 64) == 1 * 1 * 8 * 2 * 128 * 64 * 4   # capped at 8
    delta = U.delta_bytes(8192, 8)
    assert L.attn_bwd_workspace_bytes(8192, 8, 2, 128) == delta + 64 * MiB
    assert L.attn_bwd_workspace_bytes(65536, 8, 2, 128) == U.delta_bytes(65536, 8)


def test_fwd_split_accounting():
    """Forward row blocks split below 768 workgroups (128 rows x q head) aiming at 1024, at most
    8 per block, and in two from 768 to 1151; each split keeps fp32 O sums (128 x d) and 4
    floats of row statistics per row: 8K share (8 q heads, 512 workgroups) -> 2 splits; 12K and
    16K -> 2; 20K (1280) and the 64K share -> none."""
    L = U.lib()
    assert L.attn_fwd_workspace_bytes(8192, 8, 128) == 8 * 64 * 2 * 128 * (128 + 4) * 4
    assert L.attn_fwd_workspace_bytes(65536, 8, 128) == 0
    assert L.attn_fwd_workspace_bytes(12288, 8, 128) == 8 * 96 * 2 * 128 * (128 + 4) * 4    # 768 -> 2
    assert L.attn_fwd_workspace_bytes(16384, 8, 128) == 8 * 128 * 2 * 128 * (128 + 4) * 4   # 1024 -> 2
    assert L.attn_fwd_workspace_bytes(18432, 8, 128) == 0            # 1152 workgroups: no split
    assert L.attn_fwd_workspace_bytes(20480, 8, 128) == 0
    assert L.attn_fwd_workspace_bytes(8192, 11, 128) == 11 * 64 * 2 * 128 * (128 + 4) * 4   # 704 -> 2
    assert L.attn_fwd_workspace_bytes(4096, 8, 64) == 8 * 32 * 4 * 128 * (64 + 4) * 4      # 256 -> 4
    assert L.attn_fwd_workspace_bytes(100, 1, 64) == 1 * 1 * 8 * 128 * (64 + 4) * 4        # capped at 8
    assert L.attn_fwd_workspace_bytes(0, 8, 128) == 0


def test_dq_split_accounting():
    """dQ row blocks split while fewer than 1024 workgroups (128 rows x q head) would run, aiming
    at 1024, at most 8 per block: 8K share (8 q heads) -> 2 splits, 64 MiB of fp32 partials,
    the same bytes the dK/dV split needs, so attn_bwd's workspace is delta + their maximum;
    12K -> 2; 16K and the 64K share -> none."""
    L = U.lib()
    MiB = 2 ** 20
    assert L.attn_bwd_dq_workspace_bytes(8192, 8, 128) == 8 * 64 * 2 * 128 * 128 * 4 == 64 * MiB
    assert L.attn_bwd_dq_workspace_bytes(65536, 8, 128) == 0
    assert L.attn_bwd_dq_workspace_bytes(8192, 16, 128) == 0         # 1024 workgroups: full
    assert L.attn_bwd_dq_workspace_bytes(16384, 8, 128) == 0
    assert L.attn_bwd_dq_workspace_bytes(12288, 8, 128) == 8 * 96 * 2 * 128 * 128 * 4   # 768 -> 2
    assert L.attn_bwd_dq_workspace_bytes(4096, 8, 64) == 8 * 32 * 4 * 128 * 64 * 4   # 256 -> 4 splits
    assert L.attn_bwd_dq_workspace_bytes(128, 1, 64) == 1 * 1 * 8 * 128 * 64 * 4     # capped at 8
    assert L.attn_bwd_dq_workspace_bytes(0, 8, 128) == 0
    # 4K, 8 q heads, 1 kv head: dQ needs 4 splits of 32 x 8 blocks, dK/dV 8 of 32 x 1
    delta = U.delta_bytes(4096, 8)
    dq_part = 8 * 32 * 4 * 128 * 128 * 4
    dkdv_part = 1 * 32 * 8 * 2 * 128 * 128 * 4
    assert L.attn_bwd_workspace_bytes(4096, 8, 1, 128) == delta + max(dq_part, dkdv_part)
