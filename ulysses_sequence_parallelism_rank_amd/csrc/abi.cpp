// C ABI of libulysses: argument checks, dispatch to the gfx950 kernels, and the
// headwise-chunked (UPipe) schedule. Every check runs on the host before anything is
// enqueued; see include/ulysses.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "uly_internal.h"
#include "ulysses.h"

using namespace uly;

namespace {

constexpr int kAbiVersion = 7;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int esize(int dtype) { return dtype == ULY_BF16 ? 2 : 4; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int hip_status(hipError_t e) { return e == hipSuccess ? ULY_OK : ULY_ERR_HIP; }
inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

int check_dtype_dim(int dtype, int d) {
  if (dtype == ULY_BF16) return (d == 64 || d == 128) ? ULY_OK : ULY_ERR_UNSUPPORTED;
  if (dtype == ULY_F32) return d == 64 ? ULY_OK : ULY_ERR_UNSUPPORTED;
  return ULY_ERR_UNSUPPORTED;
}

// P, rank, s_l, H checks shared by the permutes and the chunked forward.
int check_ranks(int P, int rank, int64_t s_l, int H) {
  if (P < 1 || P > ULY_MAX_RANKS || rank < 0 || rank >= P) return ULY_ERR_SHAPE;
  if (s_l < 1 || H < 1 || H > ULY_MAX_HEADS || H % P != 0) return ULY_ERR_SHAPE;
  return ULY_OK;
}

// The permute kernels index 16-byte chunks with 32-bit integers.
bool chunks_fit(int P, int64_t s_l, int64_t run_bytes, int64_t row_bytes) {
  const uint64_t total = (uint64_t)P * (uint64_t)s_l * (uint64_t)(run_bytes / 16);
  const uint64_t shard = (uint64_t)s_l * (uint64_t)(row_bytes / 16);
  return total < (1ull << 32) && shard < (1ull << 32);
}

int check_attn(const void* q, const void* k, const void* v, int64_t s, int Hq, int Hkv, int d,
               int dtype, const int32_t* cu, int n_docs) {
  if (!q || !k || !v) return ULY_ERR_NULL;
  int st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (s < 1 || Hq < 1 || Hkv < 1 || Hq > ULY_MAX_HEADS || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  if (s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;  // cu_seqlens are int32
  if (cu != nullptr && n_docs < 1) return ULY_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return ULY_ERR_ALIGN;
  return ULY_OK;
}

// O's rounding residual: bf16 only (an fp32 O has none), 16-byte aligned
int check_o_lo(const void* o_lo, int dtype) {
  if (o_lo == nullptr) return ULY_OK;
  if (dtype != ULY_BF16) return ULY_ERR_UNSUPPORTED;
  return aligned16(o_lo) ? ULY_OK : ULY_ERR_ALIGN;
}

AttnArgs make_args(int64_t s, int Hq, int Hkv, int d, float scale, int causal, const int32_t* cu,
                   int n_docs) {
  AttnArgs a{};
  a.s = s;
  a.q_row = (int64_t)Hq * d;
  a.kv_row = (int64_t)Hkv * d;
  a.dkv_row = (int64_t)Hkv * d;
  a.acc_row = (int64_t)Hkv * d;
  a.lse_row = s;
  a.n_heads = Hq;
  a.n_kv = Hkv;
  a.G = Hq / Hkv;
  a.q_off = 0;
  a.kv_off = 0;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.cu = cu;
  a.n_docs = cu ? n_docs : 0;
  a.acc_init = -1;
  a.acc_final = -1;
  a.nsplit = 1;
  a.nsplit_q = 1;
  a.nsplit_o = 1;
  return a;
}

int fwd_dispatch(const AttnArgs& a, int d, int dtype, hipStream_t st) {
  const hipError_t e = dtype == ULY_BF16 ? launch_attn_fwd_bf16(a, d, st) : launch_attn_fwd_f32(a, d, st);
  return hip_status(e);
}

ShardPtrs shard_ptrs(const void* const* p, int P) {
  ShardPtrs sp{};
  for (int i = 0; i < P; ++i) sp.p[i] = p[i];
  return sp;
}

// q heads [c0, c1) of the rank's Hq_l local heads read kv heads [c0/G, (c1-1)/G] (local).
int max_kv_span(int Hq_l, int G, int u) {
  int span = 0;
  for (int c0 = 0; c0 < Hq_l; c0 += u) {
    const int c1 = std::min(c0 + u, Hq_l);
    span = std::max(span, (c1 - 1) / G - c0 / G + 1);
  }
  return span;
}

}  // namespace

namespace {

// Byte sizes of the parts of attn_bwd_chunked's workspace (see the layout there).
struct BwdChunkLayout {
  size_t qc, kv, delta, acc, out, total;
};
// the shard-reading chunked backward: delta of a chunk and the fp32 dK/dV sums of the rank's kv heads
size_t bwd_shard_chunk_bytes(int P, int64_t s_l, int Hq, int Hkv, int d, int u) {
  const size_t s = (size_t)P * (size_t)s_l;
  return round256((size_t)u * s * sizeof(float)) + 2 * round256(s * (size_t)(Hkv / P) * (size_t)d * sizeof(float));
}
BwdChunkLayout bwd_chunk_layout(int P, int64_t s_l, int Hq, int Hkv, int d, int dtype, int u) {
  const int Hq_l = Hq / P, Hkv_l = Hkv / P, G = Hq / Hkv;
  const size_t s = (size_t)P * (size_t)s_l, e = (size_t)esize(dtype);
  BwdChunkLayout L;
  L.qc = round256(s * (size_t)u * (size_t)d * e);
  L.kv = round256(s * (size_t)max_kv_span(Hq_l, G, u) * (size_t)d * e);
  L.delta = round256((size_t)u * s * sizeof(float));
  L.acc = round256(s * (size_t)Hkv_l * (size_t)d * sizeof(float));
  L.out = round256(s * (size_t)Hkv_l * (size_t)d * e);
  L.total = 4 * L.qc + 2 * L.kv + L.delta + 2 * L.acc + 2 * L.out;
  return L;
}
}  // namespace

extern "C" {

const char* uly_status_string(int status) {
  switch (status) {
    case ULY_OK: return "ULY_OK";
    case ULY_ERR_NULL: return "ULY_ERR_NULL";
    case ULY_ERR_SHAPE: return "ULY_ERR_SHAPE";
    case ULY_ERR_UNSUPPORTED: return "ULY_ERR_UNSUPPORTED";
    case ULY_ERR_ALIGN: return "ULY_ERR_ALIGN";
    case ULY_ERR_WORKSPACE: return "ULY_ERR_WORKSPACE";
    case ULY_ERR_HIP: return "ULY_ERR_HIP";
    default: return "ULY_ERR_UNKNOWN";
  }
}

int uly_abi_version(void) { return kAbiVersion; }

int uly_mfma_probe(int iters, int blocks, float* sink, uint64_t* clocks, void* stream) {
  if (!sink || !clocks) return ULY_ERR_NULL;
  if (iters < 1 || blocks < 1) return ULY_ERR_SHAPE;
  return hip_status(launch_mfma_probe(iters, blocks, sink, reinterpret_cast<unsigned long long*>(clocks),
                                      as_stream(stream)));
}

int uly_mix_probe(int kind, int iters, int blocks, float* sink, void* stream) {
  if (!sink) return ULY_ERR_NULL;
  if (iters < 1 || blocks < 1) return ULY_ERR_SHAPE;
  if (kind < 0 || kind > 2) return ULY_ERR_UNSUPPORTED;
  return hip_status(launch_mix_probe(kind, iters, blocks, sink, as_stream(stream)));
}

int ulysses_pack(const void* const* shards, int P, int rank, int64_t s_l, int H, int d, int dtype,
                 void* out, void* stream) {
  if (!shards || !out) return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, H);
  if (st != ULY_OK) return st;
  if (dtype != ULY_BF16 && dtype != ULY_F32) return ULY_ERR_UNSUPPORTED;
  if (d < 1) return ULY_ERR_SHAPE;
  const int64_t Hl = H / P, e = esize(dtype);
  const int64_t run = Hl * d * e, row = (int64_t)H * d * e;
  if (run % 16 != 0) return ULY_ERR_ALIGN;
  for (int p = 0; p < P; ++p) {
    if (!shards[p]) return ULY_ERR_NULL;
    if (!aligned16(shards[p])) return ULY_ERR_ALIGN;
  }
  if (!aligned16(out)) return ULY_ERR_ALIGN;
  if (!chunks_fit(P, s_l, run, row)) return ULY_ERR_SHAPE;
  return hip_status(launch_pack(shard_ptrs(shards, P), out, P, s_l, row, rank * run, run, as_stream(stream)));
}

int ulysses_unpack(const void* in, int P, int rank, int64_t s_l, int H, int d, int dtype,
                   void* const* shards, void* stream) {
  if (!shards || !in) return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, H);
  if (st != ULY_OK) return st;
  if (dtype != ULY_BF16 && dtype != ULY_F32) return ULY_ERR_UNSUPPORTED;
  if (d < 1) return ULY_ERR_SHAPE;
  const int64_t Hl = H / P, e = esize(dtype);
  const int64_t run = Hl * d * e, row = (int64_t)H * d * e;
  if (run % 16 != 0) return ULY_ERR_ALIGN;
  for (int p = 0; p < P; ++p) {
    if (!shards[p]) return ULY_ERR_NULL;
    if (!aligned16(shards[p])) return ULY_ERR_ALIGN;
  }
  if (!aligned16(in)) return ULY_ERR_ALIGN;
  if (!chunks_fit(P, s_l, run, row)) return ULY_ERR_SHAPE;
  return hip_status(launch_unpack(in, shard_ptrs(const_cast<const void* const*>(shards), P), P, s_l, row,
                                  rank * run, run, as_stream(stream)));
}

// Checks shared by the send-side and receive-side permutes of one rank.
static int check_send_recv(const void* a, const void* b, int P, int64_t s_l, int H, int d, int dtype) {
  if (!a || !b) return ULY_ERR_NULL;
  if (P < 1 || P > ULY_MAX_RANKS || s_l < 1 || H < 1 || H > ULY_MAX_HEADS || d < 1) return ULY_ERR_SHAPE;
  if (H % P != 0 && P % H != 0) return ULY_ERR_SHAPE;
  if (dtype != ULY_BF16 && dtype != ULY_F32) return ULY_ERR_UNSUPPORTED;
  if (((int64_t)d * esize(dtype)) % 16 != 0) return ULY_ERR_ALIGN;
  if (!aligned16(a) || !aligned16(b)) return ULY_ERR_ALIGN;
  const uint64_t units = (uint64_t)s_l * (uint64_t)std::max(H, P) * (uint64_t)(d * esize(dtype) / 16);
  if (units >= (1ull << 32)) return ULY_ERR_SHAPE;
  return ULY_OK;
}

int ulysses_send_pack(const void* shard, int P, int64_t s_l, int H, int d, int dtype, void* out, void* stream) {
  const int st = check_send_recv(shard, out, P, s_l, H, d, dtype);
  if (st != ULY_OK) return st;
  return hip_status(launch_send_pack(shard, out, P, s_l, H, (int64_t)d * esize(dtype), as_stream(stream)));
}

int ulysses_recv_unpack(const void* in, int P, int64_t s_l, int H, int d, int dtype, void* shard, void* stream) {
  const int st = check_send_recv(in, shard, P, s_l, H, d, dtype);
  if (st != ULY_OK) return st;
  return hip_status(launch_recv_unpack(in, shard, P, s_l, H, (int64_t)d * esize(dtype), dtype == ULY_BF16 ? 1 : 0,
                                       as_stream(stream)));
}

// Checks shared by the grouped permutes: every tensor as ulysses_pack / ulysses_unpack
// would check it; fills the launch segments.
static int group_segments(int n, const void* const* const* shards, const int* H, void* const* flat, int P,
                          int rank, int64_t s_l, int d, int dtype, PermSeg* segs) {
  if (!shards || !H || !flat) return ULY_ERR_NULL;
  if (n < 1 || n > ULY_PERM_GROUP_MAX) return ULY_ERR_SHAPE;
  if (dtype != ULY_BF16 && dtype != ULY_F32) return ULY_ERR_UNSUPPORTED;
  if (d < 1) return ULY_ERR_SHAPE;
  for (int i = 0; i < n; ++i) {
    int st = check_ranks(P, rank, s_l, H[i]);
    if (st != ULY_OK) return st;
    const int64_t Hl = H[i] / P, e = esize(dtype);
    const int64_t run = Hl * d * e, row = (int64_t)H[i] * d * e;
    if (run % 16 != 0) return ULY_ERR_ALIGN;
    if (!shards[i] || !flat[i]) return ULY_ERR_NULL;
    for (int p = 0; p < P; ++p) {
      if (!shards[i][p]) return ULY_ERR_NULL;
      if (!aligned16(shards[i][p])) return ULY_ERR_ALIGN;
    }
    if (!aligned16(flat[i])) return ULY_ERR_ALIGN;
    if (!chunks_fit(P, s_l, run, row)) return ULY_ERR_SHAPE;
    segs[i] = PermSeg{shard_ptrs(shards[i], P), flat[i], P, row, rank * run, run};
  }
  return ULY_OK;
}

int ulysses_pack_group(int n, const void* const* const* shards, const int* H, void* const* out, int P, int rank,
                       int64_t s_l, int d, int dtype, void* stream) {
  PermSeg segs[ULY_PERM_GROUP_MAX];
  const int st = group_segments(n, shards, H, out, P, rank, s_l, d, dtype, segs);
  if (st != ULY_OK) return st;
  return hip_status(launch_pack_group(segs, n, s_l, as_stream(stream)));
}

int ulysses_unpack_group(int n, const void* const* in, const int* H, void* const* const* shards, int P, int rank,
                         int64_t s_l, int d, int dtype, void* stream) {
  PermSeg segs[ULY_PERM_GROUP_MAX];
  const int st = group_segments(n, reinterpret_cast<const void* const* const*>(shards), H,
                                const_cast<void* const*>(in), P, rank, s_l, d, dtype, segs);
  if (st != ULY_OK) return st;
  return hip_status(launch_unpack_group(segs, n, s_l, as_stream(stream)));
}

size_t attn_fwd_workspace_bytes(int64_t s, int Hq, int d) {
  if (s < 1 || Hq < 1 || d < 1) return 0;
  return fwd_part_bytes(s, Hq, d);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse, int64_t s, int Hq,
             int Hkv, int d, int dtype, float scale, int causal, const int32_t* cu_seqlens, int n_docs,
             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_attn(q, k, v, s, Hq, Hkv, d, dtype, cu_seqlens, n_docs);
  if (st != ULY_OK) return st;
  if (!o || !lse) return ULY_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse)) return ULY_ERR_ALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  AttnArgs a = make_args(s, Hq, Hkv, d, scale, causal, cu_seqlens, n_docs);
  const size_t part = attn_fwd_workspace_bytes(s, Hq, d);
  if (dtype == ULY_BF16 && part > 0 && workspace != nullptr && workspace_bytes >= part) {
    // small grid: each row block's key tiles over several workgroups, merged in split order
    a.nsplit_o = fwd_split_count(s, Hq);
    a.o_part = static_cast<float*>(workspace);
    a.o_stat = a.o_part + fwd_part_floats(s, Hq, d);
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = o;
  a.o_lo = o_lo;
  a.lo_row = (int64_t)Hq * d;
  a.lse_out = lse;
  return fwd_dispatch(a, d, dtype, as_stream(stream));
}

// delta [Hq, s] fp32 of the backward
static size_t delta_bytes(int64_t s, int Hq) {
  if (s < 1 || Hq < 1) return 0;
  return round256((size_t)s * (size_t)Hq * sizeof(float));
}

size_t attn_bwd_dkdv_workspace_bytes(int64_t s, int Hkv, int d) {
  if (s < 1 || Hkv < 1 || d < 1) return 0;
  return dkdv_part_bytes(s, Hkv, d);
}

size_t attn_bwd_dq_workspace_bytes(int64_t s, int Hq, int d) {
  if (s < 1 || Hq < 1 || d < 1) return 0;
  return dq_part_bytes(s, Hq, d);
}

size_t attn_bwd_workspace_bytes(int64_t s, int Hq, int Hkv, int d) {
  if (s < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
  // the dK/dV and the dQ partial sums share one region: the dK/dV reduce has read the first
  // before the dQ kernel, later on the same stream, writes the second
  const size_t part = std::max(attn_bwd_dkdv_workspace_bytes(s, Hkv, d), attn_bwd_dq_workspace_bytes(s, Hq, d));
  return delta_bytes(s, Hq) + round256(part);
}

int attn_bwd_preprocess(const void* o, const void* o_lo, const void* dout, float* delta, int64_t s, int Hq, int d,
                        int dtype, void* stream) {
  if (!o || !dout || !delta) return ULY_ERR_NULL;
  int st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (s < 1 || Hq < 1 || s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  AttnArgs a = make_args(s, Hq, Hq, d, 1.f, 1, nullptr, 0);
  a.o = o;
  a.o_lo = const_cast<void*>(o_lo);
  a.lo_row = (int64_t)Hq * d;
  a.dout = dout;
  a.lse_out = delta;
  return hip_status(launch_bwd_preprocess(a, d, dtype, as_stream(stream)));
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                  const float* delta, void* dk, void* dv, int64_t s, int Hq, int Hkv, int d, int dtype,
                  float scale, int causal, const int32_t* cu_seqlens, int n_docs, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int st = check_attn(q, k, v, s, Hq, Hkv, d, dtype, cu_seqlens, n_docs);
  if (st != ULY_OK) return st;
  if (!lse || !dout || !delta || !dk || !dv) return ULY_ERR_NULL;
  if (!aligned16(lse) || !aligned16(dout) || !aligned16(delta) || !aligned16(dk) || !aligned16(dv))
    return ULY_ERR_ALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return ULY_ERR_ALIGN;
  const size_t part = attn_bwd_dkdv_workspace_bytes(s, Hkv, d);
  const bool split = dtype == ULY_BF16 && part > 0 && workspace != nullptr && workspace_bytes >= part;
  AttnArgs a = make_args(s, Hq, Hkv, d, scale, causal, cu_seqlens, n_docs);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse_in = lse;
  a.delta = delta;
  a.out_k = dk;
  a.out_v = dv;
  if (split) {  // small grid: each key block's rows over several workgroups, partials reduced in order
    a.nsplit = dkdv_split_count(s, Hkv);
    a.dkv_part = static_cast<float*>(workspace);
  }
  const hipError_t e = dtype == ULY_BF16 ? launch_attn_dkdv_bf16(a, d, as_stream(stream))
                                         : launch_attn_dkdv_f32(a, d, as_stream(stream));
  return hip_status(e);
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                const float* delta, void* dq, int64_t s, int Hq, int Hkv, int d, int dtype, float scale,
                int causal, const int32_t* cu_seqlens, int n_docs, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_attn(q, k, v, s, Hq, Hkv, d, dtype, cu_seqlens, n_docs);
  if (st != ULY_OK) return st;
  if (!lse || !dout || !delta || !dq) return ULY_ERR_NULL;
  if (!aligned16(lse) || !aligned16(dout) || !aligned16(delta) || !aligned16(dq)) return ULY_ERR_ALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return ULY_ERR_ALIGN;
  const size_t part = attn_bwd_dq_workspace_bytes(s, Hq, d);
  const bool split = dtype == ULY_BF16 && part > 0 && workspace != nullptr && workspace_bytes >= part;
  AttnArgs a = make_args(s, Hq, Hkv, d, scale, causal, cu_seqlens, n_docs);
  if (split) {  // small grid: each row block's key tiles over several workgroups, partials reduced in order
    a.nsplit_q = dq_split_count(s, Hq);
    a.dq_part = static_cast<float*>(workspace);
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse_in = lse;
  a.delta = delta;
  a.out = dq;
  const hipError_t e = dtype == ULY_BF16 ? launch_attn_dq_bf16(a, d, as_stream(stream))
                                         : launch_attn_dq_f32(a, d, as_stream(stream));
  return hip_status(e);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_lo, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int64_t s, int Hq, int Hkv, int d, int dtype, float scale,
             int causal, const int32_t* cu_seqlens, int n_docs, void* workspace, size_t* workspace_bytes,
             void* stream) {
  int st = check_attn(q, k, v, s, Hq, Hkv, d, dtype, cu_seqlens, n_docs);
  if (st != ULY_OK) return st;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  const size_t need = attn_bwd_workspace_bytes(s, Hq, Hkv, d);
  if (workspace == nullptr) {
    if (!workspace_bytes) return ULY_ERR_NULL;
    *workspace_bytes = need;
    return ULY_OK;
  }
  // delta is required; the dK/dV partial sums are optional (dK/dV run split only with room for them)
  const size_t cap = workspace_bytes ? *workspace_bytes : need;
  if (cap < delta_bytes(s, Hq)) return ULY_ERR_WORKSPACE;
  if (!o || !lse || !dout || !dq || !dk || !dv) return ULY_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(workspace))
    return ULY_ERR_ALIGN;
  float* delta = static_cast<float*>(workspace);
  st = attn_bwd_preprocess(o, o_lo, dout, delta, s, Hq, d, dtype, stream);
  if (st != ULY_OK) return st;
  const size_t dpart = delta_bytes(s, Hq);
  st = attn_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, s, Hq, Hkv, d, dtype, scale, causal, cu_seqlens, n_docs,
                     static_cast<char*>(workspace) + dpart, cap - dpart, stream);
  if (st != ULY_OK) return st;
  return attn_bwd_dq(q, k, v, lse, dout, delta, dq, s, Hq, Hkv, d, dtype, scale, causal, cu_seqlens, n_docs,
                     static_cast<char*>(workspace) + dpart, cap - dpart, stream);
}

// ---- attn_bwd without a caller workspace ---------------------------------------------
// delta lives in a file-scope device array; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name in host code is a
// host-side stand-in, not a device address).
static __device__ __align__(256) float scratch[ULY_NOALLOC_MAX_DELTA];

static std::mutex g_scratch_mu;
static float* g_scratch_ptr[ULY_MAX_DEVICES];

// this device's copy of `scratch`, looked up once per device (null on failure)
static float* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= ULY_MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  return g_scratch_ptr[dev];
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* o_lo, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int64_t s, int Hq, int Hkv, int d, int dtype,
                     float scale, int causal, const int32_t* cu_seqlens, int n_docs, void* stream) {
  int st = check_attn(q, k, v, s, Hq, Hkv, d, dtype, cu_seqlens, n_docs);
  if (st != ULY_OK) return st;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  if (!o || !lse || !dout || !dq || !dk || !dv) return ULY_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return ULY_ERR_ALIGN;
  if (Hq < 1 || (uint64_t)s * (uint64_t)Hq > (uint64_t)ULY_NOALLOC_MAX_DELTA) return ULY_ERR_WORKSPACE;
  // every argument is checked: only now is the device touched
  float* delta = device_scratch();
  if (delta == nullptr) return ULY_ERR_HIP;
  // every element of delta the kernels read is written by the preprocess first: nothing to clear;
  // dK/dV and dQ run unsplit (no partial sums, which would need more than the array)
  if ((st = attn_bwd_preprocess(o, o_lo, dout, delta, s, Hq, d, dtype, stream)) != ULY_OK) return st;
  if ((st = attn_bwd_dkdv(q, k, v, lse, dout, delta, dk, dv, s, Hq, Hkv, d, dtype, scale, causal, cu_seqlens,
                          n_docs, nullptr, 0, stream)) != ULY_OK)
    return st;
  return attn_bwd_dq(q, k, v, lse, dout, delta, dq, s, Hq, Hkv, d, dtype, scale, causal, cu_seqlens, n_docs,
                     nullptr, 0, stream);
}

// ---- UPipe headwise-chunked forward ------------------------------------------------

// The chunked schedules read the sequence shards directly (no chunk buffers) when the
// shard-reading kernels apply: bf16 and every workgroup's rows inside one shard.
static bool chunks_read_shards(int dtype, int64_t s_l) { return dtype == ULY_BF16 && s_l % 128 == 0; }

size_t attn_fwd_chunked_workspace_bytes(int P, int64_t s_l, int Hq, int Hkv, int d, int dtype,
                                        int heads_per_chunk) {
  if (P < 1 || s_l < 1 || Hq < 1 || Hkv < 1 || d < 1 || heads_per_chunk < 1) return 0;
  if (Hq % P != 0 || Hkv % P != 0 || Hq % Hkv != 0) return 0;
  if (chunks_read_shards(dtype, s_l)) return 0;
  const int Hq_l = Hq / P, G = Hq / Hkv;
  const int u = std::min(heads_per_chunk, Hq_l);
  const size_t s = (size_t)P * (size_t)s_l, e = (size_t)esize(dtype);
  const size_t qo = round256(s * (size_t)u * (size_t)d * e);
  const size_t kv = round256(s * (size_t)max_kv_span(Hq_l, G, u) * (size_t)d * e);
  return 2 * qo + 2 * kv;
}

int attn_fwd_chunked(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards,
                     void* const* o_shards, void* o_lo, float* lse, int P, int rank, int64_t s_l, int Hq, int Hkv,
                     int d, int dtype, float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                     int heads_per_chunk, void* workspace, size_t* workspace_bytes, void* stream) {
  if (!q_shards || !k_shards || !v_shards || !o_shards) return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, Hq);
  if (st != ULY_OK) return st;
  if (Hkv < 1 || Hkv % P != 0 || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (heads_per_chunk < 1) return ULY_ERR_SHAPE;
  const int64_t s = (int64_t)P * s_l;
  if (s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  if (cu_seqlens != nullptr && n_docs < 1) return ULY_ERR_SHAPE;
  const size_t need = attn_fwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk);
  if (workspace == nullptr && workspace_bytes != nullptr) {  // size query
    *workspace_bytes = need;
    return ULY_OK;
  }
  if (workspace == nullptr && need > 0) return ULY_ERR_NULL;  // both NULL: runs only when none is needed
  if (workspace_bytes && *workspace_bytes < need) return ULY_ERR_WORKSPACE;
  if (!lse) return ULY_ERR_NULL;
  if (!aligned16(lse) || (workspace != nullptr && !aligned16(workspace))) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  for (int p = 0; p < P; ++p) {
    if (!q_shards[p] || !k_shards[p] || !v_shards[p] || !o_shards[p]) return ULY_ERR_NULL;
    if (!aligned16(q_shards[p]) || !aligned16(k_shards[p]) || !aligned16(v_shards[p]) || !aligned16(o_shards[p]))
      return ULY_ERR_ALIGN;
  }
  const int Hq_l = Hq / P, Hkv_l = Hkv / P, G = Hq / Hkv;
  const int u = std::min(heads_per_chunk, Hq_l);
  const int64_t e = esize(dtype);
  const int64_t qrow = (int64_t)Hq * d * e, kvrow = (int64_t)Hkv * d * e, hb = (int64_t)d * e;
  if (!chunks_fit(P, s_l, qrow, qrow) || !chunks_fit(P, s_l, kvrow, kvrow)) return ULY_ERR_SHAPE;

  hipStream_t strm = as_stream(stream);
  if (chunks_read_shards(dtype, s_l)) {
    // each chunk's heads straight from the shards into the o shards: no buffers at all
    for (int c0 = 0; c0 < Hq_l; c0 += u) {
      const int c1 = std::min(c0 + u, Hq_l), nq = c1 - c0;
      const int g0 = c0 / G, g1 = (c1 - 1) / G + 1;
      ShardSrc src{};
      for (int p = 0; p < P; ++p) {
        src.q[p] = static_cast<const uint16_t*>(q_shards[p]) + ((int64_t)rank * Hq_l + c0) * d;
        src.k[p] = static_cast<const uint16_t*>(k_shards[p]) + ((int64_t)rank * Hkv_l + g0) * d;
        src.v[p] = static_cast<const uint16_t*>(v_shards[p]) + ((int64_t)rank * Hkv_l + g0) * d;
        src.o[p] = static_cast<uint16_t*>(o_shards[p]) + ((int64_t)rank * Hq_l + c0) * d;
      }
      src.s_l = s_l;
      AttnArgs a = make_args(s, nq, 1, d, scale, causal, cu_seqlens, n_docs);
      a.q_row = (int64_t)Hq * d;  // rows of the sequence shards hold every head
      a.kv_row = (int64_t)Hkv * d;
      a.n_heads = nq;
      a.n_kv = g1 - g0;
      a.G = G;
      a.q_off = c0;
      a.kv_off = g0;
      a.o_lo = o_lo == nullptr ? nullptr : static_cast<char*>(o_lo) + c0 * hb;
      a.lo_row = (int64_t)Hq_l * d;
      a.lse_out = lse + (int64_t)c0 * s;
      if (launch_attn_fwd_bf16_shards(a, src, d, strm) != hipSuccess) return ULY_ERR_HIP;
    }
    return ULY_OK;
  }
  const int span = max_kv_span(Hq_l, G, u);
  char* ws = static_cast<char*>(workspace);
  const size_t qo = round256((size_t)s * u * d * e);
  void* qc = ws;
  void* oc = ws + qo;
  void* kc = ws + 2 * qo;
  void* vc = ws + 2 * qo + round256((size_t)s * span * d * e);
  const ShardPtrs qs = shard_ptrs(q_shards, P), ks = shard_ptrs(k_shards, P), vs = shard_ptrs(v_shards, P);
  const ShardPtrs os = shard_ptrs(const_cast<const void* const*>(o_shards), P);

  int kv_lo = -1, kv_hi = -1;  // local kv heads currently packed in kc / vc
  for (int c0 = 0; c0 < Hq_l; c0 += u) {
    const int c1 = std::min(c0 + u, Hq_l), nq = c1 - c0;
    const int g0 = c0 / G, g1 = (c1 - 1) / G + 1;
    hipError_t err;
    if (g0 != kv_lo || g1 != kv_hi) {
      const int64_t off = ((int64_t)rank * Hkv_l + g0) * hb, run = (int64_t)(g1 - g0) * hb;
      const PermSeg kv[2] = {{ks, kc, P, kvrow, off, run}, {vs, vc, P, kvrow, off, run}};
      if ((err = launch_pack_group(kv, 2, s_l, strm)) != hipSuccess) return ULY_ERR_HIP;
      kv_lo = g0;
      kv_hi = g1;
    }
    const int64_t qoff = ((int64_t)rank * Hq_l + c0) * hb, qrun = (int64_t)nq * hb;
    if ((err = launch_pack(qs, qc, P, s_l, qrow, qoff, qrun, strm)) != hipSuccess) return ULY_ERR_HIP;

    AttnArgs a = make_args(s, nq, 1, d, scale, causal, cu_seqlens, n_docs);
    a.q_row = (int64_t)nq * d;
    a.kv_row = (int64_t)(g1 - g0) * d;
    a.n_heads = nq;
    a.n_kv = g1 - g0;
    a.G = G;
    a.q_off = c0;   // chunk head j is local head c0 + j
    a.kv_off = g0;  // which reads local kv head (c0 + j) / G, stored at index - g0
    a.q = qc;
    a.k = kc;
    a.v = vc;
    a.out = oc;
    // the residual of the chunk's heads, in the rank's [s, Hq/P, d] layout
    a.o_lo = o_lo == nullptr ? nullptr : static_cast<char*>(o_lo) + c0 * hb;
    a.lo_row = (int64_t)Hq_l * d;
    a.lse_out = lse + (int64_t)c0 * s;
    st = fwd_dispatch(a, d, dtype, strm);
    if (st != ULY_OK) return st;
    if ((err = launch_unpack(oc, os, P, s_l, qrow, qoff, qrun, strm)) != hipSuccess) return ULY_ERR_HIP;
  }
  return ULY_OK;
}

// ---------------------------------------------------------------------------------------
// Headwise-chunked backward. Workspace, in order (each part 256-byte aligned):
//   Q, O, dO, dQ chunks        4 x [s, u, d]            element type
//   K, V chunks                2 x [s, span, d]          element type
//   delta of the chunk         [u, s]                    fp32
//   dK, dV accumulators        2 x [s, Hkv/P, d]         fp32
//   dK, dV of the rank         2 x [s, Hkv/P, d]         element type

int attn_fwd_shards(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards,
                    void* const* o_shards, void* o_lo, float* lse, int P, int rank, int64_t s_l, int Hq, int Hkv,
                    int d, int dtype, float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_shards || !k_shards || !v_shards || !o_shards || !lse) return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, Hq);
  if (st != ULY_OK) return st;
  if (Hkv < 1 || Hkv % P != 0 || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (dtype != ULY_BF16 || s_l % 128 != 0) return ULY_ERR_UNSUPPORTED;
  const int64_t s = (int64_t)P * s_l;
  if (s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  if (cu_seqlens != nullptr && n_docs < 1) return ULY_ERR_SHAPE;
  if (!aligned16(lse)) return ULY_ERR_ALIGN;
  if (workspace != nullptr && !aligned16(workspace)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  const int Hq_l = Hq / P, Hkv_l = Hkv / P;
  ShardSrc src{};
  for (int p = 0; p < P; ++p) {
    const void* ptrs[4] = {q_shards[p], k_shards[p], v_shards[p], o_shards[p]};
    for (const void* x : ptrs) {
      if (!x) return ULY_ERR_NULL;
      if (!aligned16(x)) return ULY_ERR_ALIGN;
    }
    // the rank's head 0 in each shard (bf16 elements)
    src.q[p] = static_cast<const uint16_t*>(q_shards[p]) + (int64_t)rank * Hq_l * d;
    src.k[p] = static_cast<const uint16_t*>(k_shards[p]) + (int64_t)rank * Hkv_l * d;
    src.v[p] = static_cast<const uint16_t*>(v_shards[p]) + (int64_t)rank * Hkv_l * d;
    src.o[p] = static_cast<uint16_t*>(o_shards[p]) + (int64_t)rank * Hq_l * d;
  }
  src.s_l = s_l;
  AttnArgs a = make_args(s, Hq_l, Hkv_l, d, scale, causal, cu_seqlens, n_docs);
  a.q_row = (int64_t)Hq * d;  // rows of the sequence shards hold every head
  a.kv_row = (int64_t)Hkv * d;
  a.o_lo = o_lo;  // the rank's [s, Hq/P, d] layout
  a.lo_row = (int64_t)Hq_l * d;
  a.lse_out = lse;
  const size_t part = attn_fwd_workspace_bytes(s, Hq_l, d);
  if (part > 0 && workspace != nullptr && workspace_bytes >= part) {  // as attn_fwd: short grids split
    a.nsplit_o = fwd_split_count(s, Hq_l);
    a.o_part = static_cast<float*>(workspace);
    a.o_stat = a.o_part + fwd_part_floats(s, Hq_l, d);
  }
  return hip_status(launch_attn_fwd_bf16_shards(a, src, d, as_stream(stream)));
}

int attn_bwd_shards(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards,
                    const void* const* o_shards, const void* o_lo, const float* lse, const void* const* do_shards,
                    void* const* dq_shards, void* const* dk_shards, void* const* dv_shards, int P, int rank,
                    int64_t s_l, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                    const int32_t* cu_seqlens, int n_docs, void* workspace, size_t* workspace_bytes,
                    void* stream) {
  if (!q_shards || !k_shards || !v_shards || !o_shards || !do_shards || !dq_shards || !dk_shards || !dv_shards)
    return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, Hq);
  if (st != ULY_OK) return st;
  if (Hkv < 1 || Hkv % P != 0 || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (dtype != ULY_BF16 || s_l % 128 != 0) return ULY_ERR_UNSUPPORTED;
  const int64_t s = (int64_t)P * s_l;
  if (s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  if (cu_seqlens != nullptr && n_docs < 1) return ULY_ERR_SHAPE;
  const int Hq_l = Hq / P, Hkv_l = Hkv / P;
  // delta, then (optional) the partial sums of the split dK/dV and dQ runs in one region
  const size_t dpart = delta_bytes(s, Hq_l);
  const size_t kvp = attn_bwd_dkdv_workspace_bytes(s, Hkv_l, d), qp = attn_bwd_dq_workspace_bytes(s, Hq_l, d);
  if (workspace == nullptr) {
    if (!workspace_bytes) return ULY_ERR_NULL;
    *workspace_bytes = dpart + round256(std::max(kvp, qp));
    return ULY_OK;
  }
  // without a stated capacity only delta is assumed (the partial region is used when stated)
  const size_t cap = workspace_bytes ? *workspace_bytes : dpart;
  if (cap < dpart) return ULY_ERR_WORKSPACE;
  if (!lse) return ULY_ERR_NULL;
  if (!aligned16(lse) || !aligned16(workspace)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  BwdSrc src{};
  const int64_t qo = (int64_t)rank * Hq_l * d, kvo = (int64_t)rank * Hkv_l * d;  // bf16 elements
  for (int p = 0; p < P; ++p) {
    const void* ptrs[8] = {q_shards[p], k_shards[p], v_shards[p], o_shards[p], do_shards[p],
                           dq_shards[p], dk_shards[p], dv_shards[p]};
    for (const void* x : ptrs) {
      if (!x) return ULY_ERR_NULL;
      if (!aligned16(x)) return ULY_ERR_ALIGN;
    }
    src.q.p[p] = static_cast<const uint16_t*>(q_shards[p]) + qo;
    src.o.p[p] = static_cast<const uint16_t*>(o_shards[p]) + qo;
    src.g.p[p] = static_cast<const uint16_t*>(do_shards[p]) + qo;
    src.dq.p[p] = static_cast<const uint16_t*>(dq_shards[p]) + qo;
    src.k.p[p] = static_cast<const uint16_t*>(k_shards[p]) + kvo;
    src.v.p[p] = static_cast<const uint16_t*>(v_shards[p]) + kvo;
    src.dk.p[p] = static_cast<const uint16_t*>(dk_shards[p]) + kvo;
    src.dv.p[p] = static_cast<const uint16_t*>(dv_shards[p]) + kvo;
  }
  src.s_l = s_l;
  float* delta = static_cast<float*>(workspace);
  AttnArgs a = make_args(s, Hq_l, Hkv_l, d, scale, causal, cu_seqlens, n_docs);
  a.q_row = (int64_t)Hq * d;  // rows of the sequence shards hold every head
  a.kv_row = (int64_t)Hkv * d;
  a.dkv_row = (int64_t)Hkv * d;
  a.lse_in = lse;
  a.delta = delta;
  AttnArgs pre = a;
  pre.lse_out = delta;
  pre.o_lo = const_cast<void*>(o_lo);  // the rank's [s, Hq/P, d] layout
  pre.lo_row = (int64_t)Hq_l * d;
  hipStream_t strm = as_stream(stream);
  hipError_t err;
  // as attn_bwd: short grids split dK/dV and dQ when the partial region is there
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + dpart);
  AttnArgs akv = a, aq = a;
  if (kvp > 0 && cap - dpart >= kvp) {
    akv.nsplit = dkdv_split_count(s, Hkv_l);
    akv.dkv_part = part;
  }
  if (qp > 0 && cap - dpart >= qp) {
    aq.nsplit_q = dq_split_count(s, Hq_l);
    aq.dq_part = part;
  }
  if ((err = launch_bwd_preprocess_bf16_shards(pre, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
  if ((err = launch_attn_dkdv_bf16_shards(akv, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
  if ((err = launch_attn_dq_bf16_shards(aq, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
  return ULY_OK;
}

// ---- Ring Attention (the pages' comparison workload) -----------------------------------
// Hop i of rank r attends to the K/V block of rank (r - i) mod P; causal: the own block is
// causal inside, earlier blocks are fully visible, later ones are skipped.

namespace {
int ring_hops(int P, int rank, int causal, int* srcs) {
  int n = 0;
  for (int i = 0; i < P; ++i) {
    const int src = ((rank - i) % P + P) % P;
    if (causal && src > rank) continue;
    srcs[n++] = src;
  }
  return n;
}

struct RingFwdLayout {
  size_t part, part_lo, part_lse, acc, acc_lse, total;
};
RingFwdLayout ring_fwd_layout(int64_t s_l, int Hq, int d) {
  RingFwdLayout L;
  const size_t n = (size_t)s_l * (size_t)Hq * (size_t)d;
  L.part = round256(n * 2);
  L.part_lo = round256(n * 2);
  L.part_lse = round256((size_t)s_l * Hq * sizeof(float));
  L.acc = round256(n * sizeof(float));
  L.acc_lse = round256((size_t)s_l * Hq * sizeof(float));
  L.total = L.part + L.part_lo + L.part_lse + L.acc + L.acc_lse;
  return L;
}

// checks shared by the ring calls: P shards of Q, K, V (all heads), bf16
int check_ring(const void* const* qs, const void* const* ks, const void* const* vs, int P, int rank, int64_t s_l,
               int Hq, int Hkv, int d, int dtype) {
  if (!qs || !ks || !vs) return ULY_ERR_NULL;
  if (P < 1 || P > ULY_MAX_RANKS || rank < 0 || rank >= P || s_l < 1) return ULY_ERR_SHAPE;
  if (Hq < 1 || Hkv < 1 || Hq > ULY_MAX_HEADS || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  if (s_l > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  int st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (dtype != ULY_BF16) return ULY_ERR_UNSUPPORTED;
  for (int p = 0; p < P; ++p) {
    if (!qs[p] || !ks[p] || !vs[p]) return ULY_ERR_NULL;
    if (!aligned16(qs[p]) || !aligned16(ks[p]) || !aligned16(vs[p])) return ULY_ERR_ALIGN;
  }
  return ULY_OK;
}
}  // namespace

size_t ring_attn_fwd_workspace_bytes(int64_t s_l, int Hq, int d) {
  if (s_l < 1 || Hq < 1 || d < 1) return 0;
  return ring_fwd_layout(s_l, Hq, d).total;
}

int ring_attn_fwd(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards, void* o,
                  void* o_lo, float* lse, int P, int rank, int64_t s_l, int Hq, int Hkv, int d, int dtype, float scale,
                  int causal, void* workspace, size_t* workspace_bytes, void* stream) {
  int st = check_ring(q_shards, k_shards, v_shards, P, rank, s_l, Hq, Hkv, d, dtype);
  if (st != ULY_OK) return st;
  const RingFwdLayout L = ring_fwd_layout(s_l, Hq, d);
  if (workspace == nullptr) {
    if (!workspace_bytes) return ULY_ERR_NULL;
    *workspace_bytes = L.total;
    return ULY_OK;
  }
  if (workspace_bytes && *workspace_bytes < L.total) return ULY_ERR_WORKSPACE;
  if (!o || !lse) return ULY_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(workspace)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  char* ws = static_cast<char*>(workspace);
  void* part = ws;
  void* part_lo = ws + L.part;
  float* part_lse = reinterpret_cast<float*>(ws + L.part + L.part_lo);
  float* acc = reinterpret_cast<float*>(ws + L.part + L.part_lo + L.part_lse);
  float* acc_lse = reinterpret_cast<float*>(ws + L.part + L.part_lo + L.part_lse + L.acc);
  int srcs[ULY_MAX_RANKS];
  const int n = ring_hops(P, rank, causal, srcs);
  hipStream_t strm = as_stream(stream);
  for (int i = 0; i < n; ++i) {
    const int src = srcs[i];
    AttnArgs a = make_args(s_l, Hq, Hkv, d, scale, causal && src == rank, nullptr, 0);
    a.q = q_shards[rank];
    a.k = k_shards[src];
    a.v = v_shards[src];
    a.out = part;
    a.o_lo = part_lo;
    a.lo_row = (int64_t)Hq * d;
    a.lse_out = part_lse;
    if ((st = fwd_dispatch(a, d, dtype, strm)) != ULY_OK) return st;
    const hipError_t e = launch_ring_merge(part, part_lo, part_lse, acc, acc_lse, o, o_lo, lse, s_l, Hq, d, i == 0,
                                           i == n - 1, strm);
    if (e != hipSuccess) return ULY_ERR_HIP;
  }
  return ULY_OK;
}

size_t ring_attn_bwd_workspace_bytes(int64_t s_l, int Hq, int d) {
  if (s_l < 1 || Hq < 1 || d < 1) return 0;
  return round256((size_t)s_l * Hq * sizeof(float)) + round256((size_t)s_l * Hq * d * sizeof(float));
}

int ring_attn_bwd(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards,
                  const void* o, const void* o_lo, const float* lse, const void* dout, void* dq, float* dk_acc,
                  float* dv_acc, void* const* dk_shards, void* const* dv_shards, int P, int rank, int64_t s_l, int Hq,
                  int Hkv, int d, int dtype, float scale, int causal, void* workspace, size_t* workspace_bytes,
                  void* stream) {
  int st = check_ring(q_shards, k_shards, v_shards, P, rank, s_l, Hq, Hkv, d, dtype);
  if (st != ULY_OK) return st;
  const size_t need = ring_attn_bwd_workspace_bytes(s_l, Hq, d);
  if (workspace == nullptr) {
    if (!workspace_bytes) return ULY_ERR_NULL;
    *workspace_bytes = need;
    return ULY_OK;
  }
  if (workspace_bytes && *workspace_bytes < need) return ULY_ERR_WORKSPACE;
  if (!o || !lse || !dout || !dq || !dk_acc || !dv_acc || !dk_shards || !dv_shards) return ULY_ERR_NULL;
  if (!aligned16(o) || !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk_acc) ||
      !aligned16(dv_acc) || !aligned16(workspace))
    return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  for (int p = 0; p < P; ++p) {
    if (!dk_shards[p] || !dv_shards[p]) return ULY_ERR_NULL;
    if (!aligned16(dk_shards[p]) || !aligned16(dv_shards[p])) return ULY_ERR_ALIGN;
  }
  float* delta = static_cast<float*>(workspace);
  float* dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)s_l * Hq * sizeof(float)));
  hipStream_t strm = as_stream(stream);
  if ((st = attn_bwd_preprocess(o, o_lo, dout, delta, s_l, Hq, d, dtype, stream)) != ULY_OK) return st;
  int srcs[ULY_MAX_RANKS];
  const int n = ring_hops(P, rank, causal, srcs);
  const size_t blk = (size_t)s_l * Hkv * d;  // fp32 elements of one block's dK (dV) sums
  for (int i = 0; i < n; ++i) {
    const int src = srcs[i];
    AttnArgs a = make_args(s_l, Hq, Hkv, d, scale, causal && src == rank, nullptr, 0);
    a.q = q_shards[rank];
    a.k = k_shards[src];
    a.v = v_shards[src];
    a.dout = dout;
    a.lse_in = lse;
    a.delta = delta;
    // block src's dK/dV sums travel with its K/V: the first rank to attend to it starts them,
    // the last rank of the ring rounds them into the block's gradient shards
    AttnArgs kv = a;
    kv.acc_k = dk_acc + (size_t)src * blk;
    kv.acc_v = dv_acc + (size_t)src * blk;
    kv.acc_init = rank == (causal ? src : 0) ? 1 : 0;
    kv.acc_final = rank == P - 1 ? 1 : 0;
    kv.out_k = dk_shards[src];
    kv.out_v = dv_shards[src];
    if (launch_attn_dkdv_bf16(kv, d, strm) != hipSuccess) return ULY_ERR_HIP;
    // this rank's dQ: summed over its hops
    AttnArgs qa = a;
    qa.out = dq;
    qa.acc_q = dq_acc;
    qa.acc_init = i == 0 ? 1 : 0;
    qa.acc_final = i == n - 1 ? 1 : 0;
    if (launch_attn_dq_bf16(qa, d, strm) != hipSuccess) return ULY_ERR_HIP;
  }
  return ULY_OK;
}

size_t attn_bwd_chunked_workspace_bytes(int P, int64_t s_l, int Hq, int Hkv, int d, int dtype,
                                        int heads_per_chunk) {
  if (P < 1 || s_l < 1 || Hq < 1 || Hkv < 1 || d < 1 || heads_per_chunk < 1) return 0;
  if (Hq % P != 0 || Hkv % P != 0 || Hq % Hkv != 0) return 0;
  const int u = std::min(heads_per_chunk, Hq / P);
  if (chunks_read_shards(dtype, s_l)) return bwd_shard_chunk_bytes(P, s_l, Hq, Hkv, d, u);
  return bwd_chunk_layout(P, s_l, Hq, Hkv, d, dtype, u).total;
}

int attn_bwd_chunked(const void* const* q_shards, const void* const* k_shards, const void* const* v_shards,
                     const void* const* o_shards, const void* o_lo, const float* lse, const void* const* do_shards,
                     void* const* dq_shards, void* const* dk_shards, void* const* dv_shards, int P, int rank,
                     int64_t s_l, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                     const int32_t* cu_seqlens, int n_docs, int heads_per_chunk, void* workspace,
                     size_t* workspace_bytes, void* stream) {
  if (!q_shards || !k_shards || !v_shards || !o_shards || !do_shards || !dq_shards || !dk_shards || !dv_shards)
    return ULY_ERR_NULL;
  int st = check_ranks(P, rank, s_l, Hq);
  if (st != ULY_OK) return st;
  if (Hkv < 1 || Hkv % P != 0 || Hq % Hkv != 0) return ULY_ERR_SHAPE;
  st = check_dtype_dim(dtype, d);
  if (st != ULY_OK) return st;
  if (heads_per_chunk < 1) return ULY_ERR_SHAPE;
  const int64_t s = (int64_t)P * s_l;
  if (s > (int64_t)INT32_MAX) return ULY_ERR_SHAPE;
  if (cu_seqlens != nullptr && n_docs < 1) return ULY_ERR_SHAPE;
  const size_t need = attn_bwd_chunked_workspace_bytes(P, s_l, Hq, Hkv, d, dtype, heads_per_chunk);
  if (workspace == nullptr) {
    if (!workspace_bytes) return ULY_ERR_NULL;
    *workspace_bytes = need;
    return ULY_OK;
  }
  if (workspace_bytes && *workspace_bytes < need) return ULY_ERR_WORKSPACE;
  if (!lse) return ULY_ERR_NULL;
  if (!aligned16(lse) || !aligned16(workspace)) return ULY_ERR_ALIGN;
  if ((st = check_o_lo(o_lo, dtype)) != ULY_OK) return st;
  for (int p = 0; p < P; ++p) {
    const void* ptrs[8] = {q_shards[p], k_shards[p], v_shards[p], o_shards[p], do_shards[p],
                           dq_shards[p], dk_shards[p], dv_shards[p]};
    for (const void* x : ptrs) {
      if (!x) return ULY_ERR_NULL;
      if (!aligned16(x)) return ULY_ERR_ALIGN;
    }
  }
  const int Hq_l = Hq / P, Hkv_l = Hkv / P, G = Hq / Hkv;
  const int u = std::min(heads_per_chunk, Hq_l);
  const int64_t e = esize(dtype);
  const int64_t qrow = (int64_t)Hq * d * e, kvrow = (int64_t)Hkv * d * e, hb = (int64_t)d * e;
  if (!chunks_fit(P, s_l, qrow, qrow) || !chunks_fit(P, s_l, kvrow, kvrow)) return ULY_ERR_SHAPE;

  hipStream_t strm = as_stream(stream);
  hipError_t err;
  if (chunks_read_shards(dtype, s_l)) {
    // each chunk's heads read from the shards and dQ written into them; dK/dV of a kv head summed
    // in fp32 across the chunks that read it and rounded, by its last one, straight into the shards
    char* ws = static_cast<char*>(workspace);
    float* delta = reinterpret_cast<float*>(ws);
    float* acc_k = reinterpret_cast<float*>(ws + round256((size_t)u * s * sizeof(float)));
    float* acc_v = acc_k + round256(s * (size_t)Hkv_l * d * sizeof(float)) / sizeof(float);
    for (int c0 = 0; c0 < Hq_l; c0 += u) {
      const int c1 = std::min(c0 + u, Hq_l), nq = c1 - c0;
      const int g0 = c0 / G, g1 = (c1 - 1) / G + 1;
      BwdSrc src{};
      const int64_t qo = ((int64_t)rank * Hq_l + c0) * d, kvo = ((int64_t)rank * Hkv_l + g0) * d;
      for (int p = 0; p < P; ++p) {
        src.q.p[p] = static_cast<const uint16_t*>(q_shards[p]) + qo;
        src.o.p[p] = static_cast<const uint16_t*>(o_shards[p]) + qo;
        src.g.p[p] = static_cast<const uint16_t*>(do_shards[p]) + qo;
        src.dq.p[p] = static_cast<const uint16_t*>(dq_shards[p]) + qo;
        src.k.p[p] = static_cast<const uint16_t*>(k_shards[p]) + kvo;
        src.v.p[p] = static_cast<const uint16_t*>(v_shards[p]) + kvo;
        src.dk.p[p] = static_cast<const uint16_t*>(dk_shards[p]) + kvo;
        src.dv.p[p] = static_cast<const uint16_t*>(dv_shards[p]) + kvo;
      }
      src.s_l = s_l;
      AttnArgs a = make_args(s, nq, 1, d, scale, causal, cu_seqlens, n_docs);
      a.q_row = (int64_t)Hq * d;
      a.kv_row = (int64_t)Hkv * d;
      a.dkv_row = (int64_t)Hkv * d;
      a.n_heads = nq;
      a.n_kv = g1 - g0;
      a.G = G;
      a.q_off = c0;
      a.kv_off = g0;
      a.lse_in = lse + (int64_t)c0 * s;
      a.delta = delta;
      AttnArgs pre = a;
      pre.lse_out = delta;
      pre.o_lo = o_lo == nullptr ? nullptr : const_cast<char*>(static_cast<const char*>(o_lo)) + c0 * hb;
      pre.lo_row = (int64_t)Hq_l * d;
      if ((err = launch_bwd_preprocess_bf16_shards(pre, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
      AttnArgs kv = a;
      kv.acc_k = acc_k + (int64_t)g0 * d;
      kv.acc_v = acc_v + (int64_t)g0 * d;
      kv.acc_row = (int64_t)Hkv_l * d;
      if ((err = launch_attn_dkdv_bf16_shards(kv, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
      if ((err = launch_attn_dq_bf16_shards(a, src, d, strm)) != hipSuccess) return ULY_ERR_HIP;
    }
    return ULY_OK;
  }
  const BwdChunkLayout L = bwd_chunk_layout(P, s_l, Hq, Hkv, d, dtype, u);
  char* ws = static_cast<char*>(workspace);
  void* qc = ws;
  void* oc = ws + L.qc;
  void* gc = ws + 2 * L.qc;
  void* dqc = ws + 3 * L.qc;
  void* kc = ws + 4 * L.qc;
  void* vc = ws + 4 * L.qc + L.kv;
  float* delta = reinterpret_cast<float*>(ws + 4 * L.qc + 2 * L.kv);
  float* acc_k = reinterpret_cast<float*>(ws + 4 * L.qc + 2 * L.kv + L.delta);
  float* acc_v = reinterpret_cast<float*>(ws + 4 * L.qc + 2 * L.kv + L.delta + L.acc);
  char* dk_r = ws + 4 * L.qc + 2 * L.kv + L.delta + 2 * L.acc;
  char* dv_r = dk_r + L.out;
  const ShardPtrs qs = shard_ptrs(q_shards, P), ks = shard_ptrs(k_shards, P), vs = shard_ptrs(v_shards, P);
  const ShardPtrs os = shard_ptrs(o_shards, P), gs = shard_ptrs(do_shards, P);
  const ShardPtrs dqs = shard_ptrs(const_cast<const void* const*>(dq_shards), P);
  const ShardPtrs dks = shard_ptrs(const_cast<const void* const*>(dk_shards), P);
  const ShardPtrs dvs = shard_ptrs(const_cast<const void* const*>(dv_shards), P);

  int kv_lo = -1, kv_hi = -1;  // local kv heads currently packed in kc / vc
  for (int c0 = 0; c0 < Hq_l; c0 += u) {
    const int c1 = std::min(c0 + u, Hq_l), nq = c1 - c0;
    const int g0 = c0 / G, g1 = (c1 - 1) / G + 1;
    if (g0 != kv_lo || g1 != kv_hi) {
      const int64_t off = ((int64_t)rank * Hkv_l + g0) * hb, run = (int64_t)(g1 - g0) * hb;
      const PermSeg kv[2] = {{ks, kc, P, kvrow, off, run}, {vs, vc, P, kvrow, off, run}};
      if ((err = launch_pack_group(kv, 2, s_l, strm)) != hipSuccess) return ULY_ERR_HIP;
      kv_lo = g0;
      kv_hi = g1;
    }
    const int64_t qoff = ((int64_t)rank * Hq_l + c0) * hb, qrun = (int64_t)nq * hb;
    const PermSeg qog[3] = {{qs, qc, P, qrow, qoff, qrun}, {os, oc, P, qrow, qoff, qrun}, {gs, gc, P, qrow, qoff, qrun}};
    if ((err = launch_pack_group(qog, 3, s_l, strm)) != hipSuccess) return ULY_ERR_HIP;

    AttnArgs a = make_args(s, nq, 1, d, scale, causal, cu_seqlens, n_docs);
    a.q_row = (int64_t)nq * d;
    a.kv_row = (int64_t)(g1 - g0) * d;
    a.n_heads = nq;
    a.n_kv = g1 - g0;
    a.G = G;
    a.q_off = c0;   // chunk head j is local head c0 + j
    a.kv_off = g0;  // which reads local kv head (c0 + j) / G, stored at index - g0
    a.q = qc;
    a.k = kc;
    a.v = vc;
    a.o = oc;
    a.dout = gc;
    a.lse_in = lse + (int64_t)c0 * s;
    a.delta = delta;
    // delta of the chunk's heads
    AttnArgs pre = a;
    pre.lse_out = delta;
    // the residual of the chunk's heads, in the rank's [s, Hq/P, d] layout
    pre.o_lo = o_lo == nullptr ? nullptr : const_cast<char*>(static_cast<const char*>(o_lo)) + c0 * hb;
    pre.lo_row = (int64_t)Hq_l * d;
    if ((err = launch_bwd_preprocess(pre, d, dtype, strm)) != hipSuccess) return ULY_ERR_HIP;
    // dK/dV of kv heads [g0, g1): fp32 sums carried across chunks, rounded on the last one
    AttnArgs kvargs = a;
    kvargs.dkv_row = (int64_t)Hkv_l * d;
    kvargs.acc_row = (int64_t)Hkv_l * d;
    kvargs.acc_k = acc_k + (int64_t)g0 * d;
    kvargs.acc_v = acc_v + (int64_t)g0 * d;
    kvargs.out_k = dk_r + (int64_t)g0 * hb;
    kvargs.out_v = dv_r + (int64_t)g0 * hb;
    err = dtype == ULY_BF16 ? launch_attn_dkdv_bf16(kvargs, d, strm) : launch_attn_dkdv_f32(kvargs, d, strm);
    if (err != hipSuccess) return ULY_ERR_HIP;
    // dQ of the chunk's heads
    AttnArgs qargs = a;
    qargs.out = dqc;
    err = dtype == ULY_BF16 ? launch_attn_dq_bf16(qargs, d, strm) : launch_attn_dq_f32(qargs, d, strm);
    if (err != hipSuccess) return ULY_ERR_HIP;
    if ((err = launch_unpack(dqc, dqs, P, s_l, qrow, qoff, qrun, strm)) != hipSuccess) return ULY_ERR_HIP;
  }
  const int64_t kvoff = (int64_t)rank * Hkv_l * hb, kvrun = (int64_t)Hkv_l * hb;
  const PermSeg dkv[2] = {{dks, dk_r, P, kvrow, kvoff, kvrun}, {dvs, dv_r, P, kvrow, kvoff, kvrun}};
  if ((err = launch_unpack_group(dkv, 2, s_l, strm)) != hipSuccess) return ULY_ERR_HIP;
  return ULY_OK;
}

}  // extern "C"
