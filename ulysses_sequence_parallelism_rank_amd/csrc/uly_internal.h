// Host-side declarations shared by the translation units of libulysses (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ulysses.h"

namespace uly {

// The P shard base pointers, passed to kernels by value.
struct ShardPtrs {
  const void* p[ULY_MAX_RANKS];
};

// Attention problem description shared by the forward and backward kernels.
//   q / o / do / dq : [s, q_heads, D], row stride q_row elements
//   k / v           : [s, kv_heads, D], row stride kv_row elements
//   dk / dv         : [s, kv_heads, D], row stride dkv_row elements
// q head h (0 <= h < n_heads of the launch) reads kv head (h + q_off) / G - kv_off, so the
// q heads of the launch that read kv head g are [max(lo, 0), min(lo + G, n_heads)) with
// lo = (g + kv_off) G - q_off (the launch may hold a chunk of a GQA group).
// lse / delta rows are [n_heads][s] with row stride lse_row.
// dK/dV accumulation across launches (headwise-chunked backward): when acc_k is set, the
// dK/dV kernel adds its sums to the fp32 arrays acc_k / acc_v ([s, kv_heads, D], row stride
// acc_row) unless the launch holds the first q head of the kv head's group, and writes the
// rounded result to dk / dv only when it holds the last one (otherwise it stores the fp32
// sum back).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse_in;
  const float* delta;
  void* out;      // o (forward) or dq
  void* out_k;    // dk
  void* out_v;    // dv
  float* acc_k;   // fp32 dK accumulator (chunked backward) or null
  float* acc_v;   // fp32 dV accumulator
  int64_t acc_row;
  int64_t dkv_row;
  float* lse_out; // forward LSE / preprocess delta
  // O's bf16 rounding residual ([s, n_heads, D] bf16 at the launch's head 0, row stride lo_row):
  // the bf16 forward writes O_fp32 - bf16(O_fp32) rounded to bf16 here when it is set, and the
  // preprocess then forms delta from O + o_lo; null: not written / delta from O alone
  void* o_lo;
  int64_t lo_row;
  int64_t s;
  int64_t q_row, kv_row;
  int64_t lse_row;
  int n_heads;    // q heads processed by the launch
  int n_kv;       // kv heads (dkdv launch)
  int G, q_off, kv_off;
  float scale;
  int causal;
  const int32_t* cu;
  int n_docs;
  // accumulation across launches, when acc_k / acc_v (dK/dV) or acc_q (dQ, [s, n_heads, D] fp32
  // with row stride q_row) are set: acc_init / acc_final say whether this launch starts the sums
  // (does not read them) and ends them (rounds into the output instead of storing fp32); -1 in
  // the dK/dV kernel means "from the launch's q heads" (the headwise-chunked rule above)
  float* acc_q;
  int acc_init, acc_final;
  // dK/dV of one key block split over nsplit workgroups (small grids): workgroup sp walks its
  // share of the block's steps and stores fp32 partial sums (dV then dK, [128 keys][D] each) in
  // slot ((kv head * key blocks + block) * nsplit + sp) of dkv_part; a reduce kernel sums the
  // slots in split order and rounds. nsplit 1: no partials (and no accumulation across launches
  // combined with a split).
  int nsplit;
  float* dkv_part;
  // dQ of one 128-row block split over nsplit_q workgroups (small grids): workgroup sp walks its
  // share of the block's key tiles and stores its fp32 partial sums (unscaled, [128 rows][D]) in
  // slot ((q head * row blocks + block) * nsplit_q + sp) of dq_part; a reduce kernel sums the
  // slots in split order, scales and rounds. Values below 2: no split (no accumulation across
  // launches is combined with a split).
  int nsplit_q;
  float* dq_part;
  // forward of one 128-row block split over nsplit_o workgroups (small grids): workgroup sp
  // walks its share of the block's key tiles and stores, in slot ((q head * row blocks + block)
  // * nsplit_o + sp), its unnormalised fp32 O sums ([128 rows][D], of o_part) and per row its
  // running max (log2 units), fp32 weight sum and rounded-weight sum ([128 rows][4], of
  // o_stat); a combine kernel merges the slots in split order. Values below 2: no split.
  int nsplit_o;
  float* o_part;
  float* o_stat;
};
// dK/dV workgroups split per key block for a grid of n_kv * ceil(s/128) blocks (1 = no split)
int dkdv_split_count(int64_t s, int n_kv);
// dQ workgroups split per row block for a grid of n_heads * ceil(s/128) blocks (1 = no split)
int dq_split_count(int64_t s, int n_heads);
inline size_t dq_part_bytes(int64_t s, int n_heads, int d) {
  const int ns = dq_split_count(s, n_heads);
  return ns <= 1 ? 0 : (size_t)n_heads * (size_t)((s + 127) / 128) * (size_t)ns * 128 * (size_t)d * sizeof(float);
}
// forward workgroups split per row block for a grid of n_heads * ceil(s/128) blocks (1 = no split)
int fwd_split_count(int64_t s, int n_heads);
// o_part then o_stat, both in floats
inline size_t fwd_part_floats(int64_t s, int n_heads, int d) {
  const int ns = fwd_split_count(s, n_heads);
  return ns <= 1 ? 0 : (size_t)n_heads * (size_t)((s + 127) / 128) * (size_t)ns * 128 * (size_t)d;
}
inline size_t fwd_part_bytes(int64_t s, int n_heads, int d) {
  const size_t nf = fwd_part_floats(s, n_heads, d);
  return nf == 0 ? 0 : (nf + nf / (size_t)d * 4) * sizeof(float);
}
inline size_t dkdv_part_bytes(int64_t s, int n_kv, int d) {
  const int ns = dkdv_split_count(s, n_kv);
  return ns <= 1 ? 0 : (size_t)n_kv * (size_t)((s + 127) / 128) * (size_t)ns * 2 * 128 * (size_t)d * sizeof(float);
}

// One tensor of a grouped permute: its P shards (P of them used), the head-shard buffer, the
// shard row size, the byte offset of the rank's heads in a row and the bytes per row moved.
struct PermSeg {
  ShardPtrs sh;
  void* flat;
  int P;
  int64_t row_bytes, off_bytes, run_bytes;
};
constexpr int kPermGroupMax = ULY_PERM_GROUP_MAX;
// n tensors (1 <= n <= kPermGroupMax) packed / unpacked by one launch
hipError_t launch_pack_group(const PermSeg* segs, int n, int64_t s_l, hipStream_t stream);
hipError_t launch_unpack_group(const PermSeg* segs, int n, int64_t s_l, hipStream_t stream);
// send-side / receive-side permutes of one rank (head_bytes = d * element size, a multiple of 16)
hipError_t launch_send_pack(const void* shard, void* out, int P, int64_t s_l, int H, int64_t head_bytes,
                            hipStream_t stream);
hipError_t launch_recv_unpack(const void* in, void* shard, int P, int64_t s_l, int H, int64_t head_bytes, int bf16,
                              hipStream_t stream);
hipError_t launch_pack(const ShardPtrs& src, void* out, int P, int64_t s_l, int64_t row_bytes,
                       int64_t off_bytes, int64_t run_bytes, hipStream_t stream);
hipError_t launch_unpack(const void* in, const ShardPtrs& dst, int P, int64_t s_l, int64_t row_bytes,
                         int64_t off_bytes, int64_t run_bytes, hipStream_t stream);

// Where the forward kernel finds Q, K, V rows and writes O rows: row r of the sequence
// lives in shard r / s_l at row r % s_l (row strides q_row / kv_row of AttnArgs, the
// launch's head 0 at the table entry). One packed [s, H, d] buffer is the case of one
// shard with s_l = s; the sequence shards of the ranks are the case of P shards (every
// workgroup's 128 rows and every 64-key tile must then lie in one shard: s_l % 128 == 0).
struct ShardSrc {
  const void* q[ULY_MAX_RANKS];
  const void* k[ULY_MAX_RANKS];
  const void* v[ULY_MAX_RANKS];
  void* o[ULY_MAX_RANKS];
  int64_t s_l;
};

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t stream);
// the bf16 forward reading from / writing to shards (a.q/k/v/out are ignored)
hipError_t launch_attn_fwd_bf16_shards(const AttnArgs& a, const ShardSrc& src, int d, hipStream_t stream);
hipError_t launch_bwd_preprocess(const AttnArgs& a, int d, int dtype, hipStream_t stream);
hipError_t launch_attn_dkdv_bf16(const AttnArgs& a, int d, hipStream_t stream);
hipError_t launch_attn_dq_bf16(const AttnArgs& a, int d, hipStream_t stream);

// Shard tables of the backward's tensors (the layout of ShardSrc): q, k, v, o, dO read, dq,
// dk, dv written, each at the launch's head 0; a kernel receives only the tables it uses.
struct Shards {
  const void* p[ULY_MAX_RANKS];
};
struct BwdSrc {
  Shards q, k, v, o, g, dq, dk, dv;
  int64_t s_l;
};
// the three bf16 backward phases reading / writing through shard tables (a.q, a.k, a.v, a.o,
// a.dout, a.out, a.out_k, a.out_v are ignored)
hipError_t launch_bwd_preprocess_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream);
hipError_t launch_attn_dkdv_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream);
hipError_t launch_attn_dq_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream);
hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t stream);
// Ring Attention: merge one hop's partial (O bf16 + residual, LSE) into the fp32 running output;
// the last hop writes O (bf16), its residual (if out_lo) and the LSE
hipError_t launch_ring_merge(const void* part, const void* part_lo, const float* part_lse, float* acc, float* acc_lse,
                             void* out, void* out_lo, float* out_lse, int64_t s_l, int H, int d, int first, int last,
                             hipStream_t stream);
hipError_t launch_mfma_probe(int iters, int blocks, float* sink, unsigned long long* clocks, hipStream_t stream);
// kind 0: MFMA + LDS operand; 1: + 2 FMAs + 1 exp per product; 2: + 4 FMAs + 1 exp per product
hipError_t launch_mix_probe(int kind, int iters, int blocks, float* sink, hipStream_t stream);
hipError_t launch_attn_dkdv_f32(const AttnArgs& a, int d, hipStream_t stream);
hipError_t launch_attn_dq_f32(const AttnArgs& a, int d, hipStream_t stream);

}  // namespace uly
