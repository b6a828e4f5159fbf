/*
 * ulysses.h -- C ABI of one GPU's share of a Ulysses sequence-parallel attention layer
 * on MI355X (gfx950).
 *
 * What the share computes (pages: "Ulysses Sequence Parallelism: Training with
 * Million-Token Contexts", section "how Ulysses works", steps 1-5; tilnote.io
 * commentary, sections on what Ulysses changes and on activation memory):
 *   1. the local half of the first all-to-all: P sequence shards [s_l, H, d] (every
 *      head, a contiguous token chunk each) become one head shard [s, H/P, d]
 *      (every position, this rank's heads)    -> ulysses_pack (several tensors at once:
 *                                                ulysses_pack_group / ulysses_unpack_group)
 *   2. dense causal (optionally packed-document) attention over the whole sequence
 *      for the head shard, forward and backward                    -> attn_fwd, attn_bwd
 *   3. the local half of the second all-to-all: the head shard goes back to the
 *      sequence shards                                             -> ulysses_unpack
 *      (the send-side and receive-side permutes of a real all-to-all, with kv heads
 *      replicated when there are fewer than ranks -> ulysses_send_pack, ulysses_recv_unpack)
 *   4. the UPipe schedule: 1-3 run a few heads at a time so that the attention
 *      intermediates stay small                    -> attn_fwd_chunked, attn_bwd_chunked
 *   5. 1-3 with the exchange folded into the attention's own loads and stores: the
 *      kernels read the sequence shards directly      -> attn_fwd_shards, attn_bwd_shards
 *   6. the pages' comparison workload, Ring Attention   -> ring_attn_fwd, ring_attn_bwd
 * The P ranks are P separate device buffers on one GPU; no collective runs here.
 * uly_mfma_probe and uly_mix_probe are measurement helpers outside the path.
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers; arrays of pointers (the P shards) are HOST
 *     arrays read during the call only. Layouts are row-major with d fastest:
 *     a sequence shard is [s_l, H, d], a head shard [s, H_l, d], LSE [H_l, s] fp32.
 *   - Rank p holds tokens [p*s_l, (p+1)*s_l); rank r owns q heads [r*Hq/P, (r+1)*Hq/P)
 *     and kv heads [r*Hkv/P, (r+1)*Hkv/P). q head h reads kv head h / (Hq/Hkv).
 *   - dtype: ULY_BF16 (the tuned path; fp32 accumulation inside) or ULY_F32.
 *     d must be 64 or 128 (ULY_F32: 64 only).
 *   - Every call enqueues work on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream), returns without synchronising and allocates nothing. The caller
 *     owns every buffer. Inputs and outputs must not overlap.
 *   - All arguments are checked on the host before any launch; on error nothing is
 *     enqueued and the status says why. Device-array contents (cu_seqlens) are a
 *     precondition and are not checked.
 *   - Base pointers must be 16-byte aligned.
 *   - Status codes are the uly_status values below; uly_status_string() names them.
 *   - o_lo (optional, bf16 only, NULL allowed everywhere): the forward's bf16 O is O_fp32
 *     rounded once; o_lo receives that rounding's residual, O_fp32 - bf16(O_fp32), itself
 *     rounded to bf16, in the rank's head-shard layout [s, Hq_l, d] (Hq_l = the local q
 *     heads) whatever layout O has. A backward given the same o_lo forms
 *     delta_i = dO_i . (O_i + o_lo_i), i.e. from O to about 16 significant bits. Without it
 *     delta is formed from the bf16 O (the FlashAttention convention), whose rounding
 *     cancels against dP on rows where one key holds nearly all the softmax weight and
 *     then dominates dS there. ULY_ERR_UNSUPPORTED for a non-NULL o_lo with ULY_F32.
 */
#ifndef ULYSSES_H
#define ULYSSES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ULY_BF16 = 0, ULY_F32 = 1 } uly_dtype;

typedef enum {
  ULY_OK = 0,
  ULY_ERR_NULL = 1,        /* a required pointer is NULL */
  ULY_ERR_SHAPE = 2,       /* sizes inconsistent: P, rank, H % P, Hq % Hkv, s, ... */
  ULY_ERR_UNSUPPORTED = 3, /* dtype / head_dim combination not built */
  ULY_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned */
  ULY_ERR_WORKSPACE = 5,   /* workspace smaller than required */
  ULY_ERR_HIP = 6          /* a HIP launch or runtime call failed */
} uly_status;

#define ULY_MAX_RANKS 64
/* Largest head count (global or local) any call accepts: the kernels address a tile's rows
   (at most 128 rows of one tensor) with 32-bit byte offsets. Larger counts: ULY_ERR_SHAPE. */
#define ULY_MAX_HEADS 4096

/* Name of a status code (static string). */
const char* uly_status_string(int status);

/* ABI version, bumped on any signature change. */
int uly_abi_version(void);

/* ---------------------------------------------------------------------------
 * ulysses_pack -- local half of the first all-to-all (sequence shards -> head shard).
 * Pages: "how Ulysses works" steps 1 and 3 (each GPU ends up holding every sequence
 * position for a subset of heads); tilnote.io, section on what Ulysses changes.
 *   shards : host array of P device pointers, shard p is [s_l, H, d] of `dtype`
 *   P      : number of ranks, 1..ULY_MAX_RANKS;  rank in [0, P)
 *   H      : global head count, divisible by P (the commentary's divisibility rule)
 *   out    : device [P*s_l, H/P, d]; out[p*s_l + t, j, :] = shard_p[t, rank*H/P + j, :]
 * Bits are copied unchanged (bit-exact).
 * ------------------------------------------------------------------------- */
int ulysses_pack(const void* const* shards, int P, int rank, int64_t s_l, int H, int d,
                 int dtype, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * ulysses_unpack -- local half of the second all-to-all (head shard -> sequence shards);
 * also the backward of ulysses_pack. Pages: "how Ulysses works" step 5.
 *   in     : device [P*s_l, H/P, d]
 *   shards : host array of P device pointers [s_l, H, d]; for every p, t, j:
 *            shard_p[t, rank*H/P + j, :] = in[p*s_l + t, j, :]. Other heads untouched.
 * ------------------------------------------------------------------------- */
int ulysses_unpack(const void* in, int P, int rank, int64_t s_l, int H, int d, int dtype,
                   void* const* shards, void* stream);

/* ---------------------------------------------------------------------------
 * ulysses_pack_group / ulysses_unpack_group -- the permutes of several tensors that cross
 * the same all-to-all, in one launch. Pages: "how Ulysses works" steps 1 and 3 (the
 * forward exchange carries Q, K and V together; the backward one carries dQ, dK and dV).
 *   n       : number of tensors, 1..ULY_PERM_GROUP_MAX
 *   H       : host array of n global head counts, each divisible by P
 *   pack    : shards[i] is a host array of P device pointers [s_l, H[i], d]; out[i] is a
 *             device [P*s_l, H[i]/P, d] buffer; out[i] = ulysses_pack(shards[i], ...)
 *   unpack  : in[i] is a device [P*s_l, H[i]/P, d] buffer; head slice `rank` of the P shards
 *             shards[i] is written as by ulysses_unpack(in[i], ...)
 * Every tensor is checked as by ulysses_pack / ulysses_unpack before anything is enqueued;
 * the results are bit-identical to n separate calls (only the launch count differs).
 * ------------------------------------------------------------------------- */
#define ULY_PERM_GROUP_MAX 3
int ulysses_pack_group(int n, const void* const* const* shards, const int* H, void* const* out, int P,
                       int rank, int64_t s_l, int d, int dtype, void* stream);
int ulysses_unpack_group(int n, const void* const* in, const int* H, void* const* const* shards, int P,
                         int rank, int64_t s_l, int d, int dtype, void* stream);

/* ---------------------------------------------------------------------------
 * ulysses_send_pack / ulysses_recv_unpack -- the local permutes of one rank as a real
 * all-to-all needs them ("how Ulysses works", steps 1, 3 and 5): send_pack turns the rank's
 * sequence shard into P contiguous per-destination blocks, and recv_unpack turns the P blocks
 * a rank received back into its sequence shard. The collective between them moves block r of
 * rank p's send buffer to block p of rank r's receive buffer; on one GPU the ranks' buffers
 * are separate allocations and that move is the caller's. send_pack of every rank, the
 * exchange, and the receiving rank's buffer read as [P*s_l, H_l, d] give exactly
 * ulysses_pack's head shard.
 *   H heads over P ranks, H % P == 0 or P % H == 0 (ULY_ERR_SHAPE otherwise). Rank r receives
 *   H_l = H/P heads from r*H/P, or, when H < P, the one head r / (P/H): a head fewer than the
 *   ranks (the kv heads of a GQA model at large SP; the comparison table on the first page
 *   asks num_heads >= sp_size) is replicated to P/H ranks.
 *   send_pack   : shard [s_l, H, d] -> out [P, s_l, H_l, d]; out[r, t, j] = shard[t, first(r)+j]
 *   recv_unpack : in [P, s_l, H_l, d] -> shard [s_l, H, d]; shard[t, h] = in[r, t, h - first(r)]
 *                 for the rank r holding h (the bits unchanged), or, for a replicated head,
 *                 the sum over its P/H holders in rank order, in fp32 from +0, rounded once
 *                 to nearest even (the gradient of a head read by several ranks).
 *   d * element size must be a multiple of 16 (ULY_ERR_ALIGN); base pointers 16-byte aligned.
 * ------------------------------------------------------------------------- */
int ulysses_send_pack(const void* shard, int P, int64_t s_l, int H, int d, int dtype, void* out,
                      void* stream);
int ulysses_recv_unpack(const void* in, int P, int64_t s_l, int H, int d, int dtype, void* shard,
                        void* stream);

/* ---------------------------------------------------------------------------
 * attn_fwd -- attention forward of one head shard. Pages: "how Ulysses works" step 4
 * (local FlashAttention/SDPA on the assigned heads over every position); the
 * long-sequence section (FlashAttention: exact attention in O(n) memory); TRL
 * SFTTrainer section (packed documents).
 *   q [s, Hq, d], k, v [s, Hkv, d] : device, `dtype`; Hq = local q heads, Hq % Hkv == 0
 *   o [s, Hq, d]                   : device, `dtype`, written
 *   o_lo [s, Hq, d]                : device bf16 or NULL: O's rounding residual (above)
 *   lse [Hq, s]                    : device fp32, written; natural-log log-sum-exp of
 *                                    each row's visible scaled scores
 *   scale  : multiplies q.k (1/sqrt(d) for the standard layer)
 *   causal : 1 -> key j visible to row i iff j <= i; 0 -> all keys
 *   cu_seqlens : NULL, or device int32 [n_docs + 1], 0 = cu[0] < ... < cu[n_docs] = s;
 *                keys are then further restricted to the row's own document
 *   workspace : NULL, or device scratch (16-byte aligned, else ULY_ERR_ALIGN) of
 *               workspace_bytes bytes. A workgroup holds 128 rows of one q head; below 1152
 *               of them (short and mid-size sequences: one or one and a half rounds, in which
 *               the last row blocks, which see the most keys, set the time) and given
 *               attn_fwd_workspace_bytes(s, Hq, d) bytes (bf16), each row block's key tiles are
 *               split over up to 8 workgroups (aiming at 1024 below 768 of them, else 2) that
 *               store fp32 partial results (O sums, running max, weight sums),
 *               and a second kernel merges them in split order: deterministic; the last bits
 *               differ from the unsplit run. A smaller or NULL workspace runs unsplit. The
 *               size is 0 where no split applies.
 * Every row must see at least one key (true whenever causal or cu_seqlens is used).
 * ------------------------------------------------------------------------- */
size_t attn_fwd_workspace_bytes(int64_t s, int Hq, int d);
int attn_fwd(const void* q, const void* k, const void* v, void* o, void* o_lo, float* lse,
             int64_t s, int Hq, int Hkv, int d, int dtype, float scale, int causal,
             const int32_t* cu_seqlens, int n_docs, void* workspace, size_t workspace_bytes,
             void* stream);

/* ---------------------------------------------------------------------------
 * attn_bwd -- attention backward of one head shard: dq, dk, dv from dout, given the
 * forward's o and lse. Runs attn_bwd_preprocess, attn_bwd_dkdv and attn_bwd_dq.
 * The gradient of a kv head sums the G = Hq/Hkv q heads that read it.
 *   q, k, v, o, lse, dout : as produced/consumed by attn_fwd (dout shaped like o)
 *   o_lo  : the residual attn_fwd wrote, or NULL (delta then from the bf16 o)
 *   dq [s, Hq, d], dk, dv [s, Hkv, d] : device `dtype`, written (fully overwritten)
 *   workspace : device scratch of attn_bwd_workspace_bytes(s, Hq, Hkv, d) bytes: delta
 *               [Hq, s] fp32 (rounded up to 256 bytes; required) followed by room for the
 *               partial sums of a split run (attn_bwd_dkdv's, then attn_bwd_dq's in the same
 *               bytes; optional: a workspace that holds delta only runs both unsplit).
 *               If workspace == NULL the call only stores that size into
 *               *workspace_bytes and returns ULY_OK. Otherwise *workspace_bytes (if
 *               workspace_bytes != NULL) is the capacity and is checked.
 * Deterministic: no atomics, every output element is written by one thread.
 * ------------------------------------------------------------------------- */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* o_lo,
             const float* lse, const void* dout, void* dq, void* dk, void* dv,
             int64_t s, int Hq, int Hkv, int d, int dtype, float scale, int causal,
             const int32_t* cu_seqlens, int n_docs,
             void* workspace, size_t* workspace_bytes, void* stream);

size_t attn_bwd_workspace_bytes(int64_t s, int Hq, int Hkv, int d);

/* ---------------------------------------------------------------------------
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, and the same kernels (dK/dV and dQ unsplit), so the
 * results are bitwise those of attn_bwd wherever attn_bwd runs both unsplit (at least 512 key
 * blocks x kv heads, i.e. s * Hkv >= 65536, and at least 1024 row blocks x q heads, i.e.
 * ceil(s / 128) * Hq >= 1024). delta lives in a static device array of ULY_NOALLOC_MAX_DELTA floats
 * (16 MiB) that each GPU the library runs on holds until the process ends; the call
 * allocates nothing. s * Hq above ULY_NOALLOC_MAX_DELTA -> ULY_ERR_WORKSPACE; the array's
 * address not obtainable -> ULY_ERR_HIP. Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (other streams, other host threads) race and must be ordered
 * by the caller. Devices are numbered below ULY_MAX_DEVICES.
 * ------------------------------------------------------------------------- */
#define ULY_NOALLOC_MAX_DELTA (1 << 22)
#define ULY_MAX_DEVICES 64
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* o_lo,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     int64_t s, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                     const int32_t* cu_seqlens, int n_docs, void* stream);

/* The three phases of attn_bwd, exported so that each can be timed on its own.
 * delta [Hq, s] fp32: delta[h, i] = sum_x dout[i, h, x] * (o[i, h, x] + o_lo[i, h, x])
 * (o_lo NULL: the o term alone).                                                    */
int attn_bwd_preprocess(const void* o, const void* o_lo, const void* dout, float* delta,
                        int64_t s, int Hq, int d, int dtype, void* stream);
/* dk, dv for every key: per kv head, loops over the rows of its G q heads. A workgroup
 * holds 128 keys of one kv head and fills a CU; when fewer than 512 such workgroups would run
 * (short sequences: under two rounds of them, so the first key block, which sees every row,
 * sets the time) and a workspace of attn_bwd_dkdv_workspace_bytes(s, Hkv, d) bytes is
 * given (bf16), each key block's rows are split over up to 8 workgroups (aiming at 512) that
 * store fp32 partial sums, and a second kernel adds them in split order and rounds once:
 * still deterministic; the sums' order, and so the last bits, differ from the unsplit run.
 * The size is 0 when no split applies; a NULL or smaller workspace runs unsplit; a workspace
 * must be 16-byte aligned (ULY_ERR_ALIGN).                                                 */
size_t attn_bwd_dkdv_workspace_bytes(int64_t s, int Hkv, int d);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse,
                  const void* dout, const float* delta, void* dk, void* dv,
                  int64_t s, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                  const int32_t* cu_seqlens, int n_docs, void* workspace, size_t workspace_bytes,
                  void* stream);
/* dq for every row: loops over the visible keys. A workgroup holds 128 rows of one q head,
 * two share a CU; when fewer than 1024 such workgroups would run (short and mid-size
 * sequences: under two rounds, so the longest row blocks, which see the most keys, set the
 * time) and a workspace of
 * attn_bwd_dq_workspace_bytes(s, Hq, d) bytes is given (bf16), each row block's key tiles are
 * split over up to 8 workgroups (aiming at 1024) that store fp32 partial sums, and a second
 * kernel adds them in split order, scales and rounds once: deterministic; the sums' order,
 * and so the last bits, differ from the unsplit run. The size is 0 when no split applies;
 * a NULL or smaller workspace runs unsplit; a workspace must be 16-byte aligned
 * (ULY_ERR_ALIGN).                                                                    */
size_t attn_bwd_dq_workspace_bytes(int64_t s, int Hq, int d);
int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse,
                const void* dout, const float* delta, void* dq,
                int64_t s, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                const int32_t* cu_seqlens, int n_docs, void* workspace, size_t workspace_bytes,
                void* stream);

/* ---------------------------------------------------------------------------
 * attn_fwd_chunked -- the UPipe headwise-chunked forward of rank `rank` (tilnote.io
 * commentary, section on activation memory: process a few heads at a time to cut the
 * memory of attention intermediates). For each chunk of `heads_per_chunk` local q
 * heads (the last chunk may be smaller): pack those q heads and the kv heads they read
 * (kv heads are re-packed only when the range changes), run the forward, unpack the
 * chunk's output into the o shards. Same results as ulysses_pack + attn_fwd +
 * ulysses_unpack, with smaller intermediates.
 *   q_shards / o_shards : host arrays of P device pointers [s_l, Hq, d] (global Hq)
 *   k_shards / v_shards : host arrays of P device pointers [s_l, Hkv, d]
 *   o_lo : device bf16 [s, Hq/P, d] or NULL: O's rounding residual of this rank's heads
 *   lse : device fp32 [Hq/P, s], written for this rank's heads
 *   workspace : at least attn_fwd_chunked_workspace_bytes(...) bytes; NULL with a non-NULL
 *               workspace_bytes -> size query as for attn_bwd. This is the peak intermediate
 *               memory of the schedule. For bf16 with s_l a multiple of 128 the chunks read
 *               the shards and write the o shards directly (the shard-reading kernels of
 *               attn_fwd_shards with head sub-ranges), so the size is 0 and the call runs
 *               with workspace == NULL and workspace_bytes == NULL; otherwise each chunk's
 *               Q/O and its kv heads' K/V are packed into the workspace.
 * ------------------------------------------------------------------------- */
int attn_fwd_chunked(const void* const* q_shards, const void* const* k_shards,
                     const void* const* v_shards, void* const* o_shards, void* o_lo, float* lse,
                     int P, int rank, int64_t s_l, int Hq, int Hkv, int d, int dtype,
                     float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                     int heads_per_chunk, void* workspace, size_t* workspace_bytes,
                     void* stream);

size_t attn_fwd_chunked_workspace_bytes(int P, int64_t s_l, int Hq, int Hkv, int d,
                                        int dtype, int heads_per_chunk);

/* ---------------------------------------------------------------------------
 * attn_fwd_shards -- the forward of rank `rank` with the exchange folded into the
 * attention's own loads and stores ("Ulysses Sequence Parallelism: Training with
 * Million-Token Contexts", how Ulysses works, steps 1-5: after the first all-to-all a
 * rank holds every position of its heads, and the second all-to-all returns O to the
 * sequence shards). Instead of materialising the head shard, the kernel reads the rank's
 * Q heads and kv heads straight from the P sequence shards and writes O straight into
 * the rank's head slice of the o shards: no intermediate buffer. Results are bitwise
 * those of ulysses_pack + attn_fwd + ulysses_unpack given the same workspace size.
 *   q_shards / o_shards : host arrays of P device pointers [s_l, Hq, d] (global Hq);
 *                        only head slice `rank` of the o shards is written
 *   k_shards / v_shards : host arrays of P device pointers [s_l, Hkv, d]
 *   o_lo : device bf16 [s, Hq/P, d] or NULL: O's rounding residual of this rank's heads
 *   lse : device fp32 [Hq/P, s] for this rank's heads
 *   workspace : NULL, or workspace_bytes of device scratch (16-byte aligned) for the split
 *               run of short and mid-size grids, as for attn_fwd with s = P * s_l and Hq/P
 *               heads: attn_fwd_workspace_bytes(P * s_l, Hq / P, d) bytes split.
 * bf16 only (ULY_ERR_UNSUPPORTED for fp32), and every workgroup's rows must lie in one
 * shard: s_l a multiple of 128 (ULY_ERR_UNSUPPORTED otherwise). Other errors as for
 * attn_fwd_chunked.
 * ------------------------------------------------------------------------- */
int attn_fwd_shards(const void* const* q_shards, const void* const* k_shards,
                    const void* const* v_shards, void* const* o_shards, void* o_lo, float* lse,
                    int P, int rank, int64_t s_l, int Hq, int Hkv, int d, int dtype,
                    float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attn_bwd_shards -- the backward of rank `rank` with the exchange folded in, as
 * attn_fwd_shards is for the forward (same passage: in training the backward repeats the
 * two all-to-alls for the gradients). The kernels read Q, K, V, O and dO of the rank's
 * heads straight from the sequence shards and write dQ, dK and dV straight into the
 * rank's head slices of the gradient shards. Results are bitwise those of ulysses_pack +
 * attn_bwd + ulysses_unpack given the same workspace size.
 *   q_shards / o_shards / do_shards / dq_shards : host arrays of P device pointers
 *                        [s_l, Hq, d] (global Hq); o and lse as written by the forward
 *   k_shards / v_shards / dk_shards / dv_shards : host arrays of P device pointers
 *                        [s_l, Hkv, d]
 *   o_lo : the residual attn_fwd_shards wrote ([s, Hq/P, d]) or NULL
 *   lse : device fp32 [Hq/P, s]
 *   workspace : delta, 4 * P * s_l * (Hq / P) bytes rounded up to a multiple of 256
 *               (required), then room for the partial sums of the split dK/dV and dQ runs
 *               of short and mid-size grids, as in attn_bwd (optional: used only where
 *               *workspace_bytes states room for it; with workspace_bytes NULL the buffer
 *               is taken to hold delta alone and both run unsplit). NULL -> the full size
 *               (delta and partial region) is stored into *workspace_bytes: the size
 *               attn_bwd_workspace_bytes(P * s_l, Hq / P, Hkv / P, d) reports.
 * bf16 only and s_l a multiple of 128 (ULY_ERR_UNSUPPORTED otherwise); other errors as
 * for attn_bwd_chunked.
 * ------------------------------------------------------------------------- */
int attn_bwd_shards(const void* const* q_shards, const void* const* k_shards,
                    const void* const* v_shards, const void* const* o_shards, const void* o_lo,
                    const float* lse,
                    const void* const* do_shards, void* const* dq_shards, void* const* dk_shards,
                    void* const* dv_shards, int P, int rank, int64_t s_l, int Hq, int Hkv, int d,
                    int dtype, float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                    void* workspace, size_t* workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * attn_bwd_chunked -- the backward of the UPipe schedule for rank `rank` (same passage
 * as attn_fwd_chunked: only some heads are resident at a time, which matters most in
 * training). For each chunk of `heads_per_chunk` local q heads: pack the chunk's Q, O and
 * dO (and its kv heads' K and V when their range changes), form delta, dK/dV and dQ of the
 * chunk, and unpack dQ into the dq shards. The dK/dV of a kv head read by several chunks
 * are summed in fp32 across those chunks and rounded once; the rank's dK and dV are
 * unpacked into the dk / dv shards after the last chunk. dQ is identical to the
 * unchunked attn_bwd's; dK/dV differ from it only in the order of the fp32 sums.
 *   q_shards / o_shards / do_shards / dq_shards : host arrays of P device pointers
 *                        [s_l, Hq, d] (global Hq); o and lse as written by the forward
 *   k_shards / v_shards / dk_shards / dv_shards : host arrays of P device pointers
 *                        [s_l, Hkv, d]
 *   o_lo : the residual attn_fwd_chunked wrote ([s, Hq/P, d]) or NULL
 *   lse : device fp32 [Hq/P, s] of this rank's heads
 *   dq / dk / dv shards: only this rank's head slices are written.
 *   workspace : at least attn_bwd_chunked_workspace_bytes(...) bytes; NULL -> size query
 *               into *workspace_bytes as for attn_bwd. For bf16 with s_l a multiple of 128
 *               the chunks read and write the shards directly and the workspace is delta of
 *               a chunk and the fp32 dK/dV sums of the rank's kv heads; otherwise it also
 *               holds the chunk buffers (Q, O, dO, dQ of u heads, K and V of the kv heads
 *               they read) and the rank's dK/dV.
 * Errors as for attn_fwd_chunked.
 * ------------------------------------------------------------------------- */
int attn_bwd_chunked(const void* const* q_shards, const void* const* k_shards,
                     const void* const* v_shards, const void* const* o_shards, const void* o_lo,
                     const float* lse,
                     const void* const* do_shards, void* const* dq_shards, void* const* dk_shards,
                     void* const* dv_shards, int P, int rank, int64_t s_l, int Hq, int Hkv, int d,
                     int dtype, float scale, int causal, const int32_t* cu_seqlens, int n_docs,
                     int heads_per_chunk, void* workspace, size_t* workspace_bytes, void* stream);

size_t attn_bwd_chunked_workspace_bytes(int P, int64_t s_l, int Hq, int Hkv, int d,
                                        int dtype, int heads_per_chunk);

/* ---------------------------------------------------------------------------
 * ring_attn_fwd / ring_attn_bwd -- Ring Attention, the pages' comparison workload
 * ("Ulysses Sequence Parallelism: Training with Million-Token Contexts", sections on
 * communication complexity and on Ulysses compared with Ring Attention): every rank keeps its
 * token block of Q, K and V with all heads, and the K/V blocks travel round a ring of P ranks;
 * at hop i rank r attends to the block of rank (r - i) mod P and the partial outputs are merged
 * by their log-sum-exps, which gives attention over the whole sequence. On one GPU the ring's
 * point-to-point sends are reads of the other ranks' buffers. causal: the rank's own block is
 * causal inside, earlier blocks fully visible, later blocks skipped. bf16 only.
 *   q_shards, k_shards, v_shards : host arrays of P device pointers [s_l, Hq | Hkv, d]
 *   Hq, Hkv : all the heads (no head sharding), Hq % Hkv == 0
 * ring_attn_fwd: o [s_l, Hq, d] (rank's block of O), o_lo (NULL or its residual, as for
 *   attn_fwd), lse [Hq, s_l]. Each hop runs the attention forward on the pair of blocks, writing
 *   the partial O with its residual, and a merge folds it into an fp32 running output in
 *   ring order. workspace: ring_attn_fwd_workspace_bytes(s_l, Hq, d) (partial O, residual,
 *   LSE, fp32 running output and LSE); NULL -> size query into *workspace_bytes.
 * ring_attn_bwd: rank r's backward given its merged o (+ o_lo), lse and dout: writes dq
 *   [s_l, Hq, d] (summed over its hops in fp32, rounded once), and adds its contribution to
 *   the fp32 dK/dV sums of every block it attended to. dk_acc, dv_acc: device fp32
 *   [P, s_l, Hkv, d], the sums that travel with the K/V blocks in a real ring; the rank that
 *   attends first to a block (causal: its owner; else rank 0) starts them, and rank P - 1
 *   rounds them into that block's dk_shards / dv_shards [s_l, Hkv, d]. So the P ranks' calls
 *   must run in rank order on one stream. workspace: ring_attn_bwd_workspace_bytes(s_l, Hq, d)
 *   (delta and the fp32 dQ sums).
 * Deterministic (fixed hop and rank order, no atomics).
 * ------------------------------------------------------------------------- */
size_t ring_attn_fwd_workspace_bytes(int64_t s_l, int Hq, int d);
size_t ring_attn_bwd_workspace_bytes(int64_t s_l, int Hq, int d);
int ring_attn_fwd(const void* const* q_shards, const void* const* k_shards,
                  const void* const* v_shards, void* o, void* o_lo, float* lse, int P, int rank,
                  int64_t s_l, int Hq, int Hkv, int d, int dtype, float scale, int causal,
                  void* workspace, size_t* workspace_bytes, void* stream);
int ring_attn_bwd(const void* const* q_shards, const void* const* k_shards,
                  const void* const* v_shards, const void* o, const void* o_lo, const float* lse,
                  const void* dout, void* dq, float* dk_acc, float* dv_acc, void* const* dk_shards,
                  void* const* dv_shards, int P, int rank, int64_t s_l, int Hq, int Hkv, int d,
                  int dtype, float scale, int causal, void* workspace, size_t* workspace_bytes,
                  void* stream);

/* ---------------------------------------------------------------------------
 * uly_mfma_probe -- measurement helper, not part of the attention path: `blocks`
 * workgroups of 4 waves each issue `iters` x 4 back-to-back v_mfma_f32_32x32x16_bf16
 * (32768 flops each) on independent accumulators, giving the practical bf16 matrix-core
 * ceiling that the bench reports beside the published peak. Wave 0 of workgroup 0 writes
 * the shader clock cycles and the 100 MHz reference-counter ticks of its loop to
 * clocks[0], clocks[1] (device memory, 2 x uint64), hence the sustained clock. `sink`: one
 * device float, written only in a case that does not occur (it keeps the work alive).
 * Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (iters or blocks < 1), ULY_ERR_HIP.
 * ------------------------------------------------------------------------- */
int uly_mfma_probe(int iters, int blocks, float* sink, uint64_t* clocks, void* stream);

/* ---------------------------------------------------------------------------
 * uly_mix_probe -- measurement helper, not part of the attention path: the ceiling of the
 * attention kernels' inner-loop instruction mix. `blocks` workgroups of 4 waves each run
 * `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 (32768 flops each), every product's first
 * operand a 1 KiB LDS read (ds_read_b128), followed by, for `kind` 0: nothing; 1: 2 fp32
 * FMAs and 1 v_exp_f32; 2: 4 fp32 FMAs and 1 v_exp_f32, on registers of their own. The
 * kernel fits 4 workgroups per CU, so 256 * W blocks run W waves on every SIMD. `sink`: one
 * device float, written only in a case that does not occur.
 * Errors: ULY_ERR_NULL, ULY_ERR_SHAPE (iters or blocks < 1), ULY_ERR_UNSUPPORTED (kind not
 * 0..2), ULY_ERR_HIP.
 * ------------------------------------------------------------------------- */
int uly_mix_probe(int kind, int iters, int blocks, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ULYSSES_H */
