// Causal / packed-document GQA attention forward for one head shard, bf16 in, fp32
// accumulation, on gfx950 matrix cores.
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts", section
// "how Ulysses works", step 4 (each GPU runs local attention for its heads over every
// position) and the long-sequence section (FlashAttention keeps memory O(n) while the
// compute stays O(n^2)): the kernel streams K/V tiles past resident Q rows with an
// online softmax, so the s x s score matrix never exists.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one q head, three
// workgroups per CU; grids too small to fill three per CU take 64-key tiles at two per CU):
//   * each wave owns 32 query rows; its Q rows stay in VGPRs for the whole key loop as
//     MFMA B operands;
//   * K/V tiles of 32 (or 64) keys arrive in LDS by DMA (global_load_lds, XOR-swizzled
//     rows, double buffered; the next tile is requested after the current tile's last LDS
//     read) and are shared by the 4 waves; each 32 keys of a tile are S (8 MFMAs), their
//     softmax, then PV (8 MFMAs);
//   * three waves per SIMD (at most 168 VGPRs, 32 KiB of LDS per workgroup): a wave's VALU
//     work does not overlap its own MFMAs, so the softmax of one wave runs beside the
//     products of the others, and a third wave leaves that overlap less often empty than two;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 leaves each lane one query row and 16 of
//     the 32 keys, so the row max and row sum are lane-local plus one swap with the lane 32
//     away;
//   * O^T += V^T P^T: P (bf16) is already in B-operand layout, V^T comes straight from
//     the row-major V tile through the transposing LDS read (ds_read_b64_tr_b16), and the
//     O^T accumulator keeps each lane's query row, so softmax rescales stay lane-local;
//   * the exponent is exp2 with scale*log2(e) folded into one FMA, and the running max is
//     only moved when a row's max grows by more than kTau (2^8): P then stays <= 256 and
//     most tiles skip the O rescale;
//   * two row sums: l of the fp32 weights gives the LSE, and l' of the bf16-rounded weights
//     (the PV operand, summed by v_dot2_f32_bf16) normalises O, so O is an exact convex
//     combination of the V rows with the weights the MFMA used: on rows dominated by one key
//     the weight's rounding (up to 2^-9 of it, since the lagging max leaves it unequal to 1)
//     then cancels instead of reaching O, and delta = dO . O in the backward;
//   * causal / document tiles outside a row block's range are never visited; partial
//     tiles are masked per element; workgroups with the longest key range launch first.
#include <type_traits>

#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr float kTau = 8.0f;
// LDS operand read-ahead of the S^T and O^T products (k-steps / products ahead)
constexpr int kPfS = 2, kPfV = 2;

// Key tiles of BN = 32 (three workgroups per CU) or 64 keys (two): a tile is processed as
// BN / 32 halves of 32 keys, each S, its softmax and PV in turn, so both tile sizes perform the
// same operations in the same order and give bitwise-identical results. SPLIT instances can
// run a row block as nsplit_o workgroups over contiguous ranges of its key tiles, each storing
// partial results for the combine kernel below.
template <int D, int BN, bool SPLIT>
__global__ __launch_bounds__(256, BN == 32 ? 3 : 2) void attn_fwd_kernel(AttnArgs a, ShardSrc src) {
  constexpr int BM = 128, DT = D / 16, DB = D / 32;
  static_assert(BN == 32 || BN == 64, "key tile");
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hf = lane >> 5, gi = lane >> 4, li = lane & 15;
  const int64_t s = a.s;
  const int nmb = (int)((s + BM - 1) / BM);
  const int h = blockIdx.x % a.n_heads;
  // workgroups per row block (short and mid-size grids; the instance for large grids carries
  // no split code)
  const int nso = SPLIT && a.nsplit_o > 1 ? a.nsplit_o : 1;
  const int sp = (int)((blockIdx.x / a.n_heads) % nso);
  const int mb = nmb - 1 - (int)(blockIdx.x / a.n_heads / nso);
  const int64_t m0 = (int64_t)mb * BM;
  const int kvh = (h + a.q_off) / a.G - a.kv_off;
  // shard of the workgroup's rows (all in one) and the row offset of that shard
  const int ps = (int)((uint32_t)m0 / (uint32_t)src.s_l);
  const int64_t r_sh = (int64_t)ps * src.s_l;
  const uint16_t* Q = static_cast<const uint16_t*>(src.q[ps]) + (int64_t)h * D;
  const float c = a.scale * kLog2e;

  const int64_t row = m0 + wave * 32 + l32;
  // this row's key range [lo, hi) (positions fit in 32 bits: s < 2^31 is checked on the host)
  int32_t lo = 0, hi = (int32_t)s;
  if (a.cu != nullptr && row < s) {
    const int dk = doc_of(a.cu, a.n_docs, row);
    lo = a.cu[dk];
    hi = a.cu[dk + 1] < (int32_t)s ? a.cu[dk + 1] : (int32_t)s;
  }
  if (a.causal) hi = hi < (int32_t)row + 1 ? hi : (int32_t)row + 1;
  bf16x8 qf[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    u32x4 v = {0, 0, 0, 0};
    if (row < s) v = *reinterpret_cast<const u32x4*>(Q + (row - r_sh) * a.q_row + 16 * t + 8 * hf);
    qf[t] = __builtin_bit_cast(bf16x8, v);
  }

  const int64_t wr0 = m0 + wave * 32;
  const int64_t wr1 = (wr0 + 32 < s ? wr0 + 32 : s) - 1;
  const int64_t last_row = (m0 + BM < s ? m0 + BM : s) - 1;
  int64_t kbeg = 0, kend = s, w_lo_last = 0, w_hi_first = s;
  if (a.cu != nullptr) {
    // document bounds clamped to [0, s]: no tile outside the sequence is ever visited
    kbeg = a.cu[doc_of(a.cu, a.n_docs, m0)];
    kbeg = kbeg > 0 ? kbeg : 0;
    kend = a.cu[doc_of(a.cu, a.n_docs, last_row) + 1];
    kend = kend < s ? kend : s;
    if (wr0 < s) {
      w_hi_first = a.cu[doc_of(a.cu, a.n_docs, wr0) + 1];
      w_lo_last = a.cu[doc_of(a.cu, a.n_docs, wr1)];
    }
  }
  if (a.causal) kend = kend < last_row + 1 ? kend : last_row + 1;
  kbeg = (kbeg / BN) * BN;
  // Halves of 32 keys from k0 that every row of this wave sees whole: full_lo <= k0 <= full_hi
  // (keys inside the sequence, at or after the last row's document start, before the first
  // row's document end, and, causal, at or before the first row).
  const int64_t full_lo = w_lo_last;
  int64_t full_hi = (s < w_hi_first ? s : w_hi_first) - 32;
  if (a.causal) full_hi = full_hi < wr0 - 31 ? full_hi : wr0 - 31;
  const bool any_full = wr0 < s && full_hi >= full_lo;
  const uint32_t full_w = any_full ? (uint32_t)(full_hi - full_lo) : 0u;
  int ntiles = kbeg < kend ? (int)((kend - kbeg + BN - 1) / BN) : 0;
  if (nso > 1) {  // this split's share of the block's key tiles
    const int t0 = (int)((int64_t)ntiles * sp / nso), t1 = (int)((int64_t)ntiles * (sp + 1) / nso);
    kbeg += (int64_t)t0 * BN;
    ntiles = t1 - t0;
  }

  // tile k0 of K and V from its shard (rows past the sequence end read the shard's last row);
  // K and V share the row stride, so one set of lane offsets serves both
  const uint32_t kv_off = dma_lane_offset<D, 256>(a.kv_row, tid);
  auto issue_kv = [&](int64_t k0, int b) {
    const int pk = (int)((uint32_t)k0 / (uint32_t)src.s_l);
    const int64_t r0 = k0 - (int64_t)pk * src.s_l;
    const uint16_t* K = static_cast<const uint16_t*>(src.k[pk]) + (int64_t)kvh * D;
    const uint16_t* V = static_cast<const uint16_t*>(src.v[pk]) + (int64_t)kvh * D;
    if (r0 + BN <= src.s_l) {
      dma_tile_whole<D, BN, 256>(K + r0 * a.kv_row, a.kv_row, kv_off, sK[b], wave);
      dma_tile_whole<D, BN, 256>(V + r0 * a.kv_row, a.kv_row, kv_off, sV[b], wave);
    } else {
      // a shard's ragged last tile: the thread index through an empty asm, so this rare path's
      // address arithmetic is formed here rather than hoisted into registers for the whole loop
      int t1 = tid;
      asm volatile("" : "+v"(t1));
      dma_tile<D, BN, 256>(K, a.kv_row, r0, src.s_l, sK[b], t1);
      dma_tile<D, BN, 256>(V, a.kv_row, r0, src.s_l, sV[b], t1);
    }
  };
  // S^T of half hh of the tile in buffer b: the K operand of k-step t is read kPfS steps ahead
  // (a ring of kPfS + 1 registers), each product behind a scheduling barrier; left alone, the
  // compiler reads each operand just before its MFMA and waits for it
  auto qk = [&](int b, int hh, f32x16& S) {
    bf16x8 ring[kPfS + 1];
    auto ld = [&](int t) {
      return *reinterpret_cast<const bf16x8*>(&sK[b][tile_off<D>(hh * 32 + l32, 16 * t + 8 * hf)]);
    };
#pragma unroll
    for (int t = 0; t < kPfS; ++t) ring[t] = ld(t);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      if (t + kPfS < DT) ring[(t + kPfS) % (kPfS + 1)] = ld(t + kPfS);
      S = mfma32x32x16(ring[t % (kPfS + 1)], qf[t], t == 0 ? f32x16{} : S);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the 32 keys from k0 need no mask for any row of this wave (one unsigned range compare)
  auto half_full = [&](int64_t k0) { return any_full && (uint32_t)(k0 - full_lo) <= full_w; };
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f, lr = 0.f;  // running max (log2 units), sums of fp32 / rounded weights
  float nms = 0.f;  // the exponent offset -m, 0 while m is -inf (kept beside m, set when m moves)
  // mask S of the 32 keys from k0, then rescale O if the row max grew by more than kTau
  auto mask_rescale = [&](int64_t k0, f32x16& S) {
    if (!half_full(k0)) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int32_t key = (int32_t)k0 + 8 * (jj / 4) + 4 * hf + (jj % 4);
        if (key < lo || key >= hi) S[jj] = -INFINITY;
      }
    }
    // the NaN-propagating maximum (v_maximum3_f32, three values per instruction): unlike fmaxf
    // it needs no quieting of the MFMA results first
    float mx = S[0];
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) mx = __builtin_elementwise_maximum(mx, S[jj]);
    const float tmax = half_swap_max(mx) * c;
    const bool need = tmax > m + kTau;
    if (__ballot(need) != 0) {  // wave-uniform
      const float mnew = need ? tmax : m;
      const float alpha = need ? fast_exp2(m - mnew) : 1.f;
      m = mnew;
      nms = need ? -tmax : nms;  // a row whose max moved has a finite one
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = mfma32x32x16(bf16x8{}, bf16x8{}, oacc[db] * alpha);
    }
  };
  auto softmax = [&](f32x16& S, bf16x8 (&pf)[2]) {
    S[0] = fast_exp2(__builtin_fmaf(S[0], c, nms));
    float ls = S[0];  // the weights are >= +0: starting the sum at the first one is exact
#pragma unroll
    for (int jj = 1; jj < 16; ++jj) {
      const float pj = fast_exp2(__builtin_fmaf(S[jj], c, nms));
      S[jj] = pj;
      ls += pj;
    }
    pf[0] = to_bf16x8(S, 0);
    pf[1] = to_bf16x8(S, 1);
    l += ls;
    // the rounded weights, two per v_dot2_f32_bf16 against (1, 1)
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4 w = __builtin_bit_cast(u32x4, pf[t]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t we = w[e];
        lr = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, we), one2, lr, false);
      }
    }
  };
  // O^T += V^T P^T for half hh of the tile in buffer b: product i = (tt, db); its V^T operand
  // (two transposing reads) is read kPfV products ahead, as the K operands are
  auto pv = [&](int b, int hh, const bf16x8 (&pf)[2]) {
    constexpr int NPV = 2 * DB;
    auto ld = [&](int i) {
      const int tt = i / DB, db = i % DB;
      const int kr = hh * 32 + 16 * tt + 4 * hf + (li >> 2);
      const int col = db * 32 + 16 * (gi & 1) + 4 * (li & 3);
      const i16x4 v0 = lds_read_tr16(&sV[b][tile_off<D>(kr, col)]);
      const i16x4 v1 = lds_read_tr16(&sV[b][tile_off<D>(kr + 8, col)]);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 ring[kPfV + 1];
#pragma unroll
    for (int i = 0; i < kPfV; ++i) ring[i] = ld(i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + kPfV < NPV) ring[(i + kPfV) % (kPfV + 1)] = ld(i + kPfV);
      oacc[i % DB] = mfma32x32x16(ring[i % (kPfV + 1)], pf[i / DB], oacc[i % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one tile; B is the buffer (compile time: the two buffers' LDS addresses then differ by an
  // immediate offset, so no per-read address arithmetic)
  auto tile_step = [&](auto B, int t) {
    constexpr int b = decltype(B)::value;
    const int64_t k0 = kbeg + (int64_t)t * BN;
    wait_dma();
    __syncthreads();  // tile t has landed; every wave is done with tile t-1
#pragma unroll
    for (int hh = 0; hh < BN / 32; ++hh) {
      f32x16 S;
      bf16x8 p[2];
      qk(b, hh, S);
      mask_rescale(k0 + 32 * hh, S);
      // raised priority through the softmax: the other waves' products fill the matrix core
      __builtin_amdgcn_s_setprio(1);
      softmax(S, p);
      __builtin_amdgcn_s_setprio(0);
      pv(b, hh, p);
    }
    // the next tile's DMA after this tile's last LDS read: the wait the compiler places
    // before LDS reads that follow a DMA then falls on the next barrier
    if (t + 1 < ntiles) issue_kv(k0 + BN, 1 - b);
  };

  if (ntiles > 0) issue_kv(kbeg, 0);
  for (int t = 0;;) {
    if (t >= ntiles) break;
    tile_step(std::integral_constant<int, 0>{}, t);
    if (++t >= ntiles) break;
    tile_step(std::integral_constant<int, 1>{}, t);
    ++t;
  }

  const float lt = half_swap_sum(l), lrt = half_swap_sum(lr);
  if (nso > 1) {
    // this split's unnormalised fp32 sums and its row statistics; the combine kernel merges them
    if (row < s) {
      const int64_t slot = ((int64_t)h * nmb + mb) * nso + sp;
      const int64_t r = wave * 32 + l32;
      float* op = a.o_part + slot * (BM * D) + r * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(op + db * 32 + 8 * jj + 4 * hf) =
              f32x4{oacc[db][4 * jj + 0], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
      if (hf == 0) *reinterpret_cast<f32x4*>(a.o_stat + (slot * BM + r) * 4) = f32x4{m, lt, lrt, 0.f};
    }
    return;
  }
  if (row < s) {
    uint16_t* O = static_cast<uint16_t*>(src.o[ps]) + (int64_t)h * D - r_sh * a.q_row;
    // O's bf16 rounding residual, when asked for: O_fp32 - bf16(O_fp32), rounded to bf16
    uint16_t* OL = a.o_lo != nullptr ? static_cast<uint16_t*>(a.o_lo) + (int64_t)h * D + row * a.lo_row : nullptr;
    const float inv = 1.f / lrt;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float x0 = oacc[db][4 * jj + 0] * inv, x1 = oacc[db][4 * jj + 1] * inv;
        const float x2 = oacc[db][4 * jj + 2] * inv, x3 = oacc[db][4 * jj + 3] * inv;
        u32x2 w;
        w[0] = pack_bf16x2(x0, x1);
        w[1] = pack_bf16x2(x2, x3);
        *reinterpret_cast<u32x2*>(O + row * a.q_row + db * 32 + 8 * jj + 4 * hf) = w;
        if (OL != nullptr) {
          const uint32_t w0 = w[0], w1 = w[1];
          u32x2 r;
          r[0] = pack_bf16x2(x0 - bf16_lo(w0), x1 - bf16_hi(w0));
          r[1] = pack_bf16x2(x2 - bf16_lo(w1), x3 - bf16_hi(w1));
          *reinterpret_cast<u32x2*>(OL + db * 32 + 8 * jj + 4 * hf) = r;
        }
      }
    if (hf == 0) a.lse_out[(int64_t)h * a.lse_row + row] = (m + log2f(lt)) * kLn2;
  }
}

// Rows of split row blocks: for 8 consecutive elements of one row and q head, the nsplit_o
// partial results merged in split order. With M the largest running max over the splits and
// w = 2^(m_sp - M): O = sum w O_sp / sum w l'_sp (the rounded-weight sums, as the unsplit
// kernel normalises) and LSE = (M + log2 sum w l_sp) ln 2. Writes O, its residual if asked
// for, and (one thread per row) the LSE. One thread each.
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(AttnArgs a, ShardSrc src) {
  constexpr int BM = 128, PER = D / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t s = a.s, nmb = (s + BM - 1) / BM;
  if (c >= (int64_t)a.n_heads * s * PER) return;
  const int part8 = (int)(c % PER);
  const int64_t row = (c / PER) % s;
  const int h = (int)(c / PER / s);
  const int ns = a.nsplit_o;
  const int64_t mb = row / BM, r = row - mb * BM;
  const int64_t slot0 = ((int64_t)h * nmb + mb) * ns;
  float M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, a.o_stat[((slot0 + sp) * BM + r) * 4]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lt = 0.f, lrt = 0.f;
  for (int sp = 0; sp < ns; ++sp) {
    const f32x4 st = *reinterpret_cast<const f32x4*>(a.o_stat + ((slot0 + sp) * BM + r) * 4);
    const float w = st[0] == -INFINITY ? 0.f : fast_exp2(st[0] - M);  // a split that saw no key: 0
    lt = __builtin_fmaf(w, st[1], lt);
    lrt = __builtin_fmaf(w, st[2], lrt);
    const float* op = a.o_part + (slot0 + sp) * (BM * D) + r * D + part8 * 8;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(op);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = __builtin_fmaf(w, x0[e], acc[e]);
      acc[4 + e] = __builtin_fmaf(w, x1[e], acc[4 + e]);
    }
  }
  const float inv = 1.f / lrt;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  const int p = (int)((uint32_t)row / (uint32_t)src.s_l);
  uint16_t* O = static_cast<uint16_t*>(src.o[p]) + (row - (int64_t)p * src.s_l) * a.q_row + (int64_t)h * D + part8 * 8;
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[2 * e], acc[2 * e + 1]);
  *reinterpret_cast<u32x4*>(O) = w;
  if (a.o_lo != nullptr) {
    // O's bf16 rounding residual O_fp32 - bf16(O_fp32), rounded to bf16
    u32x4 rl;
#pragma unroll
    for (int e = 0; e < 4; ++e) rl[e] = pack_bf16x2(acc[2 * e] - bf16_lo(w[e]), acc[2 * e + 1] - bf16_hi(w[e]));
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o_lo) + (int64_t)h * D + row * a.lo_row + part8 * 8) = rl;
  }
  if (part8 == 0) a.lse_out[(int64_t)h * a.lse_row + row] = (M + log2f(lt)) * kLn2;
}

// Grids of at least three workgroups per CU (256 CUs) take 32-key tiles and three workgroups
// per CU; smaller grids, which would leave that third slot empty, take 64-key tiles (fewer
// barriers and tile requests per key) at two per CU, also when their row blocks split.
constexpr int64_t kFwdSmallGrid = 3 * 256;

template <int D>
hipError_t launch_fwd_t(const AttnArgs& a, const ShardSrc& src, hipStream_t stream) {
  const int64_t nmb = (a.s + 127) / 128;
  const int64_t blocks = nmb * a.n_heads;
  if (blocks == 0) return hipSuccess;
  const int nso = a.nsplit_o > 1 ? a.nsplit_o : 1;
  const dim3 grid((unsigned)(blocks * nso));
  if (blocks >= kFwdSmallGrid && nso == 1)
    hipLaunchKernelGGL((attn_fwd_kernel<D, 32, false>), grid, dim3(256), 0, stream, a, src);
  else if (blocks >= kFwdSmallGrid)
    hipLaunchKernelGGL((attn_fwd_kernel<D, 32, true>), grid, dim3(256), 0, stream, a, src);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, 64, true>), grid, dim3(256), 0, stream, a, src);
  if (nso > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = a.n_heads * a.s * (D / 8);
    hipLaunchKernelGGL((fwd_combine_kernel<D>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a, src);
  }
  return hipGetLastError();
}

}  // namespace

int fwd_split_count(int64_t s, int n_heads) {
  // Row blocks launch longest first, and the last one sees every key (about twice the mean),
  // so a grid of one or two rounds is set by its longest blocks. Below three per CU it is one
  // round of 64-key tiles at two per CU (512 slots): split every block's key tiles aiming at
  // 1024 workgroups, at most 8 per block; from there to one and a half rounds of 32-key tiles
  // at three per CU (1152 workgroups), split in two (measured: 768 and 1024 workgroups gain,
  // 1280 loses).
  const int64_t wg = (s + 127) / 128 * n_heads;
  if (wg < 1 || wg >= 3 * kFwdSmallGrid / 2) return 1;
  const int64_t ns = wg < kFwdSmallGrid ? (1024 + wg - 1) / wg : 2;
  return (int)(ns < 8 ? ns : 8);
}

hipError_t launch_attn_fwd_bf16_shards(const AttnArgs& a, const ShardSrc& src, int d, hipStream_t stream) {
  if (d == 128) return launch_fwd_t<128>(a, src, stream);
  return launch_fwd_t<64>(a, src, stream);
}

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t stream) {
  ShardSrc src{};
  src.q[0] = a.q;
  src.k[0] = a.k;
  src.v[0] = a.v;
  src.o[0] = a.out;
  src.s_l = a.s;
  return launch_attn_fwd_bf16_shards(a, src, d, stream);
}

}  // namespace uly
