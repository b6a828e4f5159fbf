// Attention backward for one head shard on gfx950: the preprocess (delta = rowsum(dO*O)),
// a dK/dV kernel and a separate dQ kernel, bf16 in, fp32 accumulation.
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts" -- the
// method trains models (title and opening section), so each rank also runs the backward
// of its local attention (step 4 of "how Ulysses works"); FlashAttention's O(n) memory
// (long-sequence section) means P is recomputed from Q, K and the saved LSE rather than
// stored.
//
// Per row i of q head h (kv head g), with P_ij = exp(scale q_i.k_j - LSE_i):
//   dV_j += sum_i P_ij dO_i                 dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - delta_i)          delta_i = dO_i . O_i
//   dQ_i  = scale sum_j dS_ij k_j           dK_j += scale sum_i dS_ij q_i
// dK/dV of a kv head sum over its G q heads inside one workgroup, in fp32, so no atomics
// are needed and the result is deterministic. dQ is a separate pass over key tiles.
//
// Both kernels use v_mfma_f32_32x32x16_bf16. Operands whose contraction index is the
// row-major tile's row (K for dQ, Q and dO for dK/dV) come from the transposing LDS read
// ds_read_b64_tr_b16, so no tile is ever transposed in memory. Both stage their streamed
// tiles by LDS DMA and run two waves per SIMD, so one wave's VALU work (exp, dS) overlaps
// the other's MFMAs.
#include <type_traits>

#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kWaves = 4;
// dQ kernel: LDS operand read-ahead of the S/dP products (k-steps) and the dQ products (products):
// left alone, the compiler reads each operand just before its MFMA (2% of the kernel at 64K)
constexpr int kDqPfA = 2, kDqPfB = 3;

// ---------------------------------------------------------------------------------------
// delta[h, i] = sum_x dO[i, h, x] * O[i, h, x] (fp32). TPR threads per (row, head), 16 B each.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(AttnArgs a, Shards o_sh, Shards g_sh, int64_t s_l) {
  constexpr int TPR = D * (int)sizeof(T) / 16;
  constexpr int EPV = 16 / (int)sizeof(T);
  const int64_t idx = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const int64_t row = idx / a.n_heads;
  const int h = (int)(idx % a.n_heads);
  float acc = 0.f;
  if (row < a.s) {
    const int ps = (int)((uint32_t)row / (uint32_t)s_l);
    const int64_t off = (row - (int64_t)ps * s_l) * a.q_row + (int64_t)h * D + part * EPV;
    const u32x4 ov = *reinterpret_cast<const u32x4*>(static_cast<const T*>(o_sh.p[ps]) + off);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(static_cast<const T*>(g_sh.p[ps]) + off);
    if constexpr (sizeof(T) == 2) {
      // O = bf16 O + its rounding residual when the forward wrote one (delta then carries no
      // bf16 rounding of O, which matters on rows dominated by one key)
      u32x4 lv = {0, 0, 0, 0};
      if (a.o_lo != nullptr)
        lv = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.o_lo) + row * a.lo_row + (int64_t)h * D +
                                              part * EPV);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc += (bf16_lo(ov[i]) + bf16_lo(lv[i])) * bf16_lo(gv[i]);
        acc += (bf16_hi(ov[i]) + bf16_hi(lv[i])) * bf16_hi(gv[i]);
      }
    } else {
      // bit-cast whole vectors: clang mis-handles __builtin_bit_cast of a vector element
      const f32x4 of = __builtin_bit_cast(f32x4, ov), gf = __builtin_bit_cast(f32x4, gv);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc += of[i] * gf[i];
    }
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (part == 0 && row < a.s) a.lse_out[(int64_t)h * a.lse_row + row] = acc;
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup = BM query rows of one q head; loops over key tiles of BN keys.
template <int D, int RB, int KB>
struct DqCfg {
  static constexpr int BM = kWaves * RB * 32;
  static constexpr int BN = KB * 32;
  static constexpr int DT = D / 16, DB = D / 32;
};

template <int D, int RB, int KB>
__global__ __launch_bounds__(kWaves * 64, 2) void attn_dq_kernel(AttnArgs a, Shards q_sh, Shards g_sh, Shards k_sh,
                                                                  Shards v_sh, Shards dq_sh, int64_t s_l) {
  using C = DqCfg<D, RB, KB>;
  constexpr int BM = C::BM, BN = C::BN, DT = C::DT, DB = C::DB;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int l32 = lane & 31, hf = lane >> 5, gi = lane >> 4, li = lane & 15;
  const int64_t s = a.s;
  const int nmb = (int)((s + BM - 1) / BM);
  const int h = blockIdx.x % a.n_heads;
  const int nsq = a.nsplit_q > 1 ? a.nsplit_q : 1;  // workgroups per row block (small grids)
  const int sp = (int)((blockIdx.x / a.n_heads) % nsq);
  const int mb = nmb - 1 - (int)(blockIdx.x / a.n_heads / nsq);
  const int64_t m0 = (int64_t)mb * BM;
  const int kvh = (h + a.q_off) / a.G - a.kv_off;
  // shard of the workgroup's rows (all in one); Q, dO and dQ addressed from its first row
  const int ps = (int)((uint32_t)m0 / (uint32_t)s_l);
  const int64_t r_sh = (int64_t)ps * s_l;
  const uint16_t* Q = static_cast<const uint16_t*>(q_sh.p[ps]) + (int64_t)h * D - r_sh * a.q_row;
  const uint16_t* dO = static_cast<const uint16_t*>(g_sh.p[ps]) + (int64_t)h * D - r_sh * a.q_row;
  const float c = a.scale * kLog2e;

  int64_t row[RB], lo[RB], hi[RB];
  float lse2[RB], dl[RB];
  bf16x8 qf[RB][DT], gf[RB][DT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    row[rb] = m0 + wave * RB * 32 + rb * 32 + l32;
    lo[rb] = 0;
    hi[rb] = s;
    lse2[rb] = 0.f;
    dl[rb] = 0.f;
    if (row[rb] < s) {
      if (a.cu != nullptr) {
        const int dk = doc_of(a.cu, a.n_docs, row[rb]);
        lo[rb] = a.cu[dk];
        hi[rb] = a.cu[dk + 1] < s ? a.cu[dk + 1] : s;
      }
      lse2[rb] = a.lse_in[(int64_t)h * a.lse_row + row[rb]] * kLog2e;
      dl[rb] = a.delta[(int64_t)h * a.lse_row + row[rb]];
    }
    if (a.causal) hi[rb] = hi[rb] < row[rb] + 1 ? hi[rb] : row[rb] + 1;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 v = {0, 0, 0, 0}, w = {0, 0, 0, 0};
      if (row[rb] < s) {
        v = *reinterpret_cast<const u32x4*>(Q + row[rb] * a.q_row + 16 * t + 8 * hf);
        w = *reinterpret_cast<const u32x4*>(dO + row[rb] * a.q_row + 16 * t + 8 * hf);
      }
      qf[rb][t] = __builtin_bit_cast(bf16x8, v);
      gf[rb][t] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // key range of the workgroup: keys any of its rows may see
  const int64_t last_row = (m0 + BM < s ? m0 + BM : s) - 1;
  int64_t kbeg = 0, kend = s;
  if (a.cu != nullptr) {
    // document bounds clamped to [0, s]: no tile outside the sequence is ever visited
    kbeg = a.cu[doc_of(a.cu, a.n_docs, m0)];
    kbeg = kbeg > 0 ? kbeg : 0;
    kend = a.cu[doc_of(a.cu, a.n_docs, last_row) + 1];
    kend = kend < s ? kend : s;
  }
  if (a.causal) kend = kend < last_row + 1 ? kend : last_row + 1;
  kbeg = (kbeg / BN) * BN;
  if (nsq > 1) {  // this split's share of the block's key tiles
    const int64_t nt = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;
    const int64_t t0 = nt * sp / nsq, t1 = nt * (sp + 1) / nsq;
    const int64_t e = kbeg + t1 * BN;
    kend = e < kend ? e : kend;
    kbeg += t0 * BN;
  }
  // key k is seen by row rb of this lane iff (uint32)(k - lo[rb]) < width[rb]
  uint32_t width[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) width[rb] = (uint32_t)(hi[rb] - lo[rb]);

  // K/V tiles travel to LDS by DMA (double buffered, XOR-swizzled rows). Two workgroups share
  // a CU (at most 256 VGPRs each), so one wave's VALU work (dS) runs while the other wave on
  // the SIMD issues MFMAs; within a wave the two 32-key halves of a tile run one after the
  // other: S/dP, dS, dQ.
  static_assert(RB == 1 && KB == 2, "the tile is two 32-key halves of one 32-row wave tile");
  // key tile k0 from its shard (rows past the sequence end read the shard's last row); K and V
  // share the row stride, so one lane offset serves both
  const uint32_t kv_off = dma_lane_offset<D, kWaves * 64>(a.kv_row, tid);
  auto issue_kv = [&](int64_t k0, int b) {
    const int pk = (int)((uint32_t)k0 / (uint32_t)s_l);
    const int64_t r0 = k0 - (int64_t)pk * s_l;
    const uint16_t* K = static_cast<const uint16_t*>(k_sh.p[pk]) + (int64_t)kvh * D;
    const uint16_t* V = static_cast<const uint16_t*>(v_sh.p[pk]) + (int64_t)kvh * D;
    if (r0 + BN <= s_l) {
      dma_tile_whole<D, BN, kWaves * 64>(K + r0 * a.kv_row, a.kv_row, kv_off, sK[b], wave);
      dma_tile_whole<D, BN, kWaves * 64>(V + r0 * a.kv_row, a.kv_row, kv_off, sV[b], wave);
    } else {
      dma_tile<D, BN, kWaves * 64>(K, a.kv_row, r0, s_l, sK[b], tid);
      dma_tile<D, BN, kWaves * 64>(V, a.kv_row, r0, s_l, sV[b], tid);
    }
  };
  auto load_sdp = [&](int b, int kb, int t, bf16x8& kx, bf16x8& vx) {
    kx = *reinterpret_cast<const bf16x8*>(&sK[b][tile_off<D>(kb * 32 + l32, 16 * t + 8 * hf)]);
    vx = *reinterpret_cast<const bf16x8*>(&sV[b][tile_off<D>(kb * 32 + l32, 16 * t + 8 * hf)]);
  };
  // K^T operands of dQ^T product i = (tt, db) of half kb; the second register is unused
  auto load_dq = [&](int b, int kb, int i, bf16x8& kt, bf16x8& unused) {
    const int tt = i / DB, db = i % DB;
    const int kr = kb * 32 + 16 * tt + 4 * hf + (li >> 2);
    const int col = db * 32 + 16 * (gi & 1) + 4 * (li & 3);
    const i16x4 k0v = lds_read_tr16(&sK[b][tile_off<D>(kr, col)]);
    const i16x4 k1v = lds_read_tr16(&sK[b][tile_off<D>(kr + 8, col)]);
    kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(k0v, k1v, 0, 1, 2, 3, 4, 5, 6, 7));
    (void)unused;
  };
  // dS of keys kb*32 + 8jj + 4hf + e (e < 4) for this lane's row, before the mask (keys
  // outside the row's range are zeroed afterwards by an unsigned compare, so no branch
  // surrounds the MFMAs)
  auto soft4 = [&](int kb, int jj, const f32x16& si, const f32x16& pi, f32x4& dv) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = fast_exp2(__builtin_fmaf(si[4 * jj + e], c, -lse2[0]));
      dv[e] = p * (pi[4 * jj + e] - dl[0]);
    }
  };
  auto pack8 = [](const f32x4& x, const f32x4& y) {
    u32x4 r;
    r[0] = pack_bf16x2(x[0], x[1]);
    r[1] = pack_bf16x2(x[2], x[3]);
    r[2] = pack_bf16x2(y[0], y[1]);
    r[3] = pack_bf16x2(y[2], y[3]);
    return __builtin_bit_cast(bf16x8, r);
  };

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

  constexpr int NC = 2 * DB;  // dQ products per half (tt, db)
  // one key tile; B is the buffer (compile time, as in the forward: the two buffers' LDS
  // addresses then differ by an immediate offset, so no per-read address arithmetic)
  auto tile_step = [&](auto B, int64_t k0) {
    constexpr int buf = decltype(B)::value;
    wait_dma();
    __syncthreads();  // tile k0 has landed and every wave is done with the previous tile
    const int32_t krel0 = (int32_t)(k0 - lo[0]) + 4 * hf;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      f32x16 sacc, pacc;
      // raised priority through S/dP and dS: the other wave on the SIMD fills the gaps with
      // its dQ products
      __builtin_amdgcn_s_setprio(1);
      {
        // K and V operands kDqPfA k-steps ahead of their products, behind scheduling barriers
        bf16x8 rk[kDqPfA + 1], rv[kDqPfA + 1];
#pragma unroll
        for (int t = 0; t < kDqPfA; ++t) load_sdp(buf, hh, t, rk[t], rv[t]);
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          if (t + kDqPfA < DT) load_sdp(buf, hh, t + kDqPfA, rk[(t + kDqPfA) % (kDqPfA + 1)], rv[(t + kDqPfA) % (kDqPfA + 1)]);
          sacc = mfma32x32x16(rk[t % (kDqPfA + 1)], qf[0][t], t == 0 ? f32x16{} : sacc);
          pacc = mfma32x32x16(rv[t % (kDqPfA + 1)], gf[0][t], t == 0 ? f32x16{} : pacc);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      f32x4 dv[4];
      bf16x8 dsf[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) soft4(hh, g, sacc, pacc, dv[g]);
      // dS is 0 outside the row's key range: applied in place, only on halves where some
      // row of the wave cannot see some key (a wave-uniform branch around VALU work)
      const int32_t kr = krel0 - 4 * hf + hh * 32;
      const bool full = (uint32_t)kr < width[0] && (uint32_t)(kr + 31) < width[0];
      if (__ballot(!full) != 0) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dv[g][e] = (uint32_t)(krel0 + hh * 32 + 8 * g + e) < width[0] ? dv[g][e] : 0.f;
      }
      dsf[0] = pack8(dv[0], dv[1]);
      dsf[1] = pack8(dv[2], dv[3]);
      __builtin_amdgcn_s_setprio(0);
      {
        // K^T operands kDqPfB products ahead
        bf16x8 rk[kDqPfB + 1], unused;
#pragma unroll
        for (int i = 0; i < kDqPfB; ++i) load_dq(buf, hh, i, rk[i], unused);
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          if (i + kDqPfB < NC) load_dq(buf, hh, i + kDqPfB, rk[(i + kDqPfB) % (kDqPfB + 1)], unused);
          dqacc[i % DB] = mfma32x32x16(rk[i % (kDqPfB + 1)], dsf[i / DB], dqacc[i % DB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the next tile's DMA after this tile's last LDS read: the wait the compiler places
    // before LDS reads that follow a DMA then falls on the next barrier
    if (k0 + BN < kend) issue_kv(k0 + BN, buf ^ 1);
  };
  if (kbeg < kend) issue_kv(kbeg, 0);
  for (int64_t k0 = kbeg;;) {
    if (k0 >= kend) break;
    tile_step(std::integral_constant<int, 0>{}, k0);
    k0 += BN;
    if (k0 >= kend) break;
    tile_step(std::integral_constant<int, 1>{}, k0);
    k0 += BN;
  }

  const int rb = 0;
  if (nsq > 1) {
    // this split's fp32 partial sums (unscaled) into its slot; the reduce kernel finishes them
    if (row[rb] < s) {
      float* slot = a.dq_part + (((int64_t)h * nmb + mb) * nsq + sp) * (BM * D) + (int64_t)(wave * 32 + l32) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(slot + db * 32 + 8 * jj + 4 * hf) =
              f32x4{dqacc[db][4 * jj + 0], dqacc[db][4 * jj + 1], dqacc[db][4 * jj + 2], dqacc[db][4 * jj + 3]};
    }
    return;
  }
  uint16_t* dQ = static_cast<uint16_t*>(const_cast<void*>(dq_sh.p[ps])) + (int64_t)h * D - r_sh * a.q_row;
  if (a.acc_q != nullptr && row[rb] < s) {
    // sums carried across launches (Ring Attention's hops): add the previous fp32 sums unless
    // this launch starts them, store them back unless it ends them
    float* accp = a.acc_q + row[rb] * a.q_row + (int64_t)h * D;
    if (a.acc_init == 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 prev = *reinterpret_cast<const f32x4*>(accp + db * 32 + 8 * jj + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) dqacc[db][4 * jj + e] += prev[e];
        }
    }
    if (a.acc_final == 0) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(accp + db * 32 + 8 * jj + 4 * hf) =
              f32x4{dqacc[db][4 * jj + 0], dqacc[db][4 * jj + 1], dqacc[db][4 * jj + 2], dqacc[db][4 * jj + 3]};
      return;
    }
  }
  if (row[rb] < s) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 w;
        w[0] = pack_bf16x2(dqacc[db][4 * jj + 0] * a.scale, dqacc[db][4 * jj + 1] * a.scale);
        w[1] = pack_bf16x2(dqacc[db][4 * jj + 2] * a.scale, dqacc[db][4 * jj + 3] * a.scale);
        *reinterpret_cast<u32x2*>(dQ + row[rb] * a.q_row + db * 32 + 8 * jj + 4 * hf) = w;
      }
  }
}

// ---------------------------------------------------------------------------------------
// dK/dV with split roles: one workgroup = 128 keys of one kv head and 8 waves, two per SIMD.
// Waves 0-3 ("P waves", keys 32w..32w+31) compute S = Q K^T, P = exp(S - LSE) (masked) and
// dV^T += dO^T P; waves 4-7 ("dS waves", the same keys) compute dP = dO V^T, read P from LDS,
// form dS = P (dP - delta) and dK^T += Q^T dS. Each wave holds one accumulator set (dV or
// dK) and one of K/V, so two waves fit a SIMD and one's VALU work overlaps the other's MFMAs.
// Per 64-row query tile: S | dP, barrier, dV | dS + dK. P crosses in fp32 through LDS, in the
// MFMA accumulator layout of the lane that made it (each dS lane reads its own twin's slot).
// Query tiles (Q, dO, LSE, delta) arrive by DMA into double buffers that are distinct LDS
// objects, with steps unrolled by two so buffer choices are compile-time: the compiler then
// knows the DMA into one buffer does not alias reads of the other.
template <int D>
struct DkvSplitCfg {
  static constexpr int BNK = 128, BMQ = 64, NW = 8;
  static constexpr int DT = D / 16, DB = D / 32;
};
// Launch order of the key blocks of a causal packed sequence (at most 64 documents): longest
// first, i.e. by decreasing count of query tiles, ties by position, so that the blocks at the
// start of a long document do not wait behind the short blocks before it. A block whose last
// key lies in document d (blocks floor(cu[d]/128) .. floor(cu[d+1]/128) - 1) sees the query
// tiles from its own first row to the document's end E_d: A_d - 2 kb of them, A_d = ceil(E_d/64).
// Every wave finds the block of rank r itself: lane d holds document d, a binary search over the
// tile count t on C(t) = #{blocks with at least t tiles} (a wave-wide sum) finds the count of
// rank r, and the block is the (r - C(t+1))-th document, in order, with a block of exactly t
// tiles (at most one per document). Bitwise-neutral: only the order of the workgroups changes.
__device__ int lpt_key_block(const int32_t* cu, int n_docs, int s, int nkb, int r) {
  const int lane = threadIdx.x & 63;
  const bool on = lane < n_docs;
  const int c0 = on ? cu[lane] : s, c1 = on ? cu[lane + 1] : s;
  const int a0 = c0 >= s ? nkb : c0 / 128;      // first block of the document
  const int b1 = (c1 >= s ? nkb : c1 / 128) - 1;  // last block of the document
  const int e = c1 < s ? c1 : s;
  const int A = (e + 63) / 64;
  auto count = [&](int t) {  // blocks of this lane's document with at least t tiles
    if (!on || b1 < a0 || A < t) return 0;
    const int hi = (A - t) / 2 < b1 ? (A - t) / 2 : b1;
    return hi >= a0 ? hi - a0 + 1 : 0;
  };
  auto wsum = [](int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
  };
  int tmax = on ? A : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int u = __shfl_xor(tmax, o);
    tmax = u > tmax ? u : tmax;
  }
  int lo = 1, hi = tmax + 1;  // C(lo) > r >= C(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (wsum(count(mid)) > r) lo = mid;
    else hi = mid;
  }
  int m = r - wsum(count(lo + 1));
  const int kbd = (A - lo) / 2;
  const bool has = on && A >= lo && ((A - lo) & 1) == 0 && kbd >= a0 && kbd <= b1;
  uint64_t mask = __ballot(has);
  for (; m > 0 && mask != 0; --m) mask &= mask - 1;
  const int res = mask != 0 ? __shfl(kbd, __builtin_ctzll(mask)) : -1;
  // a block in range whatever cu holds, made wave-uniform (what derives from it stays scalar)
  return __builtin_amdgcn_readfirstlane(res >= 0 && res < nkb ? res : r);
}

// k-step of part A at which the dS waves issue the next tile's DMA (it must land by the barrier
// that ends part A: issued later than this, its latency shows there)
constexpr int kDkvDmaAt = 2;

template <int D>
__global__ __launch_bounds__(512, 1) void attn_dkdv_split_kernel(AttnArgs a, Shards q_sh, Shards g_sh, Shards k_sh,
                                                                 Shards v_sh, Shards dk_sh, Shards dv_sh, int64_t s_l) {
  using C = DkvSplitCfg<D>;
  constexpr int BNK = C::BNK, BMQ = C::BMQ, DT = C::DT, DB = C::DB;
  // per buffer: one object for the Q and dO tiles, one for the LSE and delta rows (few DMA
  // target objects keep the compiler's per-object tracking of LDS DMA exact)
  __shared__ __attribute__((aligned(16))) uint16_t sT0[2 * BMQ * D], sT1[2 * BMQ * D];
  __shared__ __attribute__((aligned(16))) float sS0[2 * BMQ], sS1[2 * BMQ];
  // P of key group g, half qb: 4 chunks x 64 lanes x 4 floats, chunk-major, so one 16-byte
  // access per lane of a chunk covers 1 KiB of consecutive slots (no bank conflicts)
  __shared__ __attribute__((aligned(16))) float sP[4][2][64 * 16];
  struct Buf {
    uint16_t* q;
    uint16_t* g;
    float* l;
    float* d;
  };
  auto bufs = [&](auto B) -> Buf {
    if constexpr (decltype(B)::value == 0) return {sT0, sT0 + BMQ * D, sS0, sS0 + BMQ};
    else return {sT1, sT1 + BMQ * D, sS1, sS1 + BMQ};
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int role = wave >> 2, kg = wave & 3;  // role 0: P and dV; role 1: dS and dK
  const int l32 = lane & 31, hf = lane >> 5, gi = lane >> 4, li = lane & 15;
  const int64_t s = a.s;
  const int kvh = blockIdx.x % a.n_kv;
  const int sp = (int)((blockIdx.x / a.n_kv) % a.nsplit);                 // split of the key block
  int64_t kb = (int64_t)(blockIdx.x / a.n_kv) / a.nsplit;  // earliest keys (most rows) first
  if (a.cu != nullptr && a.causal && a.nsplit == 1 && a.n_docs <= 64)
    kb = lpt_key_block(a.cu, a.n_docs, (int)s, (int)((s + BNK - 1) / BNK), (int)kb);
  const int64_t n0 = kb * BNK;
  const float c = a.scale * kLog2e;

  // this lane's key, the rows that may see it [rlo, rhi), and its K (role 0) or V row
  const int64_t key = n0 + kg * 32 + l32;
  int32_t rlo = 0, rhi = (int32_t)s;  // positions fit in int32 (the boundary checks s)
  if (a.cu != nullptr && key < s) {
    const int dk = doc_of(a.cu, a.n_docs, key);
    rlo = a.cu[dk];
    rhi = a.cu[dk + 1] < (int32_t)s ? a.cu[dk + 1] : (int32_t)s;
  }
  if (a.causal) rlo = (int32_t)key;
  if (key >= s) rhi = rlo;  // padding key: seen by no row
  const uint32_t width = (uint32_t)(rhi - rlo);  // row r is seen iff (uint32)(r - rlo) < width
  // shard of the workgroup's keys (all in one); K/V rows and dK/dV addressed from its first row
  const int pk = (int)((uint32_t)n0 / (uint32_t)s_l);
  const int64_t k_sh0 = (int64_t)pk * s_l;
  const uint16_t* KV = static_cast<const uint16_t*>(role == 0 ? k_sh.p[pk] : v_sh.p[pk]) + (int64_t)kvh * D -
                       k_sh0 * a.kv_row;
  bf16x8 kv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    u32x4 x = {0, 0, 0, 0};
    if (key < s) x = *reinterpret_cast<const u32x4*>(KV + key * a.kv_row + 16 * t + 8 * hf);
    kv[t] = __builtin_bit_cast(bf16x8, x);
  }

  // row range of the workgroup: rows that may see any of its keys
  const int64_t last_key = (n0 + BNK < s ? n0 + BNK : s) - 1;
  int64_t qbeg = a.causal ? n0 : 0, qend = s;
  if (a.cu != nullptr) {
    // document bounds clamped to [0, s]: no tile outside the sequence is ever visited
    qend = a.cu[doc_of(a.cu, a.n_docs, last_key) + 1];
    qend = qend < s ? qend : s;
    if (!a.causal) qbeg = a.cu[doc_of(a.cu, a.n_docs, n0)];
    qbeg = qbeg > 0 ? qbeg : 0;
  }
  qbeg = (qbeg / BMQ) * BMQ;
  const int ntile = qend > qbeg ? (int)((qend - qbeg + BMQ - 1) / BMQ) : 0;
  const KvHeads kh = kv_heads_of(a, kvh);  // the launch's q heads reading this kv head
  const int GH = kh.j1 - kh.j0;
  // steps [st0, st0 + nsteps) of the block's ntile * GH (all of them unless split)
  const int st0 = (int)((int64_t)ntile * GH * sp / a.nsplit);
  const int nsteps = (int)((int64_t)ntile * GH * (sp + 1) / a.nsplit) - st0;

  // Steps walk the query tiles from the last one down, the GH heads of a tile back to back.
  auto tile_row0 = [&](int tile) { return qbeg + (int64_t)(ntile - 1 - tile) * BMQ; };
  // Only the dS waves issue DMA: the P waves then never hold outstanding DMA, so nothing
  // makes them wait for it before their LDS writes of P.
  // Q and dO share the row stride: one lane offset (of the dS waves' 256 threads) serves both
  const uint32_t qg_off = dma_lane_offset<D, 256>(a.q_row, tid & 255);
  auto issue_tile = [&](int tile, int hi, const Buf& b) {
    const int hq = kh.j0 + hi;
    const int64_t q0 = tile_row0(tile);
    const int pq = (int)((uint32_t)q0 / (uint32_t)s_l);
    const int64_t r0 = q0 - (int64_t)pq * s_l;
    const uint16_t* Qh = static_cast<const uint16_t*>(q_sh.p[pq]) + (int64_t)hq * D;
    const uint16_t* Gh = static_cast<const uint16_t*>(g_sh.p[pq]) + (int64_t)hq * D;
    if (r0 + BMQ <= s_l) {
      const int w4 = __builtin_amdgcn_readfirstlane(wave - 4);
      dma_tile_whole<D, BMQ, 256>(Qh + r0 * a.q_row, a.q_row, qg_off, b.q, w4);
      dma_tile_whole<D, BMQ, 256>(Gh + r0 * a.q_row, a.q_row, qg_off, b.g, w4);
    } else {
      // a shard's ragged last tile: the thread index through an empty asm, so this rare path's
      // address arithmetic is formed here rather than hoisted into registers for the whole loop
      int t2 = tid - 256;
      asm volatile("" : "+v"(t2));
      dma_tile<D, BMQ, 256>(Qh, a.q_row, r0, s_l, b.q, t2);
      dma_tile<D, BMQ, 256>(Gh, a.q_row, r0, s_l, b.g, t2);
    }
    // one fp32 per lane: lane i lands at b.l[i] (wave 4) or b.d[i] (wave 5)
    int64_t qr = q0 + (lane < BMQ ? lane : BMQ - 1);
    qr = qr < s ? qr : s - 1;
    if (wave == 4) __builtin_amdgcn_global_load_lds(a.lse_in + (int64_t)hq * a.lse_row + qr, b.l, 4, 0, 0);
    if (wave == 5) __builtin_amdgcn_global_load_lds(a.delta + (int64_t)hq * a.lse_row + qr, b.d, 4, 0, 0);
  };
  auto p_off = [&](int qb, int chunk) {  // float offset of this lane's 16-byte chunk of P
    return (((kg * 2 + qb) * 4 + chunk) * 64 + lane) * 4;
  };
  auto pack8 = [](const f32x16& x, int h) {
    u32x4 r;
    r[0] = pack_bf16x2(x[8 * h + 0], x[8 * h + 1]);
    r[1] = pack_bf16x2(x[8 * h + 2], x[8 * h + 3]);
    r[2] = pack_bf16x2(x[8 * h + 4], x[8 * h + 5]);
    r[3] = pack_bf16x2(x[8 * h + 6], x[8 * h + 7]);
    return __builtin_bit_cast(bf16x8, r);
  };
  // transposed operand (dO^T for role 0, Q^T for role 1) of product (qb, tt, db)
  auto load_tr = [&](const uint16_t* tile, int qb, int tt, int db) {
    const int qr = qb * 32 + 16 * tt + 4 * hf + (li >> 2);
    const int col = db * 32 + 16 * (gi & 1) + 4 * (li & 3);
    const i16x4 x0 = lds_read_tr16(&tile[tile_off<D>(qr, col)]);
    const i16x4 x1 = lds_read_tr16(&tile[tile_off<D>(qr + 8, col)]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 acc[DB];  // dV^T (role 0) or dK^T (role 1), d x key
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  int cur_t = st0 / (GH > 0 ? GH : 1), cur_h = st0 - cur_t * GH;  // tile and head of this step
  auto run_step = [&](auto B, int step) {
    const Buf buf = bufs(B), nbuf = bufs(std::integral_constant<int, 1 - decltype(B)::value>{});
    wait_dma();
    __syncthreads();  // tile `step` has landed; every wave is done with tile step-1 and with P
    const int nxt_h = cur_h + 1 == GH ? 0 : cur_h + 1;
    const int nxt_t = cur_h + 1 == GH ? cur_t + 1 : cur_t;
    const bool issue_next = role == 1 && step + 1 < nsteps;  // the next tile's DMA (in part A)
    const int32_t qrel0 = (int32_t)tile_row0(cur_t) - rlo + 4 * hf;
    cur_t = nxt_t;
    cur_h = nxt_h;
    // The two roles run separate code, each naming its LDS objects directly (a runtime choice
    // between buffers would hide from the compiler which object a read touches).
    f32x16 x[2];
    bf16x8 op[2][2];  // P (role 0) or dS (role 1) as bf16 MFMA operands, [qb][tt]
    auto part_a = [&](auto ROLE) {
      constexpr int r = decltype(ROLE)::value;
      // S (role 0) or dP (role 1), row x key: the query-side operand is Q or dO
      const uint16_t* qs = r == 0 ? buf.q : buf.g;
      // operands of k-step t+1 are read while the MFMAs of k-step t run (the scheduling
      // barriers keep that order; left alone, the compiler reads each just before its use)
      bf16x8 ring[2][2];
      auto ld = [&](int t, bf16x8 (&o)[2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          o[qb] = *reinterpret_cast<const bf16x8*>(&qs[tile_off<D>(qb * 32 + l32, 16 * t + 8 * hf)]);
      };
      ld(0, ring[0]);
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        if (t + 1 < DT) ld(t + 1, ring[(t + 1) & 1]);
        // the dS waves request the next tile after their first kDkvDmaAt k-steps: issued at the
        // step's start, the DMA instructions held up the wave's first products
        if constexpr (r == 1) {
          if (t == kDkvDmaAt && issue_next) issue_tile(nxt_t, nxt_h, nbuf);
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) x[qb] = mfma32x32x16(ring[t & 1][qb], kv[t], t == 0 ? f32x16{} : x[qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (r == 0) {
        // P = exp2(S c - LSE log2e) on rows 32qb + 8(j/4) + 4hf + j%4 (the LSE rows are in
        // log2 units in LDS already)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 L4 = *reinterpret_cast<const f32x4*>(&buf.l[qb * 32 + 8 * jj + 4 * hf]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[qb][4 * jj + e] = fast_exp2(__builtin_fmaf(x[qb][4 * jj + e], c, -L4[e]));
          }
        }
        // 0 outside [rlo, rhi): only where some row of the tile cannot see some key of the
        // wave (a wave-uniform branch around VALU work on P in place)
        const int32_t qr = qrel0 - 4 * hf;
        const bool full = (uint32_t)qr < width && (uint32_t)(qr + BMQ - 1) < width;
        if (__ballot(!full) != 0) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int j = 0; j < 16; ++j)
              x[qb][j] = (uint32_t)(qrel0 + qb * 32 + 8 * (j / 4) + (j % 4)) < width ? x[qb][j] : 0.f;
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            *reinterpret_cast<f32x4*>(&sP[0][0][p_off(qb, jj)]) =
                f32x4{x[qb][4 * jj], x[qb][4 * jj + 1], x[qb][4 * jj + 2], x[qb][4 * jj + 3]};
          op[qb][0] = pack8(x[qb], 0);
          op[qb][1] = pack8(x[qb], 1);
        }
      }
    };
    auto part_b = [&](auto ROLE) {
      constexpr int r = decltype(ROLE)::value;
      // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1): products i = (qb, tt, db), their
      // transposed operands read three products ahead (the first three before the dS work)
      const uint16_t* ts = r == 0 ? buf.g : buf.q;
      constexpr int NP = 4 * DB, PF = 3;
      bf16x8 ringb[PF + 1];
      auto ldb = [&](int i) { return load_tr(ts, i / (2 * DB), (i / DB) % 2, i % DB); };
#pragma unroll
      for (int i = 0; i < PF; ++i) ringb[i] = ldb(i);
      if constexpr (r == 1) {
        // dS = P (dP - delta)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 D4 = *reinterpret_cast<const f32x4*>(&buf.d[qb * 32 + 8 * jj + 4 * hf]);
            const f32x4 P4 = *reinterpret_cast<const f32x4*>(&sP[0][0][p_off(qb, jj)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[qb][4 * jj + e] = P4[e] * (x[qb][4 * jj + e] - D4[e]);
          }
          op[qb][0] = pack8(x[qb], 0);
          op[qb][1] = pack8(x[qb], 1);
        }
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + PF < NP) ringb[(i + PF) % (PF + 1)] = ldb(i + PF);
        acc[i % DB] = mfma32x32x16(ringb[i % (PF + 1)], op[i / (2 * DB)][(i / DB) % 2], acc[i % DB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (role == 0) part_a(std::integral_constant<int, 0>{});
    else part_a(std::integral_constant<int, 1>{});
    __syncthreads();  // P of this tile is in LDS
    // the dS waves go first in part B: their dS work is the longer path to the next barrier
    if (role == 0) {
      part_b(std::integral_constant<int, 0>{});
    } else {
      __builtin_amdgcn_s_setprio(1);
      part_b(std::integral_constant<int, 1>{});
      __builtin_amdgcn_s_setprio(0);
      // the wave that fetched the next tile's LSE rows turns them into log2 units once, so
      // the P waves need no multiply per element (published by the next step's barrier)
      if (wave == 4 && step + 1 < nsteps) {
        wait_dma();
        nbuf.l[lane] *= kLog2e;
      }
    }
  };

  if (nsteps > 0) {
    if (role == 1) issue_tile(cur_t, cur_h, bufs(std::integral_constant<int, 0>{}));
    if (wave == 4) {  // LSE rows of the first tile in log2 units
      wait_dma();
      bufs(std::integral_constant<int, 0>{}).l[lane] *= kLog2e;
    }
    for (int step = 0;;) {
      run_step(std::integral_constant<int, 0>{}, step);
      if (++step >= nsteps) break;
      run_step(std::integral_constant<int, 1>{}, step);
      if (++step >= nsteps) break;
    }
  }

  if (a.nsplit > 1) {
    // this split's fp32 partial sums (unscaled) into its slot; the reduce kernel finishes them
    if (key < s) {
      float* slot = a.dkv_part + ((((int64_t)kvh * ((s + BNK - 1) / BNK) + kb) * a.nsplit + sp) * 2 + role) *
                                     (BNK * D) + (int64_t)(kg * 32 + l32) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(slot + db * 32 + 8 * jj + 4 * hf) =
              f32x4{acc[db][4 * jj + 0], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]};
    }
    return;
  }
  if (key < s) {
    const bool is_k = role == 1;
    const int64_t off = (int64_t)kvh * D + key * a.dkv_row;
    const float f = is_k ? a.scale : 1.0f;
    // headwise-chunked backward: fp32 sums carried across launches, rounded once at the end
    float* accp = a.acc_k == nullptr ? nullptr
                                     : (is_k ? a.acc_k : a.acc_v) + (int64_t)kvh * D + key * a.acc_row;
    const bool acc_first = a.acc_init >= 0 ? a.acc_init != 0 : kh.first;
    const bool acc_last = a.acc_final >= 0 ? a.acc_final != 0 : kh.last;
    if (accp != nullptr && !acc_first) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 prev = *reinterpret_cast<const f32x4*>(accp + db * 32 + 8 * jj + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * jj + e] += prev[e];
        }
    }
    if (accp != nullptr && !acc_last) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(accp + db * 32 + 8 * jj + 4 * hf) =
              f32x4{acc[db][4 * jj + 0], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]};
    } else {
      uint16_t* out = static_cast<uint16_t*>(const_cast<void*>(is_k ? dk_sh.p[pk] : dv_sh.p[pk])) + off -
                      k_sh0 * a.dkv_row;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32x2 w;
          w[0] = pack_bf16x2(acc[db][4 * jj + 0] * f, acc[db][4 * jj + 1] * f);
          w[1] = pack_bf16x2(acc[db][4 * jj + 2] * f, acc[db][4 * jj + 3] * f);
          *reinterpret_cast<u32x2*>(out + db * 32 + 8 * jj + 4 * hf) = w;
        }
    }
  }
}

template <typename T, int D>
hipError_t launch_pre_t(const AttnArgs& a, const BwdSrc& src, hipStream_t stream) {
  constexpr int TPR = D * (int)sizeof(T) / 16;
  const int64_t items = a.s * a.n_heads;
  const int64_t blocks = (items + (256 / TPR) - 1) / (256 / TPR);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, a, src.o, src.g, src.s_l);
  return hipGetLastError();
}

// dQ of split row blocks: for 8 consecutive elements of one row and q head, the nsplit_q partial
// sums in split order (from +0), scaled and rounded once, one thread each
template <int D>
__global__ __launch_bounds__(256) void dq_reduce_kernel(AttnArgs a, Shards dq_sh, int64_t s_l) {
  constexpr int BM = 128, PER = D / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t s = a.s, nmb = (s + BM - 1) / BM;
  const int64_t total = (int64_t)a.n_heads * s * PER;
  if (c >= total) return;
  const int part8 = (int)(c % PER);
  const int64_t row = (c / PER) % s;
  const int h = (int)(c / PER / s);
  const int ns = a.nsplit_q;
  const int64_t mb = row / BM;
  const float* src = a.dq_part + ((int64_t)h * nmb + mb) * ns * (BM * D) + (row - mb * BM) * D + part8 * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ns; ++sp) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src + (int64_t)sp * (BM * D));
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + (int64_t)sp * (BM * D) + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += x0[e];
      acc[4 + e] += x1[e];
    }
  }
  const int p = (int)((uint32_t)row / (uint32_t)s_l);
  uint16_t* out = static_cast<uint16_t*>(const_cast<void*>(dq_sh.p[p])) + (row - (int64_t)p * s_l) * a.q_row +
                  (int64_t)h * D + part8 * 8;
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[2 * e] * a.scale, acc[2 * e + 1] * a.scale);
  *reinterpret_cast<u32x4*>(out) = w;
}

template <int D, int RB, int KB>
hipError_t launch_dq_t(const AttnArgs& a, const BwdSrc& src, hipStream_t stream) {
  using C = DqCfg<D, RB, KB>;
  const int nsq = a.nsplit_q > 1 ? a.nsplit_q : 1;
  const int64_t blocks = (a.s + C::BM - 1) / C::BM * a.n_heads * nsq;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_dq_kernel<D, RB, KB>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a, src.q,
                     src.g, src.k, src.v, src.dq, src.s_l);
  if (nsq > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)a.n_heads * a.s * (D / 8);
    hipLaunchKernelGGL((dq_reduce_kernel<D>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a, src.dq,
                       src.s_l);
  }
  return hipGetLastError();
}

// dK/dV of split key blocks: for 8 consecutive elements of one key and kv head, the nsplit
// partial sums in split order (from +0), scaled (dK) and rounded once, one thread each
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(AttnArgs a, Shards dk_sh, Shards dv_sh, int64_t s_l) {
  constexpr int BNK = 128, PER = D / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t s = a.s, nkb = (s + BNK - 1) / BNK;
  const int64_t total = 2 * (int64_t)a.n_kv * s * PER;
  if (c >= total) return;
  const int part8 = (int)(c % PER);
  const int64_t key = (c / PER) % s;
  const int64_t rest = c / PER / s;
  const int kvh = (int)(rest % a.n_kv), is_k = (int)(rest / a.n_kv);
  const int64_t kb = key / BNK;
  const float* slot0 = a.dkv_part + ((((int64_t)kvh * nkb + kb) * a.nsplit) * 2 + is_k) * (BNK * D) +
                       (key - kb * BNK) * D + part8 * 8;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* p = slot0 + (int64_t)sp * 2 * (BNK * D);
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p), hi = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] += lo[e];
      x[4 + e] += hi[e];
    }
  }
  const float f = is_k ? a.scale : 1.0f;
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i] * f, x[2 * i + 1] * f);
  const int pk = (int)((uint32_t)key / (uint32_t)s_l);
  uint16_t* out = static_cast<uint16_t*>(const_cast<void*>(is_k ? dk_sh.p[pk] : dv_sh.p[pk])) +
                  (key - (int64_t)pk * s_l) * a.dkv_row + (int64_t)kvh * D + part8 * 8;
  *reinterpret_cast<u32x4*>(out) = w;
}

template <int D>
hipError_t launch_dkdv_split_t(const AttnArgs& a, const BwdSrc& src, hipStream_t stream) {
  using C = DkvSplitCfg<D>;
  const int64_t blocks = (a.s + C::BNK - 1) / C::BNK * a.n_kv * (a.nsplit > 1 ? a.nsplit : 1);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_dkdv_split_kernel<D>), dim3((unsigned)blocks), dim3(C::NW * 64), 0, stream, a, src.q,
                     src.g, src.k, src.v, src.dk, src.dv, src.s_l);
  if (a.nsplit > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t items = 2 * (int64_t)a.n_kv * a.s * (D / 8);
    hipLaunchKernelGGL((dkdv_reduce_kernel<D>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, a, src.dk,
                       src.dv, src.s_l);
  }
  return hipGetLastError();
}

}  // namespace

int dq_split_count(int64_t s, int n_heads) {
  // two four-wave workgroups per CU (512 slots), row blocks launched longest first: the last
  // row block sees every key (twice the mean for one causal sequence), so the grid balances
  // only from about two rounds; below that, split every block's key tiles, aiming at 1024
  // workgroups, at most 8 per block
  const int64_t wg = (s + 127) / 128 * n_heads;
  if (wg >= 1024 || wg < 1) return 1;
  const int64_t ns = (1024 + wg - 1) / wg;
  return (int)(ns < 8 ? ns : 8);
}

int dkdv_split_count(int64_t s, int n_kv) {
  // one eight-wave workgroup per CU, blocks launched longest first: a causal grid balances
  // over the 256 CUs only from about two rounds (the first block walks twice the mean), so
  // split the key blocks' rows while the grid is under 512, aiming at 512 workgroups, at
  // most 8 per block
  const int64_t wg = (s + 127) / 128 * n_kv;
  if (wg >= 512 || wg < 1) return 1;
  const int64_t ns = (512 + wg - 1) / wg;
  return (int)(ns < 8 ? ns : 8);
}

namespace {
// the packed head-shard buffers of AttnArgs as one-shard tables
BwdSrc packed_src(const AttnArgs& a) {
  BwdSrc src{};
  src.q.p[0] = a.q;
  src.k.p[0] = a.k;
  src.v.p[0] = a.v;
  src.o.p[0] = a.o;
  src.g.p[0] = a.dout;
  src.dq.p[0] = a.out;
  src.dk.p[0] = a.out_k;
  src.dv.p[0] = a.out_v;
  src.s_l = a.s;
  return src;
}
}  // namespace

hipError_t launch_bwd_preprocess(const AttnArgs& a, int d, int dtype, hipStream_t stream) {
  const BwdSrc src = packed_src(a);
  if (dtype == ULY_BF16)
    return d == 128 ? launch_pre_t<uint16_t, 128>(a, src, stream) : launch_pre_t<uint16_t, 64>(a, src, stream);
  return d == 128 ? launch_pre_t<float, 128>(a, src, stream) : launch_pre_t<float, 64>(a, src, stream);
}

hipError_t launch_attn_dq_bf16(const AttnArgs& a, int d, hipStream_t stream) {
  return launch_attn_dq_bf16_shards(a, packed_src(a), d, stream);
}

hipError_t launch_attn_dkdv_bf16(const AttnArgs& a, int d, hipStream_t stream) {
  return launch_attn_dkdv_bf16_shards(a, packed_src(a), d, stream);
}

hipError_t launch_bwd_preprocess_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream) {
  return d == 128 ? launch_pre_t<uint16_t, 128>(a, src, stream) : launch_pre_t<uint16_t, 64>(a, src, stream);
}

hipError_t launch_attn_dq_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream) {
  if (d == 128) return launch_dq_t<128, 1, 2>(a, src, stream);
  return launch_dq_t<64, 1, 2>(a, src, stream);
}

hipError_t launch_attn_dkdv_bf16_shards(const AttnArgs& a, const BwdSrc& src, int d, hipStream_t stream) {
  if (d == 128) return launch_dkdv_split_t<128>(a, src, stream);
  return launch_dkdv_split_t<64>(a, src, stream);
}

}  // namespace uly
