// Causal / packed-document GQA attention forward for one head shard, bf16 in, fp32
// accumulation, on gfx950 matrix cores.
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts", section
// "how Ulysses works", step 4 (each GPU runs local attention for its heads over every
// position) and the long-sequence section (FlashAttention keeps memory O(n) while the
// compute stays O(n^2)): the kernel streams K/V tiles past resident Q rows with an
// online softmax, so the s x s score matrix never exists.
//
// Work decomposition (one workgroup = 4 waves = BM query rows of one q head):
//   * each wave owns RB blocks of 32 query rows; its Q rows stay in VGPRs for the whole
//     key loop as MFMA B operands;
//   * K/V tiles of BN keys are staged in LDS (double buffered) and shared by the 4 waves;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 leaves each lane one query row and 16 of
//     the tile's keys, so the row max and row sum are lane-local plus one swap with the
//     lane 32 away;
//   * O^T += V^T P^T: P (bf16) is already in B-operand layout, V^T comes straight from
//     the row-major V tile through the transposing LDS read (ds_read_b64_tr_b16), and the
//     O^T accumulator keeps each lane's query row, so softmax rescales stay lane-local;
//   * the exponent is exp2 with scale*log2(e) folded into one FMA, and the running max is
//     only moved when a row's max grows by more than kTau (2^8): P then stays <= 256,
//     exact in the final O / l, and most tiles skip the O rescale;
//   * causal / document tiles outside a row block's range are never visited; partial
//     tiles are masked per element; workgroups with the longest key range launch first.
#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kWaves = 4;
constexpr float kTau = 8.0f;

// Tile shape of the d=128 kernel: 32-row blocks per wave and workgroups per CU.
#ifndef ULY_FWD_RB
#define ULY_FWD_RB 1
#endif
#ifndef ULY_FWD_KB
#define ULY_FWD_KB 1
#endif
#ifndef ULY_FWD_OCC
#define ULY_FWD_OCC 2
#endif

template <int D, int RB, int KB>
struct FwdCfg {
  static constexpr int BM = kWaves * RB * 32;  // query rows per workgroup
  static constexpr int BN = KB * 32;           // keys per tile
  static constexpr int DT = D / 16;            // 16-wide contraction steps over d
  static constexpr int DB = D / 32;            // 32-wide d blocks of O^T
  static constexpr int KSTR = D + 8;           // K tile row stride (elements): conflict-free b128 reads
  static constexpr int VSTR = D + 32;          // V tile row stride: conflict-free transposing reads
  static constexpr int KVEC = BN * D / 8 / (kWaves * 64);  // 16-byte vectors per thread per tile
};

template <int D, int RB, int KB, int OCC>
__global__ __launch_bounds__(kWaves * 64, OCC) void attn_fwd_kernel(AttnArgs a) {
  using C = FwdCfg<D, RB, KB>;
  constexpr int BM = C::BM, BN = C::BN, DT = C::DT, DB = C::DB, KSTR = C::KSTR, VSTR = C::VSTR;
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t s = a.s;
  const int nmb = (int)((s + BM - 1) / BM);
  const int h = blockIdx.x % a.n_heads;
  const int mb = nmb - 1 - (int)(blockIdx.x / a.n_heads);  // longest causal rows first
  const int64_t m0 = (int64_t)mb * BM;
  const int kvh = (h + a.q_off) / a.G - a.kv_off;
  const uint16_t* Q = static_cast<const uint16_t*>(a.q) + (int64_t)h * D;
  const uint16_t* K = static_cast<const uint16_t*>(a.k) + (int64_t)kvh * D;
  const uint16_t* V = static_cast<const uint16_t*>(a.v) + (int64_t)kvh * D;
  const float c = a.scale * kLog2e;

  // ---- this lane's query rows and their visible key ranges [lo, hi)
  int64_t row[RB], lo[RB], hi[RB];
  bf16x8 qf[RB][DT];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    row[rb] = m0 + wave * RB * 32 + rb * 32 + l32;
    lo[rb] = 0;
    hi[rb] = s;
    if (a.cu != nullptr && row[rb] < s) {
      const int dk = doc_of(a.cu, a.n_docs, row[rb]);
      lo[rb] = a.cu[dk];
      hi[rb] = a.cu[dk + 1];
    }
    if (a.causal) hi[rb] = hi[rb] < row[rb] + 1 ? hi[rb] : row[rb] + 1;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      u32x4 v = {0, 0, 0, 0};
      if (row[rb] < s) v = *reinterpret_cast<const u32x4*>(Q + row[rb] * a.q_row + 16 * t + 8 * hf);
      qf[rb][t] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- key range of the workgroup and of this wave
  const int64_t wr0 = m0 + wave * RB * 32;                          // first row of the wave
  const int64_t wr1 = (wr0 + RB * 32 < s ? wr0 + RB * 32 : s) - 1;  // last valid row
  const int64_t last_row = (m0 + BM < s ? m0 + BM : s) - 1;
  int64_t kbeg = 0, kend = s, wkbeg = 0, wkend = s, w_lo_last = 0, w_hi_first = s;
  if (a.cu != nullptr) {
    kbeg = a.cu[doc_of(a.cu, a.n_docs, m0)];
    kend = a.cu[doc_of(a.cu, a.n_docs, last_row) + 1];
    if (wr0 < s) {
      wkbeg = a.cu[doc_of(a.cu, a.n_docs, wr0)];
      w_hi_first = a.cu[doc_of(a.cu, a.n_docs, wr0) + 1];
      w_lo_last = a.cu[doc_of(a.cu, a.n_docs, wr1)];
      wkend = a.cu[doc_of(a.cu, a.n_docs, wr1) + 1];
    }
  }
  if (a.causal) {
    kend = kend < last_row + 1 ? kend : last_row + 1;
    wkend = wkend < wr1 + 1 ? wkend : wr1 + 1;
  }
  kbeg = (kbeg / BN) * BN;
  const bool wave_has_rows = wr0 < s;

  // ---- K/V tile staging: global -> registers -> LDS, two LDS buffers each.
  // In iteration j the waves read K(j+1) (stored before this iteration's barrier) and V(j)
  // (stored after the previous barrier); V(j+1) is stored only after this barrier, when
  // every wave is done with V(j-1), whose buffer it reuses.
  u32x4 pk[C::KVEC], pv[C::KVEC];
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::KVEC; ++i) {
      const int vi = tid + i * kWaves * 64;
      const int r = vi / (D / 8), c8 = vi % (D / 8);
      const int64_t key = k0 + r;
      pk[i] = u32x4{0, 0, 0, 0};
      pv[i] = u32x4{0, 0, 0, 0};
      if (key < s) {
        pk[i] = *reinterpret_cast<const u32x4*>(K + key * a.kv_row + 8 * c8);
        pv[i] = *reinterpret_cast<const u32x4*>(V + key * a.kv_row + 8 * c8);
      }
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KVEC; ++i) {
      const int vi = tid + i * kWaves * 64;
      const int r = vi / (D / 8), c8 = vi % (D / 8);
      *reinterpret_cast<u32x4*>(&sK[buf][r * KSTR + 8 * c8]) = pk[i];
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::KVEC; ++i) {
      const int vi = tid + i * kWaves * 64;
      const int r = vi / (D / 8), c8 = vi % (D / 8);
      *reinterpret_cast<u32x4*>(&sV[buf][r * VSTR + 8 * c8]) = pv[i];
    }
  };
  // S^T of one tile: s_out[kb][rb][j] = q(row[rb]) . k(k0 + 32kb + 8(j/4) + 4hf + j%4)
  auto qk = [&](int kbuf, f32x16 (&s_out)[KB][RB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      bf16x8 kf[DT];
#pragma unroll
      for (int t = 0; t < DT; ++t)
        kf[t] = *reinterpret_cast<const bf16x8*>(&sK[kbuf][(kb * 32 + l32) * KSTR + 16 * t + 8 * hf]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) s_out[kb][rb] = f32x16{};
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s_out[kb][rb] = mfma32x32x16(kf[t], qf[rb][t], s_out[kb][rb]);
    }
  };
  // the tile needs no mask for any row of this wave
  auto tile_full = [&](int64_t k0) {
    return wave_has_rows && (k0 + BN <= s) && (!a.causal || k0 + BN - 1 <= wr0) && k0 + BN > wkbeg &&
           k0 < wkend && (a.cu == nullptr || (k0 >= w_lo_last && k0 + BN <= w_hi_first));
  };

  f32x16 oacc[RB][DB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x16{};
  }

  const int ntiles = kbeg < kend ? (int)((kend - kbeg + BN - 1) / BN) : 0;
  const int gi = lane >> 4, li = lane & 15;
  f32x16 sc[KB][RB];  // S^T of the current tile, masked
  float tmax[RB];     // its row max (log2 units)
  auto mask_and_max = [&](int64_t k0) {
    if (!tile_full(k0)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int64_t key = k0 + 32 * kb + 8 * (jj / 4) + 4 * hf + (jj % 4);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            if (key < lo[rb] || key >= hi[rb]) sc[kb][rb][jj] = -INFINITY;
        }
    }
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = sc[0][rb][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) mx = fmaxf(mx, sc[kb][rb][jj]);
      tmax[rb] = half_swap_max(mx) * c;
      grow = grow || (tmax[rb] > m[rb] + kTau);
    }
    return __ballot(grow) != 0;
  };

  // Pipeline: in iteration j the VALU turns S(j) into P(j) while the matrix cores compute
  // S(j+1) from K(j+1); then O^T += V(j)^T P(j).
  int j = 0;
  if (ntiles > 0) {
    load_tile(kbeg);
    store_k(0);
    store_v(0);
    __syncthreads();
    if (ntiles > 1) load_tile(kbeg + BN);
    qk(0, sc);
    mask_and_max(kbeg);
  }
  // Outer loop: the (rare) rescale of O when a row max grew by more than kTau. The inner
  // loop never writes O outside an MFMA, which keeps the accumulator in AGPRs.
  while (j < ntiles) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // wave-uniform branch: an MFMA must never run under a partial exec mask
      const bool need = tmax[rb] > m[rb] + kTau;
      if (__ballot(need) == 0) continue;
      const float mnew = need ? tmax[rb] : m[rb];
      const float alpha = need ? fast_exp2(m[rb] - mnew) : 1.f;  // m = -inf on the first visible tile -> 0
      m[rb] = mnew;
      l[rb] *= alpha;
      // Pass the scaled accumulator through an MFMA that adds zero, so that every definition
      // of oacc is an MFMA result and it stays in AGPRs across the loop.
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] = mfma32x32x16(bf16x8{}, bf16x8{}, oacc[rb][db] * alpha);
    }
    for (;;) {
      const int64_t k0 = kbeg + (int64_t)j * BN;
      const int vb = j & 1;
      if (j + 1 < ntiles) store_k((j + 1) & 1);
      __syncthreads();
      if (j + 1 < ntiles) store_v((j + 1) & 1);
      if (j + 2 < ntiles) load_tile(k0 + 2 * BN);
      // P(j) on the VALU while the matrix cores compute S(j+1); then O^T += V(j)^T P(j).
      // Raised priority up to the PV products: the other wave on the SIMD fills the gaps
      // with its own PV MFMAs.
      __builtin_amdgcn_s_setprio(1);
      bf16x8 pf[RB][KB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float ms = m[rb] == -INFINITY ? 0.f : m[rb];
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const float pj = fast_exp2(__builtin_fmaf(sc[kb][rb][jj], c, -ms));
            sc[kb][rb][jj] = pj;
            ls += pj;
          }
          pf[rb][kb][0] = to_bf16x8(sc[kb][rb], 0);
          pf[rb][kb][1] = to_bf16x8(sc[kb][rb], 1);
        }
        l[rb] += ls;
      }
      qk((j + 1) & 1, sc);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int kr = 32 * kb + 16 * tt + 4 * hf + (li >> 2);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int col = db * 32 + 16 * (gi & 1) + 4 * (li & 3);
            const i16x4 v0 = lds_read_tr16(&sV[vb][kr * VSTR + col]);
            const i16x4 v1 = lds_read_tr16(&sV[vb][(kr + 8) * VSTR + col]);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma32x32x16(vf, pf[rb][kb][tt], oacc[rb][db]);
          }
        }
      if (++j >= ntiles) break;
      if (mask_and_max(k0 + BN)) break;
    }
  }

  // ---- normalise and store O (bf16) and LSE (natural log)
  uint16_t* O = static_cast<uint16_t*>(a.out) + (int64_t)h * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float lt = half_swap_sum(l[rb]);
    if (row[rb] >= s) continue;
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[rb][db][4 * jj + 0] * inv, oacc[rb][db][4 * jj + 1] * inv);
        w[1] = pack_bf16x2(oacc[rb][db][4 * jj + 2] * inv, oacc[rb][db][4 * jj + 3] * inv);
        *reinterpret_cast<u32x2*>(O + row[rb] * a.q_row + db * 32 + 8 * jj + 4 * hf) = w;
      }
    if (hf == 0) a.lse_out[(int64_t)h * a.lse_row + row[rb]] = (m[rb] + log2f(lt)) * kLn2;
  }
}

template <int D, int RB, int KB, int OCC>
hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t stream) {
  using C = FwdCfg<D, RB, KB>;
  const int64_t nmb = (a.s + C::BM - 1) / C::BM;
  const int64_t blocks = nmb * a.n_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_kernel<D, RB, KB, OCC>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnArgs& a, int d, hipStream_t stream) {
  if (d == 128) return launch_fwd_t<128, ULY_FWD_RB, ULY_FWD_KB, ULY_FWD_OCC>(a, stream);
  return launch_fwd_t<64, 2, 1, 1>(a, stream);
}

}  // namespace uly
