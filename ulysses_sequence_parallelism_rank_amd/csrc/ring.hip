// Ring Attention's merge of per-hop partial outputs (gfx950).
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts", sections on
// communication complexity and on Ulysses compared with Ring Attention: a rank keeps its query
// block and attends to each key/value block as it comes round the ring; the partial results
// are combined into attention over the whole sequence. With per-hop (O_i, LSE_i) the combination
// is LSE = log sum_i exp(LSE_i), O = sum_i exp(LSE_i - LSE) O_i, taken here one hop at a time
// into an fp32 running output.
//
// One thread per 8 elements of a (row, head): the 16 (d = 128) or 8 (d = 64) threads of a
// (row, head) lie in one wave, so every lane reads the running LSE before any lane of the
// (row, head) stores the new one. HBM-bound elementwise work.
#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

struct MergeK {
  const uint16_t* part;     // [s_l, H, D] bf16, row stride H*D
  const uint16_t* part_lo;  // its rounding residual (same layout)
  const float* part_lse;    // [H, s_l] natural log
  float* acc;               // [s_l, H, D] fp32 running output
  float* acc_lse;           // [H, s_l]
  uint16_t* out;            // [s_l, H, D] bf16, written by the last hop
  uint16_t* out_lo;         // its residual, or null
  float* out_lse;           // [H, s_l], written by the last hop
  int64_t s_l;
  int H, D;
  int first, last;
};

__global__ __launch_bounds__(256) void ring_merge_kernel(MergeK g) {
  const int per = g.D / 8;  // threads per (row, head)
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = g.s_l * g.H * per;
  if (c >= total) return;
  const int64_t rh = c / per;
  const int part_i = (int)(c - rh * per);
  const int64_t row = rh / g.H;
  const int h = (int)(rh - row * g.H);
  const int64_t e0 = rh * g.D + part_i * 8;  // first element (row, h, 8 part_i)
  const u32x4 pv = *reinterpret_cast<const u32x4*>(g.part + e0);
  const u32x4 pl = *reinterpret_cast<const u32x4*>(g.part_lo + e0);
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = pv[i], b = pl[i];
    x[2 * i] = bf16_lo(a) + bf16_lo(b);
    x[2 * i + 1] = bf16_hi(a) + bf16_hi(b);
  }
  const float lp = g.part_lse[(int64_t)h * g.s_l + row];
  float lse = lp;
  if (!g.first) {
    const float la = g.acc_lse[(int64_t)h * g.s_l + row];
    const float m = fmaxf(la, lp);
    const float wa = __expf(la - m), wp = __expf(lp - m);
    const float tot = wa + wp, inv = 1.f / tot;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(g.acc + e0);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(g.acc + e0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (a0[i] * wa + x[i] * wp) * inv;
      x[4 + i] = (a1[i] * wa + x[4 + i] * wp) * inv;
    }
    lse = m + __logf(tot);
  }
  if (!g.last) {
    *reinterpret_cast<f32x4*>(g.acc + e0) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(g.acc + e0 + 4) = f32x4{x[4], x[5], x[6], x[7]};
    if (part_i == 0) g.acc_lse[(int64_t)h * g.s_l + row] = lse;
    return;
  }
  u32x4 o, r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const uint32_t oi = o[i];
    r[i] = pack_bf16x2(x[2 * i] - bf16_lo(oi), x[2 * i + 1] - bf16_hi(oi));
  }
  *reinterpret_cast<u32x4*>(g.out + e0) = o;
  if (g.out_lo != nullptr) *reinterpret_cast<u32x4*>(g.out_lo + e0) = r;
  if (part_i == 0) g.out_lse[(int64_t)h * g.s_l + row] = lse;
}

}  // namespace

hipError_t launch_ring_merge(const void* part, const void* part_lo, const float* part_lse, float* acc, float* acc_lse,
                             void* out, void* out_lo, float* out_lse, int64_t s_l, int H, int d, int first, int last,
                             hipStream_t stream) {
  MergeK g{};
  g.part = static_cast<const uint16_t*>(part);
  g.part_lo = static_cast<const uint16_t*>(part_lo);
  g.part_lse = part_lse;
  g.acc = acc;
  g.acc_lse = acc_lse;
  g.out = static_cast<uint16_t*>(out);
  g.out_lo = static_cast<uint16_t*>(out_lo);
  g.out_lse = out_lse;
  g.s_l = s_l;
  g.H = H;
  g.D = d;
  g.first = first;
  g.last = last;
  const int64_t total = s_l * H * (d / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace uly
