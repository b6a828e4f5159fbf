// fp32 attention forward and backward for one head shard (head_dim 64), one thread per
// query row (forward, dQ) or per key (dK/dV), with K/V or Q/dO tiles staged in LDS and
// read as broadcasts. This is the full-precision path for small problems; the bf16
// kernels are the tuned path. The arithmetic is the same as theirs except that every
// product stays in fp32 and the running max is always exact.
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts", section
// "how Ulysses works", step 4 (dense attention per head shard over every position).
#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

constexpr int kRows = 64;  // threads (rows or keys) per workgroup = one tile of the other side

template <int D>
__global__ __launch_bounds__(kRows) void f32_fwd_kernel(AttnArgs a) {
  __shared__ float sK[kRows][D];
  __shared__ float sV[kRows][D];
  const int64_t s = a.s;
  const int nmb = (int)((s + kRows - 1) / kRows);
  const int h = blockIdx.x % a.n_heads;
  const int mb = nmb - 1 - (int)(blockIdx.x / a.n_heads);
  const int64_t m0 = (int64_t)mb * kRows;
  const int64_t row = m0 + threadIdx.x;
  const int kvh = (h + a.q_off) / a.G - a.kv_off;
  const float* Q = static_cast<const float*>(a.q) + (int64_t)h * D;
  const float* K = static_cast<const float*>(a.k) + (int64_t)kvh * D;
  const float* V = static_cast<const float*>(a.v) + (int64_t)kvh * D;

  int64_t lo = 0, hi = s;
  if (a.cu != nullptr && row < s) {
    const int dk = doc_of(a.cu, a.n_docs, row);
    lo = a.cu[dk];
    hi = a.cu[dk + 1] < s ? a.cu[dk + 1] : s;
  }
  if (a.causal) hi = hi < row + 1 ? hi : row + 1;
  const int64_t last_row = (m0 + kRows < s ? m0 + kRows : s) - 1;
  int64_t kbeg = 0, kend = s;
  if (a.cu != nullptr) {
    kbeg = a.cu[doc_of(a.cu, a.n_docs, m0)];
    kend = a.cu[doc_of(a.cu, a.n_docs, last_row) + 1];
    kend = kend < s ? kend : s;  // document bounds clamped to the sequence
  }
  if (a.causal) kend = kend < last_row + 1 ? kend : last_row + 1;

  float q[D], o[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    q[x] = row < s ? Q[row * a.q_row + x] : 0.f;
    o[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t k0 = kbeg; k0 < kend; k0 += kRows) {
    __syncthreads();
    for (int i = threadIdx.x; i < kRows * D; i += kRows) {
      const int r = i / D, x = i % D;
      const int64_t key = k0 + r;
      sK[r][x] = key < s ? K[key * a.kv_row + x] : 0.f;
      sV[r][x] = key < s ? V[key * a.kv_row + x] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kRows; ++r) {
      const int64_t key = k0 + r;
      if (key < lo || key >= hi) continue;
      float dot = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) dot = __builtin_fmaf(q[x], sK[r][x], dot);
      const float sc = dot * a.scale;
      if (sc > m) {
        const float alpha = expf(m - sc);
        l *= alpha;
#pragma unroll
        for (int x = 0; x < D; ++x) o[x] *= alpha;
        m = sc;
      }
      const float p = expf(sc - m);
      l += p;
#pragma unroll
      for (int x = 0; x < D; ++x) o[x] = __builtin_fmaf(p, sV[r][x], o[x]);
    }
  }
  if (row < s) {
    float* O = static_cast<float*>(a.out) + (int64_t)h * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int x = 0; x < D; ++x) O[row * a.q_row + x] = o[x] * inv;
    a.lse_out[(int64_t)h * a.lse_row + row] = m + logf(l);
  }
}

template <int D>
__global__ __launch_bounds__(kRows) void f32_dq_kernel(AttnArgs a) {
  __shared__ float sK[kRows][D];
  __shared__ float sV[kRows][D];
  const int64_t s = a.s;
  const int nmb = (int)((s + kRows - 1) / kRows);
  const int h = blockIdx.x % a.n_heads;
  const int mb = nmb - 1 - (int)(blockIdx.x / a.n_heads);
  const int64_t m0 = (int64_t)mb * kRows;
  const int64_t row = m0 + threadIdx.x;
  const int kvh = (h + a.q_off) / a.G - a.kv_off;
  const float* Q = static_cast<const float*>(a.q) + (int64_t)h * D;
  const float* dO = static_cast<const float*>(a.dout) + (int64_t)h * D;
  const float* K = static_cast<const float*>(a.k) + (int64_t)kvh * D;
  const float* V = static_cast<const float*>(a.v) + (int64_t)kvh * D;

  int64_t lo = 0, hi = s;
  float lse = 0.f, dl = 0.f;
  if (row < s) {
    if (a.cu != nullptr) {
      const int dk = doc_of(a.cu, a.n_docs, row);
      lo = a.cu[dk];
      hi = a.cu[dk + 1] < s ? a.cu[dk + 1] : s;
    }
    lse = a.lse_in[(int64_t)h * a.lse_row + row];
    dl = a.delta[(int64_t)h * a.lse_row + row];
  } else {
    hi = 0;
  }
  if (a.causal) hi = hi < row + 1 ? hi : row + 1;
  const int64_t last_row = (m0 + kRows < s ? m0 + kRows : s) - 1;
  int64_t kbeg = 0, kend = s;
  if (a.cu != nullptr) {
    kbeg = a.cu[doc_of(a.cu, a.n_docs, m0)];
    kend = a.cu[doc_of(a.cu, a.n_docs, last_row) + 1];
    kend = kend < s ? kend : s;  // document bounds clamped to the sequence
  }
  if (a.causal) kend = kend < last_row + 1 ? kend : last_row + 1;

  float q[D], g[D], dq[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    q[x] = row < s ? Q[row * a.q_row + x] : 0.f;
    g[x] = row < s ? dO[row * a.q_row + x] : 0.f;
    dq[x] = 0.f;
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += kRows) {
    __syncthreads();
    for (int i = threadIdx.x; i < kRows * D; i += kRows) {
      const int r = i / D, x = i % D;
      const int64_t key = k0 + r;
      sK[r][x] = key < s ? K[key * a.kv_row + x] : 0.f;
      sV[r][x] = key < s ? V[key * a.kv_row + x] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < kRows; ++r) {
      const int64_t key = k0 + r;
      if (key < lo || key >= hi) continue;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < D; ++x) {
        dot = __builtin_fmaf(q[x], sK[r][x], dot);
        dp = __builtin_fmaf(g[x], sV[r][x], dp);
      }
      const float p = expf(dot * a.scale - lse);
      const float ds = p * (dp - dl);
#pragma unroll
      for (int x = 0; x < D; ++x) dq[x] = __builtin_fmaf(ds, sK[r][x], dq[x]);
    }
  }
  if (row < s) {
    float* dQ = static_cast<float*>(a.out) + (int64_t)h * D;
#pragma unroll
    for (int x = 0; x < D; ++x) dQ[row * a.q_row + x] = dq[x] * a.scale;
  }
}

template <int D>
__global__ __launch_bounds__(kRows) void f32_dkdv_kernel(AttnArgs a) {
  __shared__ float sQ[kRows][D];
  __shared__ float sG[kRows][D];
  __shared__ float sL[kRows], sD[kRows];
  const int64_t s = a.s;
  const int kvh = blockIdx.x % a.n_kv;
  const int64_t n0 = (int64_t)(blockIdx.x / a.n_kv) * kRows;
  const int64_t key = n0 + threadIdx.x;
  const float* K = static_cast<const float*>(a.k) + (int64_t)kvh * D;
  const float* V = static_cast<const float*>(a.v) + (int64_t)kvh * D;

  int64_t rlo = 0, rhi = s;
  if (a.cu != nullptr && key < s) {
    const int dk = doc_of(a.cu, a.n_docs, key);
    rlo = a.cu[dk];
    rhi = a.cu[dk + 1] < s ? a.cu[dk + 1] : s;
  }
  if (a.causal) rlo = key;
  if (key >= s) rhi = rlo;
  const int64_t last_key = (n0 + kRows < s ? n0 + kRows : s) - 1;
  int64_t qbeg = a.causal ? n0 : 0, qend = s;
  if (a.cu != nullptr) {
    qend = a.cu[doc_of(a.cu, a.n_docs, last_key) + 1];
    qend = qend < s ? qend : s;  // document bounds clamped to the sequence
    if (!a.causal) qbeg = a.cu[doc_of(a.cu, a.n_docs, n0)];
  }

  float k[D], v[D], dk[D], dv[D];
#pragma unroll
  for (int x = 0; x < D; ++x) {
    k[x] = key < s ? K[key * a.kv_row + x] : 0.f;
    v[x] = key < s ? V[key * a.kv_row + x] : 0.f;
    dk[x] = 0.f;
    dv[x] = 0.f;
  }
  const KvHeads kh = kv_heads_of(a, kvh);  // the launch's q heads reading this kv head
  for (int hq = kh.j0; hq < kh.j1; ++hq) {
    const float* Q = static_cast<const float*>(a.q) + (int64_t)hq * D;
    const float* dO = static_cast<const float*>(a.dout) + (int64_t)hq * D;
    for (int64_t q0 = qbeg; q0 < qend; q0 += kRows) {
      __syncthreads();
      for (int i = threadIdx.x; i < kRows * D; i += kRows) {
        const int r = i / D, x = i % D;
        const int64_t qr = q0 + r;
        sQ[r][x] = qr < s ? Q[qr * a.q_row + x] : 0.f;
        sG[r][x] = qr < s ? dO[qr * a.q_row + x] : 0.f;
      }
      {
        const int64_t qr = q0 + threadIdx.x;
        sL[threadIdx.x] = qr < s ? a.lse_in[(int64_t)hq * a.lse_row + qr] : 0.f;
        sD[threadIdx.x] = qr < s ? a.delta[(int64_t)hq * a.lse_row + qr] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < kRows; ++r) {
        const int64_t qr = q0 + r;
        if (qr < rlo || qr >= rhi) continue;
        float dot = 0.f, dp = 0.f;
#pragma unroll
        for (int x = 0; x < D; ++x) {
          dot = __builtin_fmaf(sQ[r][x], k[x], dot);
          dp = __builtin_fmaf(sG[r][x], v[x], dp);
        }
        const float p = expf(dot * a.scale - sL[r]);
        const float ds = p * (dp - sD[r]);
#pragma unroll
        for (int x = 0; x < D; ++x) {
          dv[x] = __builtin_fmaf(p, sG[r][x], dv[x]);
          dk[x] = __builtin_fmaf(ds, sQ[r][x], dk[x]);
        }
      }
    }
  }
  if (key < s) {
    const int64_t off = (int64_t)kvh * D + key * a.dkv_row;
    // headwise-chunked backward: sums carried across launches in fp32, scaled once at the end
    const bool carry_in = a.acc_k != nullptr && !kh.first;
    const bool carry_out = a.acc_k != nullptr && !kh.last;
    if (carry_in) {
#pragma unroll
      for (int x = 0; x < D; ++x) {
        dk[x] += a.acc_k[off + x];
        dv[x] += a.acc_v[off + x];
      }
    }
    if (carry_out) {
#pragma unroll
      for (int x = 0; x < D; ++x) {
        a.acc_k[off + x] = dk[x];
        a.acc_v[off + x] = dv[x];
      }
    } else {
      float* dK = static_cast<float*>(a.out_k) + off;
      float* dV = static_cast<float*>(a.out_v) + off;
#pragma unroll
      for (int x = 0; x < D; ++x) {
        dK[x] = dk[x] * a.scale;
        dV[x] = dv[x];
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnArgs& a, int d, hipStream_t stream) {
  (void)d;
  const int64_t blocks = (a.s + kRows - 1) / kRows * a.n_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_fwd_kernel<64>, dim3((unsigned)blocks), dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_dq_f32(const AttnArgs& a, int d, hipStream_t stream) {
  (void)d;
  const int64_t blocks = (a.s + kRows - 1) / kRows * a.n_heads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_dq_kernel<64>, dim3((unsigned)blocks), dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_dkdv_f32(const AttnArgs& a, int d, hipStream_t stream) {
  (void)d;
  const int64_t blocks = (a.s + kRows - 1) / kRows * a.n_kv;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(f32_dkdv_kernel<64>, dim3((unsigned)blocks), dim3(kRows), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uly
