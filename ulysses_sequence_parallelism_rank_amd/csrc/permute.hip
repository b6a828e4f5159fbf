// Local permutes on either side of Ulysses' all-to-alls (gfx950).
//
// Pages: "Ulysses Sequence Parallelism: Training with Million-Token Contexts", section
// "how Ulysses works", steps 1, 3 and 5: P sequence shards [s_l, H, d] (a token chunk
// with every head) become one head shard [s, H/P, d] (every token, a head subset) and back.
//
// Both directions are pure copies of contiguous runs: for each (p, t) one run of
// nh*d elements (nh*d*e bytes, a multiple of 16) moves between shard p row t at head
// offset h0 and head-shard row p*s_l + t. The kernels move 16-byte vectors with
// nontemporal loads and stores (the data is touched once; caching it only evicts the
// attention's working set). One vector per thread and many small workgroups measured
// fastest on gfx950: at the 64K share, 5.5 TB/s for a Q-shaped pack (2 KiB runs) against
// 4.5 TB/s with four vectors per thread and cached stores; more vectors per thread was
// slower still (8 per thread: about half the rate). HBM-bound: algorithmic traffic is
// 2 * P*s_l*nh*d*e bytes.
#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

constexpr int kPermThreads = 256;

// One tensor of a (grouped) permute launch, in 16-byte units: the P shards with rows of
// row_in units, the head-shard buffer `flat` with runs of `run` units taken from offset
// h_off of every shard row, `total` = P*s_l*run units, and the first workgroup of the launch
// that works on it.
struct PermSegK {
  ShardPtrs sh;
  u32x4* flat;
  uint32_t run, row_in, h_off, total, block0;
};
// Up to kPermGroupMax tensors moved by one launch (one ramp-up and drain instead of several).
static_assert(kPermGroupMax == 3, "pack_kernel / unpack_kernel select among three tensors");
struct PermGroupK {
  PermSegK seg[kPermGroupMax];
  uint32_t s_l;
  int n;
};

// gather: flat[(p*s_l + t)*run + w] = shard_p[t*row_in + h_off + w]   (one unit per thread)
__device__ __forceinline__ void pack_unit(const PermSegK& g, uint32_t s_l, uint32_t c) {
  if (c >= g.total) return;
  const uint32_t row = c / g.run, w = c - row * g.run;
  const uint32_t p = row / s_l, t = row - p * s_l;
  const u32x4* s = reinterpret_cast<const u32x4*>(g.sh.p[p]);
  __builtin_nontemporal_store(__builtin_nontemporal_load(s + (size_t)t * g.row_in + g.h_off + w), g.flat + c);
}
// scatter: shard_p[t*row_in + h_off + w] = flat[(p*s_l + t)*run + w]
__device__ __forceinline__ void unpack_unit(const PermSegK& g, uint32_t s_l, uint32_t c) {
  if (c >= g.total) return;
  const uint32_t row = c / g.run, w = c - row * g.run;
  const uint32_t p = row / s_l, t = row - p * s_l;
  u32x4* d = reinterpret_cast<u32x4*>(const_cast<void*>(g.sh.p[p]));
  __builtin_nontemporal_store(__builtin_nontemporal_load(g.flat + c), d + (size_t)t * g.row_in + g.h_off + w);
}

// The workgroup's tensor is found by comparing its index with the tensors' first workgroups
// (wave-uniform branches; each branch reads its tensor's fields at a constant index).
__global__ __launch_bounds__(kPermThreads) void pack_kernel(PermGroupK g) {
  const uint32_t b = blockIdx.x;
  if (g.n > 2 && b >= g.seg[2].block0)
    pack_unit(g.seg[2], g.s_l, (b - g.seg[2].block0) * kPermThreads + threadIdx.x);
  else if (g.n > 1 && b >= g.seg[1].block0)
    pack_unit(g.seg[1], g.s_l, (b - g.seg[1].block0) * kPermThreads + threadIdx.x);
  else
    pack_unit(g.seg[0], g.s_l, b * kPermThreads + threadIdx.x);
}

__global__ __launch_bounds__(kPermThreads) void unpack_kernel(PermGroupK g) {
  const uint32_t b = blockIdx.x;
  if (g.n > 2 && b >= g.seg[2].block0)
    unpack_unit(g.seg[2], g.s_l, (b - g.seg[2].block0) * kPermThreads + threadIdx.x);
  else if (g.n > 1 && b >= g.seg[1].block0)
    unpack_unit(g.seg[1], g.s_l, (b - g.seg[1].block0) * kPermThreads + threadIdx.x);
  else
    unpack_unit(g.seg[0], g.s_l, b * kPermThreads + threadIdx.x);
}

// ---------------------------------------------------------------------------------------
// The exchange as a real all-to-all performs it (pages: "how Ulysses works", steps 1, 3 and 5;
// the comparison table's num_heads >= sp_size): every source rank permutes its sequence shard
// into P contiguous per-destination blocks, the collective swaps blocks, and every destination
// rank permutes what it received back into its sequence shard. With fewer heads than ranks
// (P a multiple of H) each head goes to the R = P / H ranks r with r / R == head, and on the way
// back the R copies of a head's gradient are summed in fp32 in rank order (from +0, so the sign
// of a zero sum is +), then rounded once.
struct SendK {
  const u32x4* shard;  // [s_l, H, d]
  u32x4* out;          // [P, s_l, H_l, d]
  uint32_t s_l, run, row_in, head_units, total, per_rank_heads, rep;
};
// out[(r*s_l + t)*run + w] = shard[t*row_in + first(r)*head_units + w]
__global__ __launch_bounds__(kPermThreads) void send_pack_kernel(SendK g) {
  const uint32_t c = blockIdx.x * kPermThreads + threadIdx.x;
  if (c >= g.total) return;
  const uint32_t row = c / g.run, w = c - row * g.run;
  const uint32_t r = row / g.s_l, t = row - r * g.s_l;
  const uint32_t first = g.rep > 1 ? r / g.rep : r * g.per_rank_heads;
  __builtin_nontemporal_store(
      __builtin_nontemporal_load(g.shard + (size_t)t * g.row_in + (size_t)first * g.head_units + w), g.out + c);
}

struct RecvK {
  const u32x4* in;  // [P, s_l, H_l, d]
  u32x4* shard;     // [s_l, H, d]
  uint32_t s_l, run, row_out, head_units, total, per_rank_heads, rep;
  int bf16;
};
// shard[t*row_out + h*head_units + w] = sum over the holders r of head h of
// in[(r*s_l + t)*run + (h - first(r))*head_units + w]
__global__ __launch_bounds__(kPermThreads) void recv_unpack_kernel(RecvK g) {
  const uint32_t c = blockIdx.x * kPermThreads + threadIdx.x;
  if (c >= g.total) return;
  const uint32_t t = c / g.row_out, rem = c - t * g.row_out;
  const uint32_t h = rem / g.head_units, w = rem - h * g.head_units;
  if (g.rep <= 1) {  // one holder: the bits move unchanged
    const uint32_t r = h / g.per_rank_heads, j = h - r * g.per_rank_heads;
    __builtin_nontemporal_store(
        __builtin_nontemporal_load(g.in + ((size_t)r * g.s_l + t) * g.run + (size_t)j * g.head_units + w),
        g.shard + c);
    return;
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (uint32_t k = 0; k < g.rep; ++k) {
    const uint32_t r = h * g.rep + k;
    const u32x4 x = __builtin_nontemporal_load(g.in + ((size_t)r * g.s_l + t) * g.run + w);
    if (g.bf16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t xi = x[i];
        acc[2 * i] += bf16_lo(xi);
        acc[2 * i + 1] += bf16_hi(xi);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t xi = x[i];
        acc[i] += __builtin_bit_cast(float, xi);
      }
    }
  }
  u32x4 o;
  if (g.bf16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_bit_cast(uint32_t, acc[i]);
  }
  __builtin_nontemporal_store(o, g.shard + c);
}

namespace {

// Sizes are in bytes; the caller has checked alignment, that every size is a multiple of 16,
// that each tensor's 16-byte unit count fits in 32 bits and that 1 <= n <= kPermGroupMax.
hipError_t launch_group(bool pack, const PermSeg* segs, int n, int64_t s_l, hipStream_t stream) {
  PermGroupK g{};
  g.s_l = (uint32_t)s_l;
  g.n = n;
  uint64_t blocks = 0;
  for (int i = 0; i < n; ++i) {
    PermSegK& k = g.seg[i];
    k.sh = segs[i].sh;
    k.flat = reinterpret_cast<u32x4*>(segs[i].flat);
    k.run = (uint32_t)(segs[i].run_bytes / 16);
    k.row_in = (uint32_t)(segs[i].row_bytes / 16);
    k.h_off = (uint32_t)(segs[i].off_bytes / 16);
    k.total = (uint32_t)((uint64_t)segs[i].P * s_l * k.run);
    k.block0 = (uint32_t)blocks;
    blocks += (k.total + kPermThreads - 1) / kPermThreads;
  }
  if (blocks == 0) return hipSuccess;
  if (blocks > 0xFFFFFFFFull) return hipErrorInvalidValue;
  if (pack)
    hipLaunchKernelGGL(pack_kernel, dim3((uint32_t)blocks), dim3(kPermThreads), 0, stream, g);
  else
    hipLaunchKernelGGL(unpack_kernel, dim3((uint32_t)blocks), dim3(kPermThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_group(const PermSeg* segs, int n, int64_t s_l, hipStream_t stream) {
  return launch_group(true, segs, n, s_l, stream);
}

hipError_t launch_unpack_group(const PermSeg* segs, int n, int64_t s_l, hipStream_t stream) {
  return launch_group(false, segs, n, s_l, stream);
}

// Sizes in bytes, checked by the caller: P % H == 0 or H % P == 0, head_bytes a multiple of 16,
// the 16-byte unit counts within 32 bits.
hipError_t launch_send_pack(const void* shard, void* out, int P, int64_t s_l, int H, int64_t head_bytes,
                            hipStream_t stream) {
  SendK g{};
  const int rep = H < P ? P / H : 1, nh = H < P ? 1 : H / P;
  g.shard = static_cast<const u32x4*>(shard);
  g.out = static_cast<u32x4*>(out);
  g.s_l = (uint32_t)s_l;
  g.head_units = (uint32_t)(head_bytes / 16);
  g.run = (uint32_t)(nh * g.head_units);
  g.row_in = (uint32_t)(H * g.head_units);
  g.total = (uint32_t)((uint64_t)P * s_l * g.run);
  g.per_rank_heads = (uint32_t)nh;
  g.rep = (uint32_t)rep;
  const uint32_t blocks = (g.total + kPermThreads - 1) / kPermThreads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(send_pack_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_recv_unpack(const void* in, void* shard, int P, int64_t s_l, int H, int64_t head_bytes, int bf16,
                              hipStream_t stream) {
  RecvK g{};
  const int rep = H < P ? P / H : 1, nh = H < P ? 1 : H / P;
  g.in = static_cast<const u32x4*>(in);
  g.shard = static_cast<u32x4*>(shard);
  g.s_l = (uint32_t)s_l;
  g.head_units = (uint32_t)(head_bytes / 16);
  g.run = (uint32_t)(nh * g.head_units);
  g.row_out = (uint32_t)(H * g.head_units);
  g.total = (uint32_t)((uint64_t)s_l * g.row_out);
  g.per_rank_heads = (uint32_t)nh;
  g.rep = (uint32_t)rep;
  g.bf16 = bf16;
  const uint32_t blocks = (g.total + kPermThreads - 1) / kPermThreads;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(recv_unpack_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_pack(const ShardPtrs& src, void* out, int P, int64_t s_l, int64_t row_bytes,
                       int64_t off_bytes, int64_t run_bytes, hipStream_t stream) {
  const PermSeg seg{src, out, P, row_bytes, off_bytes, run_bytes};
  return launch_group(true, &seg, 1, s_l, stream);
}

hipError_t launch_unpack(const void* in, const ShardPtrs& dst, int P, int64_t s_l, int64_t row_bytes,
                         int64_t off_bytes, int64_t run_bytes, hipStream_t stream) {
  const PermSeg seg{dst, const_cast<void*>(in), P, row_bytes, off_bytes, run_bytes};
  return launch_group(false, &seg, 1, s_l, stream);
}

}  // namespace uly
