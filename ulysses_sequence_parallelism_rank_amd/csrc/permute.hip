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

// gather: out[(p*s_l + t)*run + w] = shard_p[t*row_in + h_off + w]   (units of 16 B; one per thread)
__global__ __launch_bounds__(kPermThreads) void pack_kernel(ShardPtrs src, u32x4* __restrict__ out,
                                                            uint32_t s_l, uint32_t run, uint32_t row_in,
                                                            uint32_t h_off, uint32_t total) {
  const uint32_t c = blockIdx.x * kPermThreads + threadIdx.x;
  if (c >= total) return;
  const uint32_t row = c / run, w = c - row * run;
  const uint32_t p = row / s_l, t = row - p * s_l;
  const u32x4* s = reinterpret_cast<const u32x4*>(src.p[p]);
  __builtin_nontemporal_store(__builtin_nontemporal_load(s + (size_t)t * row_in + h_off + w), out + c);
}

// scatter: shard_p[t*row_in + h_off + w] = in[(p*s_l + t)*run + w]
__global__ __launch_bounds__(kPermThreads) void unpack_kernel(const u32x4* __restrict__ in, ShardPtrs dst,
                                                              uint32_t s_l, uint32_t run, uint32_t row_in,
                                                              uint32_t h_off, uint32_t total) {
  const uint32_t c = blockIdx.x * kPermThreads + threadIdx.x;
  if (c >= total) return;
  const uint32_t row = c / run, w = c - row * run;
  const uint32_t p = row / s_l, t = row - p * s_l;
  u32x4* d = reinterpret_cast<u32x4*>(const_cast<void*>(dst.p[p]));
  __builtin_nontemporal_store(__builtin_nontemporal_load(in + c), d + (size_t)t * row_in + h_off + w);
}

// Host launchers. Sizes are in bytes; the caller has checked alignment, that every
// size is a multiple of 16 and that the 16-byte chunk count fits in 32 bits.
hipError_t launch_pack(const ShardPtrs& src, void* out, int P, int64_t s_l, int64_t row_bytes,
                       int64_t off_bytes, int64_t run_bytes, hipStream_t stream) {
  const uint64_t total = (uint64_t)P * s_l * (run_bytes / 16);
  if (total == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)((total + kPermThreads - 1) / kPermThreads);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, src,
                     reinterpret_cast<u32x4*>(out), (uint32_t)s_l, (uint32_t)(run_bytes / 16),
                     (uint32_t)(row_bytes / 16), (uint32_t)(off_bytes / 16), (uint32_t)total);
  return hipGetLastError();
}

hipError_t launch_unpack(const void* in, const ShardPtrs& dst, int P, int64_t s_l, int64_t row_bytes,
                         int64_t off_bytes, int64_t run_bytes, hipStream_t stream) {
  const uint64_t total = (uint64_t)P * s_l * (run_bytes / 16);
  if (total == 0) return hipSuccess;
  const uint32_t blocks = (uint32_t)((total + kPermThreads - 1) / kPermThreads);
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks), dim3(kPermThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(in), dst, (uint32_t)s_l, (uint32_t)(run_bytes / 16),
                     (uint32_t)(row_bytes / 16), (uint32_t)(off_bytes / 16), (uint32_t)total);
  return hipGetLastError();
}

}  // namespace uly
