// Measurement helpers: the practical bf16 MFMA ceiling and the sustained shader clock on
// this GPU, the secondary denominators beside the published peaks, and the ceiling of the
// attention kernels' inner-loop instruction mix at a given number of waves per SIMD.
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on four independent
// accumulators (enough to keep the matrix core of its SIMD busy); wave 0 of workgroup 0
// reads the shader clock counter (s_memtime) and the constant 100 MHz counter
// (s_memrealtime) before and after its loop, so their ratio gives the clock under load.
#include "uly_device.h"
#include "uly_internal.h"

namespace uly {

namespace {

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink, unsigned long long* clocks) {
  const int lane = threadIdx.x & 63;
  // small lane-dependent operands (not foldable), sums stay finite for any iteration count
  u32x4 ra, rb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = 0x3C003C00u + (uint32_t)((lane + i) & 7);  // bf16 pairs near 2^-7
    rb[i] = 0x3C003C00u + (uint32_t)((lane * 3 + i) & 7);
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ra), b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c0{}, c1{}, c2{}, c3{};
  const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_readcyclecounter();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32x32x16(a, b, c0);
    c1 = mfma32x32x16(a, b, c1);
    c2 = mfma32x32x16(a, b, c2);
    c3 = mfma32x32x16(a, b, c3);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc += c0[j] + c1[j] + c2[j] + c3[j];
  if (timer) {
    const unsigned long long t1 = __builtin_readcyclecounter();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      clocks[0] = t1 - t0;
      clocks[1] = r1 - r0;
    }
  }
  // a store the compiler cannot drop, taken by no lane in practice
  if (acc == -1.0f) sink[0] = acc;
}

// The attention kernels' inner loop without its data dependences: per round, 16
// v_mfma_f32_32x32x16_bf16 whose first operand is a 1 KiB ds_read_b128 from a 32 KiB LDS tile
// (as the K / V / Q / dO operand reads), each product followed by NV fp32 FMAs and NE
// v_exp_f32 on registers of their own (the softmax's VALU work). At most 128 VGPRs and 32 KiB
// of LDS, so W workgroups of 4 waves per CU run W waves on every SIMD: the rate then shows how
// much of one wave's VALU work the matrix core hides behind the other waves' products.
template <int NV, int NE>
__global__ __launch_bounds__(256, 4) void mix_probe_kernel(int iters, float* sink) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[8192];
  for (int i = threadIdx.x; i < 8192; i += 256) tile[i] = 0x3C003C00u + (uint32_t)(i & 7);  // bf16 near 2^-7
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u32x4 rb;
#pragma unroll
  for (int i = 0; i < 4; ++i) rb[i] = 0x3C003C00u + (uint32_t)((lane * 3 + i) & 7);
  const bf16x8 b = __builtin_bit_cast(bf16x8, rb);
  f32x16 c[4] = {};
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 0.001f * (float)(lane + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      // a lane-contiguous 1 KiB read (no bank conflicts), moving with the round
      const int w = ((wave * 16 + j) * 256 + (it & 15) * 64 + lane * 4) & 8191;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&tile[w]);
      c[j & 3] = mfma32x32x16(a, b, c[j & 3]);
#pragma unroll
      for (int k = 0; k < NV; ++k) v[(j * NV + k) & 15] = __builtin_fmaf(v[(j * NV + k) & 15], 0.999f, 0.0001f);
#pragma unroll
      for (int k = 0; k < NE; ++k) v[(j * NE + k + 7) & 15] = fast_exp2(v[(j * NE + k + 7) & 15] - 1.0f);
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc += c[0][j] + c[1][j] + c[2][j] + c[3][j] + v[j];
  // a store the compiler cannot drop, taken by no lane in practice
  if (acc == -1.0f) sink[0] = acc;
}

}  // namespace

hipError_t launch_mix_probe(int kind, int iters, int blocks, float* sink, hipStream_t stream) {
  switch (kind) {
    case 0: hipLaunchKernelGGL((mix_probe_kernel<0, 0>), dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink); break;
    case 1: hipLaunchKernelGGL((mix_probe_kernel<2, 1>), dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink); break;
    default: hipLaunchKernelGGL((mix_probe_kernel<4, 1>), dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int iters, int blocks, float* sink, unsigned long long* clocks, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink, clocks);
  return hipGetLastError();
}

}  // namespace uly
