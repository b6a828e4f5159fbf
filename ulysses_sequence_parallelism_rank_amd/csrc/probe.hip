// Measurement helper: the practical bf16 MFMA ceiling and the sustained shader clock on
// this GPU, the secondary denominators beside the published peaks.
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

}  // namespace

hipError_t launch_mfma_probe(int iters, int blocks, float* sink, unsigned long long* clocks, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, sink, clocks);
  return hipGetLastError();
}

}  // namespace uly
