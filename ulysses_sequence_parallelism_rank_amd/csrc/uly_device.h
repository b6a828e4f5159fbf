// Device-side helpers shared by the gfx950 kernels of the Ulysses attention share.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uly {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Operand lanes: lane l supplies row (A) / column (B) l%32 and the 8 contraction
// elements 8*(l/32) .. 8*(l/32)+7. Result lane l holds column l%32, rows
// 8*(j/4) + 4*(l/32) + j%4 for j = 0..15 (checked on gfx950 by the layout test).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// v_permlane32_swap on two copies of x: r[0] holds x of lanes 0..31 in both halves and r[1]
// x of lanes 32..63 in both halves, so max(r[0], r[1]) / r[0] + r[1] combine lanes l and l^32.
// (Elements are copied to scalars before any bit cast: clang's __builtin_bit_cast of a vector
// element reads element 0.)
__device__ __forceinline__ void half_swap(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                  false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float half_swap_max(float x) {
  float a, b;
  half_swap(x, a, b);
  return __builtin_elementwise_maximum(a, b);  // NaN-propagating: no quieting of a and b first
}
__device__ __forceinline__ float half_swap_sum(float x) {
  float a, b;
  half_swap(x, a, b);
  return a + b;
}

// the two bf16 halves of a packed pair (low half = first element) as fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// 16 fp32 accumulator values j = 8t..8t+7 -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& a, int t) {
  u32x4 r;
  r[0] = pack_bf16x2(a[8 * t + 0], a[8 * t + 1]);
  r[1] = pack_bf16x2(a[8 * t + 2], a[8 * t + 3]);
  r[2] = pack_bf16x2(a[8 * t + 4], a[8 * t + 5]);
  r[3] = pack_bf16x2(a[8 * t + 6], a[8 * t + 7]);
  return __builtin_bit_cast(bf16x8, r);
}

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane i
// receives element e (e = 0..3) from the 8 bytes addressed by lane 4*e + i/4 of the
// group, taking that lane's element i%4. If lane 4*r + c of the group points at row r,
// columns 4c..4c+3 of a row-major [rows][cols] bf16 tile, lane i receives column i of
// those 4 rows (checked on gfx950 by the layout test).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(lds_ptr));
}

// Bank-conflict-free layout for row-major bf16 tiles of D columns in LDS: the 16-byte
// chunks of row r are XOR-permuted by swz_chunk(r). Both access patterns of the MFMA
// operands hit 64 distinct banks: 16-byte reads of one column chunk by 16 consecutive rows
// (ds_read_b128), and the transposing read of 4 consecutive rows x 4 chunks by 32 lanes
// (ds_read_b64_tr_b16).
template <int D>
__device__ __forceinline__ int swz_chunk(int row) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
// element offset of (row, col) in a swizzled [rows][D] tile; col is a multiple of 4
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + ((((col >> 3) ^ swz_chunk<D>(row)) << 3) | (col & 7));
}

// Copy rows [r0, r0 + ROWS) of a row-major bf16 matrix (row stride `stride` elements, D
// columns) into a swizzled LDS tile (tile_off layout) with LDS DMA (global_load_lds_dwordx4):
// no registers hold the data on its way. Each wave instruction fills 64 consecutive 16-byte
// slots; a lane fetches the logical chunk that the swizzle maps to its slot. Rows at or past
// `nrows` are read from row nrows - 1 (finite values for rows the caller masks). The data is
// visible to the workgroup after the next __syncthreads (its fence waits for the DMA).
template <int D, int ROWS, int NTHREADS>
__device__ __forceinline__ void dma_tile(const uint16_t* src, int64_t stride, int64_t r0, int64_t nrows,
                                         uint16_t* lds_tile, int tid) {
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int SLOTS = ROWS * CPR;   // 16-byte slots in the tile
  static_assert(SLOTS % NTHREADS == 0, "tile must be a whole number of wave instructions");
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < SLOTS / NTHREADS; ++i) {
    const int sl0 = (i * (NTHREADS / 64) + wave) * 64;  // first slot of this instruction (wave-uniform)
    const int sl = sl0 + lane;
    const int row = sl / CPR, pc = sl % CPR;
    const int c = pc ^ swz_chunk<D>(row);
    int64_t gr = r0 + row;
    gr = gr < nrows ? gr : nrows - 1;
    __builtin_amdgcn_global_load_lds(src + gr * stride + c * 8, lds_tile + sl0 * 8, 16, 0, 0);
  }
}

// The lane-dependent part of dma_tile's addresses: the byte offset of this lane's 16-byte chunk
// in the tile's first wave instruction (row stride `stride` elements). Instruction i reads the
// rows NTHREADS / (D / 8) * i further on, a multiple of the swizzle's 16-row period, so its
// lanes keep the same chunk order and only a wave-uniform row step is added. Computed once per
// kernel: a tile whose rows all lie inside the matrix then costs scalar address arithmetic only.
template <int D, int NTHREADS>
__device__ __forceinline__ uint32_t dma_lane_offset(int64_t stride, int tid) {
  constexpr int CPR = D / 8;
  static_assert((NTHREADS / CPR) % 16 == 0, "rows per wave instruction must be a multiple of 16");
  const int sl = (tid >> 6) * 64 + (tid & 63);
  const int row = sl / CPR, pc = sl % CPR;
  return (uint32_t)(row * stride + (pc ^ swz_chunk<D>(row)) * 8) * 2u;
}
// dma_tile for a tile whose ROWS rows all lie inside the matrix: `tile` is the wave-uniform
// address of its first row, `off` this lane's dma_lane_offset, `wave` the wave index (uniform).
template <int D, int ROWS, int NTHREADS>
__device__ __forceinline__ void dma_tile_whole(const uint16_t* tile, int64_t stride, uint32_t off, uint16_t* lds_tile,
                                               int wave) {
  constexpr int CPR = D / 8, RPI = NTHREADS / CPR;
  static_assert(ROWS % RPI == 0, "tile must be a whole number of wave instructions");
#pragma unroll
  for (int i = 0; i < ROWS / RPI; ++i) {
    const int sl0 = (i * (NTHREADS / 64) + wave) * 64;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(tile + (int64_t)i * RPI * stride) + off,
                                     lds_tile + sl0 * 8, 16, 0, 0);
  }
}

// The wave index as a wave-uniform value: tid >> 6 is the same on every lane of a wave, but the
// compiler cannot see that, and values derived from it would otherwise live in vector registers
// (branches on them turned into per-lane selects, LDS DMA bases moved to scalars per use).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Wait until this wave's LDS DMA (global_load_lds) has landed: s_waitcnt vmcnt(0), the other
// counters left alone (gfx9 encoding: expcnt 7 in bits 6:4, lgkmcnt 15 in bits 11:8). A
// workgroup barrier does not order another wave's DMA writes before this wave's LDS reads, so
// every wave waits for its own DMA before the barrier that publishes a DMA'd tile.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// q heads [j0, j1) of a launch that read its kv head g (see AttnArgs), and whether the launch
// holds the first (lo >= 0) and the last (lo + G <= n_heads) q head of that kv head's group.
struct KvHeads {
  int j0, j1;
  bool first, last;
};
template <typename Args>
__device__ __forceinline__ KvHeads kv_heads_of(const Args& a, int g) {
  const int lo = (g + a.kv_off) * a.G - a.q_off;
  KvHeads r;
  r.j0 = lo > 0 ? lo : 0;
  r.j1 = lo + a.G < a.n_heads ? lo + a.G : a.n_heads;
  r.first = lo >= 0;
  r.last = lo + a.G <= a.n_heads;
  return r;
}

// First document boundary > i, searched in cu[0..n]; returns index k with cu[k] <= i < cu[k+1].
__device__ __forceinline__ int doc_of(const int32_t* cu, int n, int64_t i) {
  int lo = 0, hi = n;  // invariant: cu[lo] <= i < cu[hi]
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= i) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace uly
