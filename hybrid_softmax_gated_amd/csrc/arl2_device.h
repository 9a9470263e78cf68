// Device helpers shared by the libarl2 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace arl2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kL2Eps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;

// D(32x32) += A(32x16) * B(16x32) on the matrix cores, bf16 operands, fp32
// accumulation. Lane l supplies A[row = l%32][k = 8*(l/32) .. +7] and
// B[k = 8*(l/32) .. +7][col = l%32]; the accumulator register i of lane l
// holds D[row = 8*(i/4) + 4*(l/32) + i%4][col = l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 operands, fp32 accumulation. Lane l
// supplies A[row = l%16][k = 8*(l/16) .. +7] and B[k = 8*(l/16) .. +7]
// [col = l%16]; accumulator register i of lane l holds
// D[row = 4*(l/16) + i][col = l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Accumulator rows come in the order 8*(i/4) + 4*(l/32) + i%4; an operand's
// k index runs 8*(l/32) + j. Within a group of 16, row r of an accumulator
// therefore lines up with operand position swap_bits23(r): registers
// 8*g2 .. 8*g2+7 of an accumulator can be fed to the next MFMA as its k
// operand unchanged, provided the other operand stores its k dimension in
// this permuted order. The map is an involution.
__device__ __host__ __forceinline__ constexpr int swap_bits23(int p) {
  return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}

// True if the predicate holds on any lane of the wavefront.
__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lane l and x of lane l ^ 32 (the other half of the wavefront), on
// every lane, with one VALU lane swap (gfx950 v_permlane32_swap on two
// copies of x) instead of a cross-lane read through the LDS unit, which
// would queue behind the tile reads.
__device__ __forceinline__ void halves_pair(float x, float &a, float &b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
// max and sum of x over lanes l and l ^ 32 (the same value on both; a sum
// of two terms does not depend on their order).
__device__ __forceinline__ float halves_max(float x) {
  float a, b;
  halves_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a, b;
  halves_pair(x, a, b);
  return a + b;
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// LDS tile of 16-bit elements with 256-byte rows (128 bf16), stored as 16
// units of 16 bytes per row; unit u of row r sits at position u ^ tile_swz(r)
// so that both access patterns below are free of bank conflicts:
//  * 16 lanes reading the same unit of 16 consecutive rows (b128 reads);
//  * transpose reads: 4 consecutive rows x 2 adjacent units per 16 lanes.
__device__ __host__ __forceinline__ constexpr int tile_swz(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
__device__ __forceinline__ int tile_off(int row, int unit) {
  return row * 256 + ((unit ^ tile_swz(row & 15)) << 4);
}

// Transposed LDS read (gfx950): within each group of 16 lanes, lane i
// receives element i%4 of the 8-byte words addressed by lanes i/4, 4+i/4,
// 8+i/4 and 12+i/4 of its group. If lane j of a group addresses row
// r0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major 16-bit matrix, lane i
// receives rows r0 .. r0+3 of column c0 + i.
__device__ __forceinline__ s16x4 lds_read_tr16(const void *lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(lds_byte_addr));
}

// MFMA operand read transposed from a swizzled row-major 128-column bf16
// tile (tile_off): lane l gets column 32bb + l%32 of the tile, rows k0 ..
// k0+3 in elements 0..3 and rows k1 .. k1+3 in elements 4..7 (k0 and k1
// may differ between the wave halves). A and B operands share this
// register layout, so the result serves as either.
__device__ __forceinline__ bf16x8 tile_col_operand(const char *tile, int k0, int k1, int lane,
                                                   int bb) {
  const int gi = lane & 15, g = lane >> 4;
  const int col = 32 * bb + 16 * (g & 1) + 4 * (gi & 3);
  const s16x4 lo = lds_read_tr16(tile + tile_off(k0 + (gi >> 2), col >> 3) + 2 * (col & 7));
  const s16x4 hi = lds_read_tr16(tile + tile_off(k1 + (gi >> 2), col >> 3) + 2 * (col & 7));
  return __builtin_bit_cast(bf16x8, (short __attribute__((ext_vector_type(8)))){
                                        lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

// Direct global -> LDS copy of 16 bytes per lane: lane i's 16 bytes land at
// lds_base + 16 * i (lds_base must be uniform across the wavefront).
__device__ __forceinline__ void global_to_lds16(const void *gsrc, void *lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t *)lds_base, 16, 0, 0);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base` (raw, no stride): loads at
// offsets past the end return zeros instead of touching memory. Both
// arguments must be the same on every lane; they are read from the first
// active lane so the descriptor lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, n, 0x00020000);
}
__device__ __forceinline__ bf16x8 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// Buffer -> LDS copy of 16 bytes per lane: lane i's bytes land at
// lds_base + 16 * i (lds_base uniform across the wavefront); dwords past the
// resource's end are written as zeros.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void *lds_base, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 16, voff, 0, 0, 0);
}

// Waits until at most N vector-memory loads of this wavefront are in flight
// (they complete in issue order), then meets the workgroup barrier. Unlike
// __syncthreads, this adds no wait for the loads issued after those N.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Split an fp32 value into bf16 high and low parts, x ~= hi + lo (the
// three-product bf16 scheme of Henry, Tang and Heinecke, ARITH 2019).
__device__ __forceinline__ void split_bf16(float x, bf16 &hi, bf16 &lo) {
  hi = (bf16)x;
  lo = (bf16)(x - (float)hi);
}

}  // namespace arl2
