// Shared device helpers for the gfx950 kernels (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum DType { kBF16 = 0, kF32 = 1 };

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair, round to nearest even: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v));
}

// Value of the same register in lane (lane ^ 32): v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second, so {r[0], r[1]} = {own, partner}.
__device__ __forceinline__ float partner32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on XCD w % 8).
// Remap so that each XCD walks one contiguous range of logical tiles: neighbouring query
// blocks of a head then share that XCD's L2 for the key/value blocks they have in common.
__device__ __forceinline__ int xcd_remap(int w, int n) {
  const int per = n >> 3;
  if (w >= (per << 3)) return w;
  return (w & 7) * per + (w >> 3);
}

// Row order of the block-sparse attention kernels over their rows (b, h, block). XCD x takes
// chunks x, x + 8, x + 16, ... of kWorkChunk consecutive rows: each XCD works on neighbouring
// blocks, which keep mostly the same key (or query) blocks, and on a share of every head, so that
// heads of very different densities spread evenly over the XCDs (one contiguous range per XCD,
// as xcd_remap gives, hands whole heads to single XCDs). Rows outside whole chunks are split into
// one contiguous piece per XCD.
constexpr int kWorkChunk = 128;
__device__ __forceinline__ int xcd_chunk_row(int w, int n) {
  const int per = n >> 3;
  if (w >= (per << 3)) return w;
  const int x = w & 7, l = w >> 3;
  const int full = per / kWorkChunk;
  const int c = l / kWorkChunk, off = l - c * kWorkChunk;
  if (c < full) return (c * 8 + x) * kWorkChunk + off;
  return full * 8 * kWorkChunk + x * (per - full * kWorkChunk) + off;
}

}  // namespace sa
