// LDS tile layout, DMA helpers and operand types shared by the bf16 attention kernels
// (internal; not part of the C ABI).
#pragma once

#include "sa_common.h"

namespace sa {

constexpr int BK = 64;  // keys per key block

// bf16 inputs need no conversion on the way into LDS, so K and V blocks are copied HBM -> LDS by
// global_load_lds_dwordx4 (lane i of an instruction fills bytes 16 i .. 16 i + 15 of a 1 KiB
// stretch) and never occupy VGPRs. Both tiles keep their natural [key][channel] layout:
//  - K fragments (A operand of S^T = K Q^T) are 16-byte ds_read_b128 of one key row;
//  - V^T fragments (A operand of O^T += V^T P^T) come from ds_read_b64_tr_b16. Within each group
//    of 16 lanes, lane i receives element (i % 4) of the 8 bytes addressed by lanes
//    4k + i / 4, k = 0..3. When lane s of the group addresses key key0 + s / 4, channels
//    base + 4 (s % 4) .. + 3, lane i therefore gets channel base + i of keys key0 .. key0 + 3:
//    four keys of one channel, which is exactly a run of the PV MFMA's K dimension.
// 16-byte chunks are XOR-swizzled per row (kv_swz) so that the 16 rows of a K read and the
// 8 rows x 4 chunks of a V^T read both spread evenly over the LDS banks.

typedef __attribute__((address_space(3))) char lchar;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);  // 16 chunks per 256-byte row
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);              // 8 chunks per 128-byte row
}

// Launch geometry of the forward kernel: one workgroup per (b, h, query block), BQ / 32 waves.
// The tile helpers below use its TILE / PER_WAVE split.
template <int D, int BQ>
struct DCfg {
  static constexpr int NW = BQ / 32;
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = 2 * D;               // bytes per key row
  static constexpr int TILE = BK * ROWB;           // bytes of one K (or V) block
  static constexpr int INSTR = TILE / 1024;        // DMA instructions per tile
  static constexpr int PER_WAVE = INSTR / NW;      // DMA instructions per wave per tile
  static constexpr int OROW = D * 2 + 16;          // bytes per staged output row
  static_assert(INSTR % NW == 0, "DMA instructions must split evenly over the waves");
  static_assert(((NW + 1) / 2) * 32 * OROW <= 2 * TILE, "output staging must fit in one buffer pair");
};

// Per-lane byte offsets, relative to the first row of a key block, of this wave's DMA copies of
// one tile (K and V tiles share them): instruction u of wave w copies 1 KiB stretch
// m = w * PER_WAVE + u; lane i fills bytes 16 i .. 16 i + 15 of it, i.e. row (m * 1024 + 16 i) / ROWB
// and swizzled chunk slot ((m * 1024 + 16 i) % ROWB) / 16, which holds logical chunk
// slot ^ kv_swz(row).
template <int D, int BQ>
__device__ __forceinline__ void dma_offsets(int wave, int lane, uint32_t (&off)[DCfg<D, BQ>::PER_WAVE]) {
  using C = DCfg<D, BQ>;
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) {
    const int byte = (wave * C::PER_WAVE + u) * 1024 + lane * 16;
    const int row = byte / C::ROWB;
    const int chunk = ((byte % C::ROWB) >> 4) ^ kv_swz<D>(row);
    off[u] = (uint32_t)((row * D + chunk * 8) * 2);
  }
}

// Issue this wave's DMA copies of the K or V tile of key block kb into dst. In a ragged last
// block, keys past N are clamped to N - 1: their scores are masked, so the copy only has to be
// finite and in bounds.
template <int D, int BQ>
__device__ __forceinline__ void dma_tile(const char* __restrict__ base, int kb, int N, int wave, int lane,
                                         const uint32_t (&off)[DCfg<D, BQ>::PER_WAVE], lchar* dst) {
  using C = DCfg<D, BQ>;
  const char* blk = base + (size_t)kb * BK * C::ROWB;
  if (kb * BK + BK <= N) {
#pragma unroll
    for (int u = 0; u < C::PER_WAVE; ++u)
      __builtin_amdgcn_global_load_lds(blk + off[u], dst + (wave * C::PER_WAVE + u) * 1024, 16, 0, 0);
  } else {
#pragma unroll
    for (int u = 0; u < C::PER_WAVE; ++u) {
      const int row = ((wave * C::PER_WAVE + u) * 1024 + lane * 16) / C::ROWB;
      const int over = kb * BK + row - (N - 1);
      const uint32_t o = over > 0 ? off[u] - (uint32_t)(over * C::ROWB) : off[u];
      __builtin_amdgcn_global_load_lds(blk + o, dst + (wave * C::PER_WAVE + u) * 1024, 16, 0, 0);
    }
  }
}

// dma_tile through a buffer resource: the descriptor covers the rows from key block kb to the end
// of the head (uniform, built in SGPRs), each lane adds its constant 32-bit offset, and rows past
// N lie outside the descriptor's range, so the hardware reads them as zeros instead of the copy
// clamping them. No per-lane address arithmetic. One head's rows must stay below 2 GiB.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* __restrict__ base, int kb, int N,
                                                            int rowb) {
  const int first = kb * BK;
  const int bytes = max(0, N - first) * rowb;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base) + (size_t)first * rowb, (short)0, bytes,
                                           0x00020000);
}

template <int D, int BQ>
__device__ __forceinline__ void dma_tile_rsrc(const char* __restrict__ base, int kb, int N, int wave,
                                              const uint32_t (&off)[DCfg<D, BQ>::PER_WAVE], lchar* dst) {
  using C = DCfg<D, BQ>;
  const __amdgpu_buffer_rsrc_t r = tile_rsrc(base, kb, N, C::ROWB);
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst + (wave * C::PER_WAVE + u) * 1024, 16, off[u], 0, 0, 0);
}

}  // namespace sa
