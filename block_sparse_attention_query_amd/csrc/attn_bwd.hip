// Block-sparse attention backward (gfx950, bf16 MFMA, fp32 accumulation).
//
// The sparse student of the SpargeAttention2 page ("SpargeAttention2とは？..." on ai-papers.net,
// section "ハイブリッドマスキングと蒸留微調整") is fine-tuned by distillation, which needs the gradients
// of the block-sparse attention for the same mask. With s = scale Q K^T over the kept keys,
// P = exp(s - LSE) (LSE saved by the forward), D = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Two passes: dQ per query block over its kept key blocks (the forward's walk), which also computes
// D and LSE * log2(e) for its queries and publishes them; then dK, dV per key block over the query
// blocks that keep it (the mask's columns). Every output
// element is written by exactly one workgroup, in a fixed order: no atomics, bitwise repeatable.
#include "attn_tiles.h"

namespace sa {

// ---------------------------------------------------------------- mask columns

// maskT[bh][j][i] = mask[bh][i][j], through a 64 x 64 LDS tile.
__global__ __launch_bounds__(256) void mask_transpose_kernel(const uint8_t* __restrict__ mask,
                                                             uint8_t* __restrict__ mask_t, int nqb, int nkb) {
  __shared__ uint8_t t[64][65];
  const int bh = blockIdx.z, i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const uint8_t* m = mask + (size_t)bh * nqb * nkb;
  uint8_t* mt = mask_t + (size_t)bh * nkb * nqb;
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    t[r][c] = (i0 + r < nqb && j0 + c < nkb) ? m[(size_t)(i0 + r) * nkb + j0 + c] : 0;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * 64; e += 256) {
    const int r = e >> 6, c = e & 63;
    if (j0 + r < nkb && i0 + c < nqb) mt[(size_t)(j0 + r) * nqb + i0 + c] = t[c][r];
  }
}

// ---------------------------------------------------------------- shared fragment helpers

// A or B operand of a 32x32x16 MFMA whose K dimension runs along the rows of a [row][col] bf16
// tile in LDS (rows of ROWB bytes, 16-byte chunks XOR-swizzled by SWZ(row)): the operand's 32
// M (or N) indices are columns col0 .. col0 + 31 and its 16 K indices are rows row0 .. row0 + 15.
// Two ds_read_b64_tr_b16 per lane: within each 16-lane group, lane s addresses row
// row0 + 8 u + 4 (group / 2) + s / 4 at columns col0 + 16 (group % 2) + 4 (s % 4) .. + 3, so lane i
// of the group receives column col0 + 16 (group % 2) + i of four consecutive rows.
// The swizzle of a row depends only on its low four bits, so for row0 a multiple of 16 the two
// read addresses are tile + off[u] + row0 ROWB with lane offsets off[u] that depend on col0 alone:
// tr_offsets computes them once, and tr_read adds row0 ROWB as an immediate.
template <int ROWB, int SWZD>
__device__ __forceinline__ void tr_offsets(int col0, int lane, int* off) {
  const int i16 = lane & 15, grp = lane >> 4;
  const int half = grp >> 1, gsub = grp & 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 8 * u + 4 * half + (i16 >> 2);
    const int chunk = ((col0 + 16 * gsub) >> 3) + ((i16 & 3) >> 1);
    off[u] = row * ROWB + ((chunk ^ kv_swz<SWZD>(row)) << 4) + (i16 & 1) * 8;
  }
}

template <int ROWB>
__device__ __forceinline__ bf16x8 tr_read(const lchar* tile, const int* off, int row0) {
  v4i16 part[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    part[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lchar*>(tile) + off[u] + row0 * ROWB));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------- dQ

// One workgroup per (b, h, query block), BQ / 32 waves of 32 queries, walking the kept list:
//   S^T = K Q^T, dP^T = V dO^T (A operands: 16-byte row reads of the K and V tiles),
//   dS^T = P^T * (dP^T - D) in registers (the B operand layout of the forward's P^T),
//   dQ^T += K^T dS^T (K^T by transpose reads of the K tile); the scale multiplies dQ once, in the
//   epilogue.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? 2 : 1) void attn_bwd_dq_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, const void* __restrict__ dout,
    const void* __restrict__ o, const float* __restrict__ lse, float* __restrict__ lse2p, float* __restrict__ deltap,
    const int32_t* __restrict__ kidx,
    const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float scale, float c_log2, void* __restrict__ dq) {
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char buf0_[2 * C::TILE];  // [K | V], even blocks
  __shared__ __attribute__((aligned(1024))) char buf1_[2 * C::TILE];  // [K | V], odd blocks
  lchar* const buf0 = (lchar*)buf0_;
  lchar* const buf1 = (lchar*)buf1_;

  const int tile = xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nqb;
  const int qb = tile - bh * nqb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(kcnt[tile], 0), nkb);
  const int32_t* list = kidx + (size_t)tile * nkb;
  auto blk = [&](int i) { return min(max(list[i], 0), nkb - 1); };

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;
  const char* gbase = static_cast<const char*>(dout) + head_off;

  uint32_t doff[C::PER_WAVE];
  dma_offsets<D, BQ>(wave, lane, doff);
  if (cnt > 0) {
    dma_tile_rsrc<D, BQ>(kbase, blk(0), N, wave, doff, buf0);
    dma_tile_rsrc<D, BQ>(vbase, blk(0), N, wave, doff, buf0 + C::TILE);
  }

  const int qrow = qb * BQ + wave * 32 + ln;
  const bool qvalid = qrow < N;
  bf16x8 qf[D / 16], gf[D / 16];  // Q^T and dO^T fragments: query qrow, channels 16 s + 8 hf .. + 7
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const size_t off = ((size_t)qrow * D + 16 * s + 8 * hf) * 2;
    qf[s] = __builtin_bit_cast(bf16x8, qvalid ? *reinterpret_cast<const uint4*>(qbase + off) : make_uint4(0, 0, 0, 0));
    gf[s] = __builtin_bit_cast(bf16x8, qvalid ? *reinterpret_cast<const uint4*>(gbase + off) : make_uint4(0, 0, 0, 0));
  }
  // D = rowsum(dO * O) of query qrow: this lane holds channels 16 s + 8 hf .. + 7 of dO, the lane
  // 32 apart the others. Rows past N (padding of the last block) get D = 0 and LSE = +inf, so
  // that their P and dS vanish without a mask. Both values go to deltap / lse2p (NP = nQB * BQ
  // per head) for the dK/dV pass; every padded row belongs to exactly one workgroup and lane.
  float dpart = 0.f;
  {
    const char* obase = static_cast<const char*>(o) + head_off;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const size_t off = ((size_t)qrow * D + 16 * s + 8 * hf) * 2;
      const uint4 ov = qvalid ? *reinterpret_cast<const uint4*>(obase + off) : make_uint4(0, 0, 0, 0);
      const uint4 gv = __builtin_bit_cast(uint4, gf[s]);
      const uint32_t wa[4] = {gv.x, gv.y, gv.z, gv.w}, wb[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) dpart += bf16_lo(wa[i]) * bf16_lo(wb[i]) + bf16_hi(wa[i]) * bf16_hi(wb[i]);
    }
  }
  const float dlt = partner32_sum(dpart);
  const float lse2 = qvalid ? lse[(size_t)bh * N + qrow] * 1.4426950408889634f : INFINITY;
  if (hf == 0) {
    lse2p[(size_t)bh * nqb * BQ + qrow] = lse2;
    deltap[(size_t)bh * nqb * BQ + qrow] = dlt;
  }

  int koff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = ln * C::ROWB + (((2 * s + hf) ^ sw) << 4);
  }
  int toff[D / 32][2];  // transpose-read offsets of K^T, channel tile r
#pragma unroll
  for (int r = 0; r < D / 32; ++r) tr_offsets<C::ROWB, D>(32 * r, lane, toff[r]);
  f32x16 acc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;

  // Block t of the list sits in buffer t & 1. The walk is unrolled by two so that each copy of the
  // step reads a fixed buffer and its base folds into the LDS reads' immediate offsets. The list
  // entries of blocks t and t + 1 are in scalar registers at step t; entry t + 2 is fetched during
  // step t by a vector load (counted by vmcnt, not by the lgkmcnt that the LDS reads wait on).
  int e0 = cnt > 0 ? blk(0) : 0, e1 = cnt > 1 ? blk(1) : -1;
  int vl = 0, lz = 0;
  asm volatile("" : "+v"(lz));  // a zero opaque to the compiler, which makes the list load a vector load
  auto step = [&](int t, const lchar* kt, lchar* nb) {
    const lchar* vt = kt + C::TILE;
    const int kb = e0, kn = e1;
    if (t + 2 < cnt) vl = list[t + 2 + lz];
    f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
    // operands of channel slice s + 1 are read while the products of slice s run
    bf16x8 ra[2][4];
    auto rd = [&](int s, bf16x8 (&r)[4]) {
      r[0] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s]);
      r[1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s] + 32 * C::ROWB);
      r[2] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s]);
      r[3] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s] + 32 * C::ROWB);
    };
    rd(0, ra[0]);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 1 < D / 16) rd(s + 1, ra[(s + 1) & 1]);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s & 1][0], qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s & 1][1], qf[s], s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s & 1][2], gf[s], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s & 1][3], gf[s], p1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keeps the reads of slice s + 1 ahead of these products
    }
    // block t + 1 into the other buffer, issued behind the products so that the waves released by
    // the barrier start on the matrix cores
    if (kn >= 0) {
      dma_tile_rsrc<D, BQ>(kbase, kn, N, wave, doff, nb);
      dma_tile_rsrc<D, BQ>(vbase, kn, N, wave, doff, nb + C::TILE);
    }
    if (kb * BK + BK > N) {  // ragged last key block: keys past N take no part
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
        float a = key >= N ? -INFINITY : s0[i], b = key + 32 >= N ? -INFINITY : s1[i];
        // the empty asm cannot be speculated, which keeps this a branch: as selects hoisted out
        // of it the mask would cost every block
        asm volatile("" : "+v"(a), "+v"(b));
        s0[i] = a;
        s1[i] = b;
      }
    }
    // dS^T as the B operand: key chunk c = 2 t + u takes elements 8u .. 8u+7 of tile t. This
    // vector-bound phase runs at raised priority, so that the other wave on the SIMD fills the
    // matrix core around it.
    __builtin_amdgcn_s_setprio(1);
    bf16x8 db[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 8 * u + 2 * e + h;
          x[h] = __builtin_amdgcn_exp2f(fmaf(s0[i], c_log2, -lse2)) * (p0[i] - dlt);
          x[2 + h] = __builtin_amdgcn_exp2f(fmaf(s1[i], c_log2, -lse2)) * (p1[i] - dlt);
        }
        w0[e] = pack_bf16(x[0], x[1]);
        w1[e] = pack_bf16(x[2], x[3]);
      }
      db[u] = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      db[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    }
    __builtin_amdgcn_s_setprio(0);
    // dQ^T (channels x queries) += K^T (channels x keys) dS^T (keys x queries)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < D / 32; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<C::ROWB>(kt, toff[r], 16 * c), db[c], acc[r], 0, 0, 0);
    e0 = e1;
    e1 = t + 2 < cnt ? min(max(__builtin_amdgcn_readfirstlane(vl), 0), nkb - 1) : -1;
  };
  for (int t = 0; t < cnt; t += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block t is resident in buffer 0; every wave is done with buffer 1
    step(t, buf0, buf1);
    if (t + 1 < cnt) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // block t + 1 is resident in buffer 1; every wave is done with buffer 0
      step(t + 1, buf1, buf0);
    }
  }
  __syncthreads();

  // epilogue: dQ^T staged through LDS (two waves per buffer) for row-contiguous stores
  lchar* ol = ((wave & 1) ? buf1 : buf0) + (wave >> 1) * 32 * C::OROW;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * r + 8 * a + 4 * hf;
      const u32x2 w = {pack_bf16(acc[r][4 * a] * scale, acc[r][4 * a + 1] * scale),
                       pack_bf16(acc[r][4 * a + 2] * scale, acc[r][4 * a + 3] * scale)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(ol + ln * C::OROW + ch * 2) = w;
    }
  __syncthreads();
  constexpr int CH16 = D * 2 / 16;
  char* obase = static_cast<char*>(dq) + head_off;
  for (int e = lane; e < 32 * CH16; e += 64) {
    const int r = e / CH16, cc = e % CH16;
    const int qr = qb * BQ + wave * 32 + r;
    if (qr < N)
      *reinterpret_cast<u32x4*>(obase + (size_t)qr * D * 2 + cc * 16) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(ol + r * C::OROW + cc * 16);
  }
}

// ---------------------------------------------------------------- dK, dV

// Launch geometry of the dK / dV kernel: one workgroup of two waves per (b, h, key block j);
// wave w owns keys 32 w .. 32 w + 31 of the block. The query side streams through LDS in steps
// of 64 queries (one 64-row Q tile, one dO tile, their 64 LSE and 64 D values), double buffered.
template <int D>
struct KVCfg {
  static constexpr int NW = 2;
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = 2 * D;         // bytes per token row
  static constexpr int TILE = 64 * ROWB;     // 64 rows of Q or of dO
  static constexpr int OFF_G = TILE;         // dO tile
  static constexpr int OFF_L = 2 * TILE;     // 64 floats: LSE * log2(e) (+inf on padded rows)
  static constexpr int OFF_D = 2 * TILE + 256;  // 64 floats: D (0 on padded rows)
  static constexpr int BUF = 2 * TILE + 512;
  static constexpr int OROW = D * 2 + 16;    // bytes per staged output row
  static_assert(64 * OROW <= BUF, "output staging must fit in one buffer");
};

// Copies of the 64-row tile sb (token rows 64 sb .. + 63) of a [N][D] bf16 tensor into a
// swizzled LDS tile by the two waves: instruction u of wave w fills the 1 KiB stretch
// m = w PW + u; lane i fills its bytes 16 i .. + 15, i.e. row (1024 m + 16 i) / ROWB and swizzled
// chunk slot ((1024 m + 16 i) % ROWB) / 16, which holds logical chunk slot ^ kv_swz(row).
// kv_dma_offsets gives each lane's byte offsets inside a tile.
template <int D>
struct KVDma {
  static constexpr int ROWB = 2 * D;
  static constexpr int PW = 64 * ROWB / 1024 / 2;
};

template <int D>
__device__ __forceinline__ void kv_dma_offsets(int wave, int lane, uint32_t* off) {
  constexpr int ROWB = KVDma<D>::ROWB;
#pragma unroll
  for (int u = 0; u < KVDma<D>::PW; ++u) {
    const int byte = (wave * KVDma<D>::PW + u) * 1024 + lane * 16;
    const int row = byte / ROWB;
    off[u] = (uint32_t)(row * ROWB + ((((byte % ROWB) >> 4) ^ kv_swz<D>(row)) << 4));
  }
}

// The copies of one step, as 2 PW + 1 single instructions per wave that the walk spreads between
// matrix products: part u < PW fills the wave's stretch u of the Q tile, PW <= u < 2 PW stretch
// u - PW of the dO tile, part 2 PW the step's 64 LSE (wave 0) or D (wave 1) values. The tiles go
// through buffer descriptors covering query rows 64 sb .. N - 1, so rows past N read as zeros;
// such padded queries have LSE +inf and D 0, which makes their P and dS zero.
struct KVStep {
  __amdgpu_buffer_rsrc_t rq, rg;
  const float* ld;
  lchar* dst;
};

template <int D>
__device__ __forceinline__ KVStep kv_step(const char* qbase, const char* gbase, const float* ldbase, int sb, int N,
                                          lchar* dst) {
  return {tile_rsrc(qbase, sb, N, KVDma<D>::ROWB), tile_rsrc(gbase, sb, N, KVDma<D>::ROWB), ldbase + sb * 64, dst};
}

// (a plain function: the host pass rejects templates whose bodies hold these copy builtins)
__device__ __forceinline__ void kv_part(const KVStep& c, int wave, int lane, const uint32_t* off, int part, int pw,
                                        int off_g, int off_l) {
  if (part < pw)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rq, c.dst + (wave * pw + part) * 1024, 16, off[part], 0, 0, 0);
  else if (part < 2 * pw)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rg, c.dst + off_g + (wave * pw + part - pw) * 1024, 16, off[part - pw],
                                             0, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(c.ld + lane, c.dst + off_l + wave * 256, 4, 0, 0);
}

// One workgroup per (b, h, key block j), walking the 64-query steps of the query blocks that keep
// j (the mask's column, ascending). The key side is resident in registers for the whole walk: K
// and V rows of the wave's 32 keys are the B operands of S = Q K^T and dP = dO V^T (queries in
// M, keys in N). The products' results leave each lane one key and 16 queries, which is the A
// operand layout of dV += P^T dO and dK += dS^T Q (keys in M, queries in K) up to an order of the
// queries inside each run of 16; the dO and Q operands of those products are transpose reads
// whose row order matches it. So P and dS never leave registers and a step has one barrier: the
// one that hands the next buffer to the copies.
template <int D, int BQ>
__global__ __launch_bounds__(128, 1) void attn_bwd_dkdv_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, const void* __restrict__ dout,
    const float* __restrict__ lse2p, const float* __restrict__ deltap, const int32_t* __restrict__ cidx,
    const int32_t* __restrict__ ccnt, int N, int nqb, int nkb, float scale, float c_log2, void* __restrict__ dk,
    void* __restrict__ dv) {
  using C = KVCfg<D>;
  constexpr int SPB = BQ / 64;  // 64-query steps per query block
  // the two buffers are separate arrays, so that the compiler can tell the reads of one from the
  // copies into the other and does not wait for those copies before the transpose reads
  __shared__ __attribute__((aligned(1024))) char buf0_[C::BUF];
  __shared__ __attribute__((aligned(1024))) char buf1_[C::BUF];
  lchar* const base0 = (lchar*)buf0_;
  lchar* const base1 = (lchar*)buf1_;

  const int tile = xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nkb;
  const int kb = tile - bh * nkb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(ccnt[tile], 0), nqb);
  const int32_t* list = cidx + (size_t)tile * nqb;
  const int NP = nqb * BQ;  // padded queries per head of the LSE and D arrays
  // steps are the 64-query sub-blocks of the listed query blocks; when the last query block is
  // ragged and its second half lies wholly past N, that half is not a step
  int T = cnt * SPB;
  if (SPB == 2 && cnt > 0 && min(max(list[cnt - 1], 0), nqb - 1) == nqb - 1 && (nqb - 1) * BQ + 64 >= N) T -= 1;

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* gbase = static_cast<const char*>(dout) + head_off;
  const float* l2base = lse2p + (size_t)bh * NP;
  const float* dlbase = deltap + (size_t)bh * NP;
  uint32_t doff[KVDma<D>::PW];
  kv_dma_offsets<D>(wave, lane, doff);
  const float* ldbase = wave == 0 ? l2base : dlbase;
  constexpr int NPART = 2 * KVDma<D>::PW + 1;  // copy instructions per wave and step
  // query sub-block of step t (list entries clamped to [0, nQB))
  auto sbof = [&](int t) { return min(max(list[t / SPB], 0), nqb - 1) * SPB + t % SPB; };
  if (T > 0) {
    const KVStep c0 = kv_step<D>(qbase, gbase, ldbase, sbof(0), N, base0);
#pragma unroll
    for (int part = 0; part < NPART; ++part) kv_part(c0, wave, lane, doff, part, KVDma<D>::PW, C::OFF_G, C::OFF_L);
  }

  // K and V rows of key 32 w + ln, channels 16 s + 8 hf .. + 7: the B operands (keys past N are 0)
  const int key = kb * BK + wave * 32 + ln;
  const bool kvalid = key < N;
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const size_t off = head_off + ((size_t)key * D + 16 * s + 8 * hf) * 2;
    kf[s] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const uint4*>(static_cast<const char*>(k) + off)
                                              : make_uint4(0, 0, 0, 0));
    vf[s] = __builtin_bit_cast(bf16x8, kvalid ? *reinterpret_cast<const uint4*>(static_cast<const char*>(v) + off)
                                              : make_uint4(0, 0, 0, 0));
  }
  // A operands of S and dP: query row ln (+ 32 h) of the tile, logical chunk 2 s + hf
  int roff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) roff[s] = ln * C::ROWB + (((2 * s + hf) ^ sw) << 4);
  }

  int toff[D / 32][2];  // transpose-read offsets of dO and Q, channel tile c
#pragma unroll
  for (int c = 0; c < D / 32; ++c) tr_offsets<C::ROWB, D>(32 * c, lane, toff[c]);
  f32x16 acc_k[D / 32], acc_v[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc_k[c][i] = 0.f;
      acc_v[c][i] = 0.f;
    }

  // Step t sits in buffer t & 1. The walk is unrolled by two so that each copy of the step reads
  // a fixed buffer and its address folds into the LDS reads' immediate offsets.
  // The step reading buffer qt also copies step sbn's tiles (sbn < 0: none) into nb, two copy
  // instructions after each of the first S / dP product pairs.
  auto step = [&](const lchar* qt, lchar* nb, int sbn) {
    const lchar* gt = qt + C::OFF_G;
    const KVStep cp = kv_step<D>(qbase, gbase, ldbase, max(sbn, 0), N, nb);

    // S = Q K^T and dP = dO V^T for queries 32 h .. 32 h + 31 of the step: element i of lane
    // (ln, hf) is key 32 w + ln, query 32 h + 8 (i / 4) + 4 hf + i % 4.
    // The step runs in four phases so that the vector work lies under matrix products of the same
    // wave (one wave per SIMD): A. S, dP of half 0; B. S, dP of half 1, with P and dS of half 0
    // computed between the products; C. dV, dK of half 0, with P and dS of half 1 between them;
    // D. dV, dK of half 1. Operands are read one product step ahead throughout.
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[h][i] = 0.f;
        dp[h][i] = 0.f;
      }
    // P = exp(s - LSE) and dS = P (dP - D) of queries 32 h + 16 u + 8 g + 4 hf .. + 3 (the scale
    // multiplies dK in the epilogue), packed to bf16 as words 2 g, 2 g + 1 of the A operands of
    // run u of half h (elements 8 u + 4 g .. + 3)
    uint32_t wp[2][2][4], ws[2][2][4];
    auto ps_quad = [&](int h, int u, int g) {
      const int qi = 32 * h + 16 * u + 8 * g + 4 * hf;
      const f32x4 lv = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(qt + C::OFF_L + qi * 4);
      const f32x4 dv4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(qt + C::OFF_D + qi * 4);
      float pv[4], sv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * u + 4 * g + e;
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[h][i], c_log2, -lv[e]));
        sv[e] = pv[e] * (dp[h][i] - dv4[e]);
      }
      wp[h][u][2 * g] = pack_bf16(pv[0], pv[1]);
      wp[h][u][2 * g + 1] = pack_bf16(pv[2], pv[3]);
      ws[h][u][2 * g] = pack_bf16(sv[0], sv[1]);
      ws[h][u][2 * g + 1] = pack_bf16(sv[2], sv[3]);
      // empty asms keep this work where the schedule puts it (IR passes would sink it to its use)
      asm volatile("" : "+v"(wp[h][u][2 * g]), "+v"(wp[h][u][2 * g + 1]), "+v"(ws[h][u][2 * g]),
                   "+v"(ws[h][u][2 * g + 1]));
    };
    // phases A and B: step n = 8 h + s of the S / dP products, their Q and dO operands read two
    // product steps ahead (a ring of three)
    constexpr int SS = D / 16;
    bf16x8 ring[3][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      ring[a][0] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qt + roff[a % SS] + 32 * (a / SS) * C::ROWB);
      ring[a][1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(gt + roff[a % SS] + 32 * (a / SS) * C::ROWB);
    }
#pragma unroll
    for (int n = 0; n < 2 * SS; ++n) {
      const int h = n / SS, s = n % SS;
      if (n + 2 < 2 * SS) {
        const int h1 = (n + 2) / SS, s1 = (n + 2) % SS;
        ring[(n + 2) % 3][0] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qt + roff[s1] + 32 * h1 * C::ROWB);
        ring[(n + 2) % 3][1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(gt + roff[s1] + 32 * h1 * C::ROWB);
      }
      sc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % 3][0], kf[s], sc[h], 0, 0, 0);
      dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[n % 3][1], vf[s], dp[h], 0, 0, 0);
      if (2 * n < NPART && sbn >= 0) {
        kv_part(cp, wave, lane, doff, 2 * n, KVDma<D>::PW, C::OFF_G, C::OFF_L);
        if (2 * n + 1 < NPART) kv_part(cp, wave, lane, doff, 2 * n + 1, KVDma<D>::PW, C::OFF_G, C::OFF_L);
      }
      // half 0's P and dS under half 1's products (four quads over its SS steps)
      if (h == 1 && (s % (SS / 4)) == (SS / 4) - 1) {
        const int qd = s / (SS / 4);
        ps_quad(0, qd >> 1, qd & 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // phases C and D: dV += P^T dO and dK += dS^T Q, item j = (h, u, channel tile c); the
    // transposed operands of item j + PD are read while the products of item j run (PD items of
    // LDS latency covered; phase B, not these phases, sets the register peak)
    constexpr int NC = D / 32, NJ = 4 * NC, PD = 2;
    auto item_row = [](int j) { return 32 * (j / (2 * NC)) + 16 * ((j / NC) & 1); };
    bf16x8 rg[PD + 1], rq[PD + 1];
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      rg[j] = tr_read<C::ROWB>(gt, toff[j % NC], item_row(j));
      rq[j] = tr_read<C::ROWB>(qt, toff[j % NC], item_row(j));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int h = j / (2 * NC), u = (j / NC) & 1, c = j % NC;
      if (j + PD < NJ) {
        rg[(j + PD) % (PD + 1)] = tr_read<C::ROWB>(gt, toff[(j + PD) % NC], item_row(j + PD));
        rq[(j + PD) % (PD + 1)] = tr_read<C::ROWB>(qt, toff[(j + PD) % NC], item_row(j + PD));
      }
      const bf16x8 pa = __builtin_bit_cast(bf16x8, make_uint4(wp[h][u][0], wp[h][u][1], wp[h][u][2], wp[h][u][3]));
      const bf16x8 sa = __builtin_bit_cast(bf16x8, make_uint4(ws[h][u][0], ws[h][u][1], ws[h][u][2], ws[h][u][3]));
      acc_v[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, rg[j % (PD + 1)], acc_v[c], 0, 0, 0);
      acc_k[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, rq[j % (PD + 1)], acc_k[c], 0, 0, 0);
      // half 1's P and dS under half 0's products (four quads over the 2 NC items of half 0)
      if (h == 0 && (j % (2 * NC / 4)) == (2 * NC / 4) - 1) {
        const int qd = j / (2 * NC / 4);
        ps_quad(1, qd >> 1, qd & 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The list entry of step t + 2 is fetched during step t by a vector load (counted by vmcnt, not
  // by the lgkmcnt that the LDS reads wait on) and moved to a scalar register after the step.
  int vl = 0, lz = 0;
  asm volatile("" : "+v"(lz));  // a zero opaque to the compiler, which makes the list load a vector load
  auto sb_at = [&](int t, int entry) { return min(max(entry, 0), nqb - 1) * SPB + t % SPB; };
  int sbn = T > 1 ? sbof(1) : -1;
  for (int t = 0; t < T; t += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // step t is resident in buffer 0; both waves are done with buffer 1
    if (t + 2 < T) vl = list[(t + 2) / SPB + lz];
    step(base0, base1, sbn);
    sbn = t + 2 < T ? sb_at(t + 2, __builtin_amdgcn_readfirstlane(vl)) : -1;
    if (t + 1 < T) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // step t + 1 is resident in buffer 1; both waves are done with buffer 0
      if (t + 3 < T) vl = list[(t + 3) / SPB + lz];
      step(base1, base0, sbn);
      sbn = t + 3 < T ? sb_at(t + 3, __builtin_amdgcn_readfirstlane(vl)) : -1;
    }
  }
  __syncthreads();  // every wave is done with the last step's buffer

  // epilogue: dK (times the scale) then dV, staged through LDS as [key][channel] rows. Element i
  // of tile c: channel 32 c + ln, key 32 w + 8 (i / 4) + 4 hf + i % 4
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const f32x16& acc = which == 0 ? acc_k[c] : acc_v[c];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 32 * wave + 8 * (i >> 2) + 4 * hf + (i & 3);
        *reinterpret_cast<__attribute__((address_space(3))) __bf16*>(base0 + kr * C::OROW + (32 * c + ln) * 2) =
            (__bf16)(which == 0 ? acc[i] * scale : acc[i]);
      }
    }
    __syncthreads();
    char* obase = static_cast<char*>(which == 0 ? dk : dv) + head_off;
    constexpr int CH16 = D * 2 / 16;
    for (int e = threadIdx.x; e < BK * CH16; e += C::NT) {
      const int r = e / CH16, cc = e % CH16;
      const int kr = kb * BK + r;
      if (kr < N)
        *reinterpret_cast<u32x4*>(obase + (size_t)kr * D * 2 + cc * 16) =
            *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base0 + r * C::OROW + cc * 16);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launcher

hipError_t launch_compact(const uint8_t* mask, int rows, int nkb, int32_t* kidx, int32_t* kcnt, hipStream_t stream);

size_t bwd_workspace_bytes(int BH, int N, int Bq) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nqb = (N + Bq - 1) / Bq, nkb = (N + BK - 1) / BK;
  return al(BH * nqb * nkb * 4) + al(BH * nqb * 4) + al(BH * nkb * nqb * 4) + al(BH * nkb * 4) + al(BH * nkb * nqb) +
         2 * al((size_t)BH * nqb * Bq * 4);
}

template <int D, int BQ>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, const uint8_t* mask, int BH, int N, float scale, void* dq, void* dk,
                               void* dv, void* ws, hipStream_t stream) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const int nqb = (N + BQ - 1) / BQ, nkb = (N + BK - 1) / BK;
  char* p = static_cast<char*>(ws);
  int32_t* ridx = reinterpret_cast<int32_t*>(p);
  p += al((size_t)BH * nqb * nkb * 4);
  int32_t* rcnt = reinterpret_cast<int32_t*>(p);
  p += al((size_t)BH * nqb * 4);
  int32_t* cidx = reinterpret_cast<int32_t*>(p);
  p += al((size_t)BH * nkb * nqb * 4);
  int32_t* ccnt = reinterpret_cast<int32_t*>(p);
  p += al((size_t)BH * nkb * 4);
  uint8_t* mask_t = reinterpret_cast<uint8_t*>(p);
  p += al((size_t)BH * nkb * nqb);
  const int NP = nqb * BQ;
  float* deltap = reinterpret_cast<float*>(p);
  p += al((size_t)BH * NP * 4);
  float* lse2p = reinterpret_cast<float*>(p);

  hipError_t e = launch_compact(mask, BH * nqb, nkb, ridx, rcnt, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mask_transpose_kernel, dim3((unsigned)((nkb + 63) / 64), (unsigned)((nqb + 63) / 64), (unsigned)BH),
                     dim3(256), 0, stream, mask, mask_t, nqb, nkb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_compact(mask_t, BH * nkb, nqb, cidx, ccnt, stream)) != hipSuccess) return e;
  const float c_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, BQ>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D, BQ>::NT), 0, stream, q, k, v,
                     dout, o, lse, lse2p, deltap, ridx, rcnt, N, nqb, nkb, scale, c_log2, dq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  using C = KVCfg<D>;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BQ>), dim3((unsigned)(BH * nkb)), dim3(C::NT), 0, stream, q, k, v,
                     dout, lse2p, deltap, cidx, ccnt, N, nqb, nkb, scale, c_log2, dk, dv);
  return hipGetLastError();
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      const uint8_t* mask, int BH, int N, int d, int Bq, double scale, void* dq, void* dk, void* dv,
                      void* ws, hipStream_t stream) {
  const float sc = (float)scale;
  if (d == 128 && Bq == 128) return launch_bwd_t<128, 128>(q, k, v, o, dout, lse, mask, BH, N, sc, dq, dk, dv, ws, stream);
  if (d == 128 && Bq == 64) return launch_bwd_t<128, 64>(q, k, v, o, dout, lse, mask, BH, N, sc, dq, dk, dv, ws, stream);
  if (d == 64 && Bq == 128) return launch_bwd_t<64, 128>(q, k, v, o, dout, lse, mask, BH, N, sc, dq, dk, dv, ws, stream);
  if (d == 64 && Bq == 64) return launch_bwd_t<64, 64>(q, k, v, o, dout, lse, mask, BH, N, sc, dq, dk, dv, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
