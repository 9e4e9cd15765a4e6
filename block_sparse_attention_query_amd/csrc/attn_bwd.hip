// Block-sparse attention backward (gfx950, bf16 MFMA, fp32 accumulation).
//
// The sparse student of the SpargeAttention2 page ("SpargeAttention2とは？..." on ai-papers.net,
// section "ハイブリッドマスキングと蒸留微調整") is fine-tuned by distillation, which needs the gradients
// of the block-sparse attention for the same mask. With s = scale Q K^T over the kept keys,
// P = exp(s - LSE) (LSE saved by the forward), D = rowsum(dO * O):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// Three passes: D per query; dQ per query block over its kept key blocks (the forward's walk);
// dK, dV per key block over the query blocks that keep it (the mask's columns). Every output
// element is written by exactly one workgroup, in a fixed order: no atomics, bitwise repeatable.
#include "attn_tiles.h"

namespace sa {

// ---------------------------------------------------------------- D = rowsum(dO * O)

template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const char* __restrict__ dout, const char* __restrict__ o,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int VPR = D / 8;  // 16-byte chunks per bf16 row; VPR lanes reduce one row
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long r = e / VPR;
  const int c = (int)(e % VPR);
  float acc = 0.f;
  if (r < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(dout + (size_t)r * D * 2 + c * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(o + (size_t)r * D * 2 + c * 16);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(wa[i]) * bf16_lo(wb[i]) + bf16_hi(wa[i]) * bf16_hi(wb[i]);
  }
#pragma unroll
  for (int off = VPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (r < rows && c == 0) delta[r] = acc;
}

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
template <int ROWB, int SWZD>
__device__ __forceinline__ bf16x8 tr_operand(const lchar* tile, int row0, int col0, int lane) {
  const int i16 = lane & 15, grp = lane >> 4;
  const int half = grp >> 1, gsub = grp & 1;
  v4i16 part[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = row0 + 8 * u + 4 * half + (i16 >> 2);
    const int chunk = ((col0 + 16 * gsub) >> 3) + ((i16 & 3) >> 1);
    const int off = row * ROWB + ((chunk ^ kv_swz<SWZD>(row)) << 4) + (i16 & 1) * 8;
    part[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lchar*>(tile) + off));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// bf16 fragment of 8 consecutive elements of row `row`, logical 16-byte chunk `chunk`, from a
// swizzled [row][col] tile (the layout the DMA helpers write).
template <int ROWB, int SWZD>
__device__ __forceinline__ bf16x8 row_operand(const lchar* tile, int row, int chunk) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
      tile + row * ROWB + ((chunk ^ kv_swz<SWZD>(row)) << 4));
}

// DMA of `rows` consecutive token rows (from row0; rows past N are clamped to N - 1) of a
// [N][D] bf16 tensor into a swizzled LDS tile, by the NW waves of the workgroup.
template <int D, int NW>
__device__ __forceinline__ void dma_rows(const char* __restrict__ base, int row0, int rows, int N, int wave,
                                         int lane, lchar* dst) {
  constexpr int ROWB = 2 * D;
  const int instr = rows * ROWB / 1024;
  for (int m = wave; m < instr; m += NW) {
    const int byte = m * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int chunk = ((byte % ROWB) >> 4) ^ kv_swz<D>(row);
    const int src = min(row0 + row, N - 1);
    __builtin_amdgcn_global_load_lds(base + ((size_t)src * D + chunk * 8) * 2, dst + m * 1024, 16, 0, 0);
  }
}

// ---------------------------------------------------------------- dQ

// One workgroup per (b, h, query block), BQ / 32 waves of 32 queries, walking the kept list:
//   S^T = K Q^T, dP^T = V dO^T (A operands: 16-byte row reads of the K and V tiles),
//   dS^T = P^T * (dP^T - D) * scale in registers (the B operand layout of the forward's P^T),
//   dQ^T += K^T dS^T (K^T by transpose reads of the K tile).
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 2) void attn_bwd_dq_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, const void* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const int32_t* __restrict__ kidx,
    const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float scale, float c_log2, void* __restrict__ dq) {
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char buf0_[2 * C::TILE];  // [K | V], even blocks
  __shared__ __attribute__((aligned(1024))) char buf1_[2 * C::TILE];  // [K | V], odd blocks
  lchar* const buf0 = (lchar*)buf0_;
  lchar* const buf1 = (lchar*)buf1_;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
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
    dma_tile<D, BQ>(kbase, blk(0), N, wave, lane, doff, buf0);
    dma_tile<D, BQ>(vbase, blk(0), N, wave, lane, doff, buf0 + C::TILE);
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
  const float lse2 = qvalid ? lse[(size_t)bh * N + qrow] * 1.4426950408889634f : INFINITY;
  const float dlt = qvalid ? delta[(size_t)bh * N + qrow] : 0.f;

  int koff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = ln * C::ROWB + (((2 * s + hf) ^ sw) << 4);
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;

  for (int t = 0; t < cnt; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block t is resident; every wave is done with the other buffer
    if (t + 1 < cnt) {
      lchar* nb = (t & 1) ? buf0 : buf1;
      dma_tile<D, BQ>(kbase, blk(t + 1), N, wave, lane, doff, nb);
      dma_tile<D, BQ>(vbase, blk(t + 1), N, wave, lane, doff, nb + C::TILE);
    }
    const lchar* kt = (t & 1) ? buf1 : buf0;
    const lchar* vt = kt + C::TILE;
    const int kb = blk(t);
    f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s] + 32 * C::ROWB);
      const bf16x8 b0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s]);
      const bf16x8 b1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s] + 32 * C::ROWB);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, gf[s], p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, gf[s], p1, 0, 0, 0);
    }
    if (kb * BK + BK > N) {  // ragged last key block: keys past N take no part
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (key >= N) s0[i] = -INFINITY;
        if (key + 32 >= N) s1[i] = -INFINITY;
      }
    }
    // dS^T as the B operand: key chunk c = 2 t + u takes elements 8u .. 8u+7 of tile t
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
          x[h] = __builtin_amdgcn_exp2f(fmaf(s0[i], c_log2, -lse2)) * (p0[i] - dlt) * scale;
          x[2 + h] = __builtin_amdgcn_exp2f(fmaf(s1[i], c_log2, -lse2)) * (p1[i] - dlt) * scale;
        }
        w0[e] = pack_bf16(x[0], x[1]);
        w1[e] = pack_bf16(x[2], x[3]);
      }
      db[u] = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      db[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    }
    // dQ^T (channels x queries) += K^T (channels x keys) dS^T (keys x queries)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < D / 32; ++r)
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<C::ROWB, D>(kt, 16 * c, 32 * r, lane), db[c],
                                                          acc[r], 0, 0, 0);
  }
  __syncthreads();

  // epilogue: dQ^T staged through LDS (two waves per buffer) for row-contiguous stores
  lchar* ol = ((wave & 1) ? buf1 : buf0) + (wave >> 1) * 32 * C::OROW;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * r + 8 * a + 4 * hf;
      const u32x2 w = {pack_bf16(acc[r][4 * a], acc[r][4 * a + 1]), pack_bf16(acc[r][4 * a + 2], acc[r][4 * a + 3])};
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

template <int D, int BQ>
struct BCfg {
  static constexpr int NW = BQ / 32;
  static constexpr int NT = NW * 64;
  static constexpr int ROWB = 2 * D;              // bytes per token row of K, V, Q, dO tiles
  static constexpr int KT = BK * ROWB;            // K or V tile
  static constexpr int QT = BQ * ROWB;            // Q or dO tile
  static constexpr int PROWB = 2 * BK;            // bytes per query row of the P^T / dS^T tiles
  static constexpr int PT = BQ * PROWB;
  static constexpr int OFF_V = KT, OFF_Q = 2 * KT, OFF_G = 2 * KT + QT, OFF_P = 2 * KT + 2 * QT,
                       OFF_S = 2 * KT + 2 * QT + PT;
  static constexpr int LDS = 2 * KT + 2 * QT + 2 * PT;
  static constexpr int TILES = 2 * (D / 32);      // 32 x 32 output tiles of dK (and of dV)
  static constexpr int TPW = TILES / NW;          // per wave
  static constexpr int OROW = D * 2 + 16;
  static_assert(TILES % NW == 0, "output tiles must split evenly over the waves");
  static_assert(BK * OROW <= LDS, "output staging must fit");
};

// One workgroup per (b, h, key block j), walking the query blocks that keep j. Per query block:
//   phase A, wave w on queries 32 w .. 32 w + 31: S^T = K_j Q^T and dP^T = V_j dO^T, then
//     P^T = exp(S^T - LSE) and dS^T = P^T * (dP^T - D) * scale, written to LDS as [query][key];
//   phase B, wave w on its output tiles: dV_j += P^T dO and dK_j += dS^T Q, every operand by
//     transpose reads (the K dimension is the query, the rows of all four tiles).
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 1) void attn_bwd_dkdv_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, const void* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const int32_t* __restrict__ cidx,
    const int32_t* __restrict__ ccnt, int N, int nqb, int nkb, float scale, float c_log2, void* __restrict__ dk,
    void* __restrict__ dv) {
  using C = BCfg<D, BQ>;
  extern __shared__ __attribute__((aligned(1024))) char lds_[];
  lchar* const base = (lchar*)lds_;
  lchar* const kt = base;
  lchar* const vt = base + C::OFF_V;
  lchar* const qt = base + C::OFF_Q;
  lchar* const gt = base + C::OFF_G;
  lchar* const pt = base + C::OFF_P;
  lchar* const st = base + C::OFF_S;

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / nkb;
  const int kb = tile - bh * nkb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(ccnt[tile], 0), nqb);
  const int32_t* list = cidx + (size_t)tile * nqb;

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;
  const char* gbase = static_cast<const char*>(dout) + head_off;
  dma_rows<D, C::NW>(kbase, kb * BK, BK, N, wave, lane, kt);
  dma_rows<D, C::NW>(vbase, kb * BK, BK, N, wave, lane, vt);

  int koff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = ln * C::ROWB + (((2 * s + hf) ^ sw) << 4);
  }
  f32x16 acc_v[C::TPW], acc_k[C::TPW];
#pragma unroll
  for (int a = 0; a < C::TPW; ++a)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc_v[a][i] = 0.f;
      acc_k[a][i] = 0.f;
    }

  for (int t = 0; t < cnt; ++t) {
    const int ib = min(max(list[t], 0), nqb - 1);
    __syncthreads();  // phase B of the previous query block is done with the Q, dO, P, dS tiles
    dma_rows<D, C::NW>(qbase, ib * BQ, BQ, N, wave, lane, qt);
    dma_rows<D, C::NW>(gbase, ib * BQ, BQ, N, wave, lane, gt);
    const int qrow = ib * BQ + wave * 32 + ln;
    const bool qvalid = qrow < N;
    const float lse2 = qvalid ? lse[(size_t)bh * N + qrow] * 1.4426950408889634f : INFINITY;
    const float dlt = qvalid ? delta[(size_t)bh * N + qrow] : 0.f;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // phase A: S^T and dP^T for this wave's 32 queries (rows 32 w + ln of the Q and dO tiles)
    f32x16 s0 = {}, s1 = {}, p0 = {}, p1 = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int qo = koff[s] + wave * 32 * C::ROWB;  // the swizzle depends on the row's low bits only
      const bf16x8 bq = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qt + qo);
      const bf16x8 bg = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(gt + qo);
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s] + 32 * C::ROWB);
      const bf16x8 c0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s]);
      const bf16x8 c1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(vt + koff[s] + 32 * C::ROWB);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bq, s1, 0, 0, 0);
      p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c0, bg, p0, 0, 0, 0);
      p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c1, bg, p1, 0, 0, 0);
    }
    // P^T and dS^T to LDS, [query][key]: element i of tile h holds key 32 h + 8 (i / 4) + 4 hf + i % 4
    // of query 32 w + ln, so each group of four is 8 contiguous bytes of the query's row
    const int prow = wave * 32 + ln;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float pv[4], sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g + e;
          const float sc = h == 0 ? s0[i] : s1[i];
          const float dp = h == 0 ? p0[i] : p1[i];
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sc, c_log2, -lse2));
          sv[e] = pv[e] * (dp - dlt) * scale;
        }
        const int chunk = 4 * h + g;  // 16-byte chunk of keys 32 h + 8 g .. + 7; this lane half's 8 bytes
        const int off = prow * C::PROWB + ((chunk ^ kv_swz<BK>(prow)) << 4) + hf * 8;
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(pt + off) =
            (u32x2){pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3])};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(st + off) =
            (u32x2){pack_bf16(sv[0], sv[1]), pack_bf16(sv[2], sv[3])};
      }
    __syncthreads();

    // phase B: dV += P^T dO and dK += dS^T Q over the BQ queries, this wave's output tiles
#pragma unroll
    for (int a = 0; a < C::TPW; ++a) {
      const int ot = wave * C::TPW + a;
      const int ktile = ot & 1, ctile = ot >> 1;  // keys 32 ktile .., channels 32 ctile ..
#pragma unroll
      for (int s = 0; s < BQ / 16; ++s) {
        const bf16x8 ap = tr_operand<C::PROWB, BK>(pt, 16 * s, 32 * ktile, lane);
        const bf16x8 as = tr_operand<C::PROWB, BK>(st, 16 * s, 32 * ktile, lane);
        const bf16x8 bg = tr_operand<C::ROWB, D>(gt, 16 * s, 32 * ctile, lane);
        const bf16x8 bq = tr_operand<C::ROWB, D>(qt, 16 * s, 32 * ctile, lane);
        acc_v[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bg, acc_v[a], 0, 0, 0);
        acc_k[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as, bq, acc_k[a], 0, 0, 0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // with no query block, the K/V copies are still in flight
  __syncthreads();

  // epilogue: dK then dV, each staged through LDS as [key][channel] rows
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int a = 0; a < C::TPW; ++a) {
      const int ot = wave * C::TPW + a;
      const int ktile = ot & 1, ctile = ot >> 1;
      const f32x16& acc = which == 0 ? acc_k[a] : acc_v[a];
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        // element i: channel 32 ctile + ln, key 32 ktile + 8 (i / 4) + 4 hf + i % 4
        const int key = 32 * ktile + 8 * (i >> 2) + 4 * hf + (i & 3);
        const int ch = 32 * ctile + ln;
        *reinterpret_cast<__attribute__((address_space(3))) __bf16*>(base + key * C::OROW + ch * 2) = (__bf16)acc[i];
        *reinterpret_cast<__attribute__((address_space(3))) __bf16*>(base + (key + 1) * C::OROW + ch * 2) =
            (__bf16)acc[i + 1];
      }
    }
    __syncthreads();
    char* obase = static_cast<char*>(which == 0 ? dk : dv) + head_off;
    constexpr int CH16 = D * 2 / 16;
    for (int e = threadIdx.x; e < BK * CH16; e += C::NT) {
      const int r = e / CH16, cc = e % CH16;
      const int key = kb * BK + r;
      if (key < N)
        *reinterpret_cast<u32x4*>(obase + (size_t)key * D * 2 + cc * 16) =
            *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(base + r * C::OROW + cc * 16);
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
         al((size_t)BH * N * 4);
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
  float* delta = reinterpret_cast<float*>(p);

  hipError_t e = launch_compact(mask, BH * nqb, nkb, ridx, rcnt, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mask_transpose_kernel, dim3((unsigned)((nkb + 63) / 64), (unsigned)((nqb + 63) / 64), (unsigned)BH),
                     dim3(256), 0, stream, mask, mask_t, nqb, nkb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_compact(mask_t, BH * nkb, nqb, cidx, ccnt, stream)) != hipSuccess) return e;
  const long long rows = (long long)BH * N;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const char*>(dout), static_cast<const char*>(o), delta, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const float c_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, BQ>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D, BQ>::NT), 0, stream, q, k, v,
                     dout, lse, delta, ridx, rcnt, N, nqb, nkb, scale, c_log2, dq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  using C = BCfg<D, BQ>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, BQ>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BQ>), dim3((unsigned)(BH * nkb)), dim3(C::NT), C::LDS, stream, q, k, v,
                     dout, lse, delta, cidx, ccnt, N, nqb, nkb, scale, c_log2, dk, dv);
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
