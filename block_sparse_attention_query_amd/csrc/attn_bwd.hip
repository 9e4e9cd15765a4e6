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

// ---------------------------------------------------------------- dQ

// One workgroup per (b, h, query block), BQ / 32 waves of 32 queries, walking the kept list:
//   S^T = K Q^T, dP^T = V dO^T (A operands: 16-byte row reads of the K and V tiles),
//   dS^T = P^T * (dP^T - D) * scale in registers (the B operand layout of the forward's P^T),
//   dQ^T += K^T dS^T (K^T by transpose reads of the K tile).
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
  static constexpr int LDS = 2 * BUF;
  static constexpr int OROW = D * 2 + 16;    // bytes per staged output row
  static_assert(64 * OROW <= LDS, "output staging must fit");
};

// Copies of the 64-row tile sb (token rows 64 sb .. + 63) of a [N][D] bf16 tensor into a
// swizzled LDS tile by the two waves: instruction u of wave w fills the 1 KiB stretch
// m = w PW + u; lane i fills its bytes 16 i .. + 15, i.e. row (1024 m + 16 i) / ROWB and swizzled
// chunk slot ((1024 m + 16 i) % ROWB) / 16, which holds logical chunk slot ^ kv_swz(row).
// kv_dma_offsets gives each lane's byte offsets inside a tile; rows past N (only in the last
// tile) are clamped to N - 1.
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

template <int D>
__device__ __forceinline__ void kv_dma(const char* __restrict__ base, int sb, int N, int wave, int lane,
                                       const uint32_t* off, lchar* dst) {
  constexpr int ROWB = KVDma<D>::ROWB, PW = KVDma<D>::PW;
  const char* blk = base + (size_t)sb * 64 * ROWB;
  // The empty asm marks each 32-bit offset as redefined at its use, so that the compiler cannot
  // hoist 64-bit zero-extended copies of the offsets out of the walk; the copy then takes the
  // uniform base in SGPRs and the 32-bit offset in one VGPR.
  if (sb * 64 + 64 <= N) {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      uint32_t o = off[u];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(blk + o, dst + (wave * PW + u) * 1024, 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int row = ((wave * PW + u) * 1024 + lane * 16) / ROWB;
      const int over = sb * 64 + row - (N - 1);
      uint32_t o = over > 0 ? off[u] - (uint32_t)(over * ROWB) : off[u];
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(blk + o, dst + (wave * PW + u) * 1024, 16, 0, 0);
    }
  }
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
  extern __shared__ __attribute__((aligned(1024))) char lds_[];
  lchar* const base = (lchar*)lds_;

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
  // copies of step t into buffer t & 1: both tiles, then wave 0 the LSE and wave 1 the D values
#define SA_KV_ISSUE(T_)                                                                                  \
  {                                                                                                      \
    const int t_ = (T_);                                                                                 \
    const int sb_ = min(max(list[t_ / SPB], 0), nqb - 1) * SPB + t_ % SPB;                               \
    lchar* b_ = base + (t_ & 1) * C::BUF;                                                                \
    kv_dma<D>(qbase, sb_, N, wave, lane, doff, b_);                                                      \
    kv_dma<D>(gbase, sb_, N, wave, lane, doff, b_ + C::OFF_G);                                           \
    __builtin_amdgcn_global_load_lds((wave == 0 ? l2base : dlbase) + sb_ * 64 + lane, b_ + C::OFF_L + wave * 256, \
                                     4, 0, 0);                                                           \
  }
  if (T > 0) SA_KV_ISSUE(0)

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

  f32x16 acc_k[D / 32], acc_v[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc_k[c][i] = 0.f;
      acc_v[c][i] = 0.f;
    }

  for (int t = 0; t < T; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // step t is resident; both waves are done with the buffer of step t - 1
    if (t + 1 < T) SA_KV_ISSUE(t + 1)
    const lchar* qt = base + (t & 1) * C::BUF;
    const lchar* gt = qt + C::OFF_G;

    // S = Q K^T and dP = dO V^T for queries 32 h .. 32 h + 31 of the step: element i of lane
    // (ln, hf) is key 32 w + ln, query 32 h + 8 (i / 4) + 4 hf + i % 4. The A operands of
    // channel slice s + 1 are read while the products of slice s run.
    f32x16 sc[2], dp[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[h][i] = 0.f;
        dp[h][i] = 0.f;
      }
    bf16x8 cur[4], nxt[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      cur[2 * h] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qt + roff[0] + 32 * h * C::ROWB);
      cur[2 * h + 1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(gt + roff[0] + 32 * h * C::ROWB);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 1 < D / 16) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          nxt[2 * h] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(qt + roff[s + 1] + 32 * h * C::ROWB);
          nxt[2 * h + 1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(gt + roff[s + 1] + 32 * h * C::ROWB);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sc[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[2 * h], kf[s], sc[h], 0, 0, 0);
        dp[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur[2 * h + 1], vf[s], dp[h], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
    }

    // the first transposed operands of the dV / dK products, read ahead of the softmax work
    bf16x8 cg = tr_operand<C::ROWB, D>(gt, 0, 0, lane), cq = tr_operand<C::ROWB, D>(qt, 0, 0, lane);

    // P = exp(s - LSE) and dS = P (dP - D) scale, packed to bf16 as A operands: run u of half h
    // takes elements 8 u .. 8 u + 7, i.e. queries 32 h + 16 u + 8 (e / 4) + 4 hf + e % 4
    bf16x8 pa[2][2], sa[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t wp[4], ws[4];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int qi = 32 * h + 16 * u + 8 * g + 4 * hf;  // four consecutive queries
          const f32x4 lv = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(qt + C::OFF_L + qi * 4);
          const f32x4 dv4 = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(qt + C::OFF_D + qi * 4);
          float pv[4], sv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * u + 4 * g + e;
            pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[h][i], c_log2, -lv[e]));
            sv[e] = pv[e] * (dp[h][i] - dv4[e]) * scale;
          }
          wp[2 * g] = pack_bf16(pv[0], pv[1]);
          wp[2 * g + 1] = pack_bf16(pv[2], pv[3]);
          ws[2 * g] = pack_bf16(sv[0], sv[1]);
          ws[2 * g + 1] = pack_bf16(sv[2], sv[3]);
        }
        pa[h][u] = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
        sa[h][u] = __builtin_bit_cast(bf16x8, make_uint4(ws[0], ws[1], ws[2], ws[3]));
      }
    __builtin_amdgcn_sched_barrier(0);

    // dV += P^T dO and dK += dS^T Q over the step's 64 queries, item j = (h, u, channel tile c);
    // the operands of item j + 1 are read while the products of item j run
    constexpr int NC = D / 32;
#pragma unroll
    for (int j = 0; j < 4 * NC; ++j) {
      const int h = j / (2 * NC), u = (j / NC) & 1, c = j % NC;
      bf16x8 ng = cg, nq = cq;
      if (j + 1 < 4 * NC) {
        const int h1 = (j + 1) / (2 * NC), u1 = ((j + 1) / NC) & 1, c1 = (j + 1) % NC;
        ng = tr_operand<C::ROWB, D>(gt, 32 * h1 + 16 * u1, 32 * c1, lane);
        nq = tr_operand<C::ROWB, D>(qt, 32 * h1 + 16 * u1, 32 * c1, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      acc_v[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[h][u], cg, acc_v[c], 0, 0, 0);
      acc_k[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa[h][u], cq, acc_k[c], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      cg = ng;
      cq = nq;
    }
  }
#undef SA_KV_ISSUE
  __syncthreads();  // every wave is done with the last step's buffer

  // epilogue: dK then dV, staged through LDS as [key][channel] rows. Element i of tile c: channel
  // 32 c + ln, key 32 w + 8 (i / 4) + 4 hf + i % 4
  for (int which = 0; which < 2; ++which) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const f32x16& acc = which == 0 ? acc_k[c] : acc_v[c];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 32 * wave + 8 * (i >> 2) + 4 * hf + (i & 3);
        *reinterpret_cast<__attribute__((address_space(3))) __bf16*>(base + kr * C::OROW + (32 * c + ln) * 2) =
            (__bf16)acc[i];
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
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D, BQ>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, BQ>), dim3((unsigned)(BH * nkb)), dim3(C::NT), C::LDS, stream, q, k, v,
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
