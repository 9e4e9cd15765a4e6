// Block-sparse flash attention forward (gfx950, bf16 MFMA, fp32 online softmax).
//
// Each query block attends only to the key blocks its mask row keeps: the scattered K/V blocks
// are loaded and the contiguous query block is computed densely against them (Sparse VideoGen2
// page, "2. 手法" C), and all queries of a block share the block's key support
// ("Partition the Support, Reconstruct the Residual" abstract). Softmax over the kept keys is
// computed in one streaming pass with a running maximum and sum (the flash-attention rewrite,
// exact up to rounding).
//
// Launch: one workgroup per (b, h, query block), BQ/32 waves; wave w owns queries 32w..32w+31.
// Per kept key block of 64 keys:
//   S^T (64 keys x 32 queries) = K_blk (LDS) x Q^T (registers)  : 2 x (D/16) MFMA 32x32x16
//   online softmax on S^T: every lane holds one query column and 32 of its 64 keys, so the row
//   max and row sum need one exchange with lane^32 (v_permlane32_swap)
//   O^T (D x 32) += V^T_blk (LDS) x P^T (registers)             : (D/32) x 4 MFMA 32x32x16
// P^T never leaves registers: the MFMA result layout of S^T is reused as the B operand of the
// PV product, so the V^T operand is read with its keys in that same order.
// Two kernels share this scheme. The bf16 kernel copies K/V blocks HBM -> LDS with DMA loads and
// reads V^T with transpose reads, in a two-stage software pipeline (scores of the next block
// overlap the softmax and P V of the current one). The fp32 kernel stages blocks through
// registers, rounding them to bf16, and writes V^T to LDS with its keys permuted.
#include <type_traits>

#include "attn_tiles.h"

namespace sa {

// ---------------------------------------------------------------- mask -> kept-block lists

// One wave per mask row: ascending kept indices and their count.
__global__ __launch_bounds__(256) void compact_kernel(const uint8_t* __restrict__ mask, int rows, int nkb,
                                                      int32_t* __restrict__ kidx, int32_t* __restrict__ kcnt) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t* m = mask + (size_t)row * nkb;
  int32_t* out = kidx + (size_t)row * nkb;
  int cnt = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    const bool f = j < nkb && m[j] != 0;
    const uint64_t b = __ballot(f);
    if (f) out[cnt + __popcll(b & ((1ull << lane) - 1ull))] = j;
    cnt += __popcll(b);
  }
  if (lane == 0) kcnt[row] = cnt;
}

// ---------------------------------------------------------------- attention

template <int DT, int D, int BQ>
struct AttnCfg {
  static constexpr int NW = BQ / 32;          // waves
  static constexpr int NT = NW * 64;          // threads
  static constexpr int ES = DT == kBF16 ? 2 : 4;
  static constexpr int KROW = D * 2 + 16;     // LDS bytes per K row (bf16, padded)
  static constexpr int VROW = BK * 2 + 16;    // LDS bytes per V^T row (bf16, padded)
  static constexpr int KBYTES = BK * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int TASKS = 2 * D;         // D tasks for V, D for K; 8 x 16-byte rows each
  static constexpr int TPT = (TASKS + NT - 1) / NT;
  static constexpr int OROW = D * ES + 16;    // LDS bytes per staged output row
  static_assert(NW * 32 * OROW <= 2 * BUF, "output staging must fit in the K/V buffers");
};

// Load 8 consecutive elements at `p` (element type DT) as 8 packed bf16 (round to nearest even).
template <int DT>
__device__ __forceinline__ uint4 load8_bf16(const char* p) {
  if constexpr (DT == kBF16) {
    return *reinterpret_cast<const uint4*>(p);
  } else {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    uint4 r;
    r.x = pack_bf16(__uint_as_float(a.x), __uint_as_float(a.y));
    r.y = pack_bf16(__uint_as_float(a.z), __uint_as_float(a.w));
    r.z = pack_bf16(__uint_as_float(b.x), __uint_as_float(b.y));
    r.w = pack_bf16(__uint_as_float(b.z), __uint_as_float(b.w));
    return r;
  }
}

// V^T rows in LDS hold their 64 keys with bits 2 and 3 of the key index swapped: lane half h
// of the PV MFMA then finds its 8 keys {16c + 4h + b, 16c + 8 + 4h + b : b < 4} as 16
// contiguous bytes at position 16c + 8h. Each V staging task loads exactly those 8 keys.

template <int DT, int D, int BQ>
__device__ __forceinline__ void stage_load(const char* __restrict__ kbase, const char* __restrict__ vbase, int kb,
                                           int N, uint4 (&st)[AttnCfg<DT, D, BQ>::TPT][8]) {
  using C = AttnCfg<DT, D, BQ>;
  constexpr int CPR = D / 8;  // 8-element chunks per token row
#pragma unroll
  for (int u = 0; u < C::TPT; ++u) {
    const int task = threadIdx.x + u * C::NT;
    if (task >= C::TASKS) continue;
    if (task < D) {
      // V task: 8 keys x 8 channels, keys chosen so they land on 8 adjacent V^T positions
      const int dch = task % CPR;
      const int ch = task / CPR;  // 0..7 = (c, h)
      const int c = ch >> 1, h = ch & 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb * BK + 16 * c + 4 * h + (e & 3) + 8 * (e >> 2);
        st[u][e] = (key >= 0 && key < N) ? load8_bf16<DT>(vbase + ((size_t)key * D + 8 * dch) * C::ES) : make_uint4(0, 0, 0, 0);
      }
    } else {
      // K task: 8 chunks of 8 channels, strided so a wave reads whole rows
      const int t = task - D;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int ci = t + r * D;
        const int row = ci / CPR, col = ci % CPR;
        const int key = kb * BK + row;
        st[u][r] = (key >= 0 && key < N) ? load8_bf16<DT>(kbase + ((size_t)key * D + 8 * col) * C::ES) : make_uint4(0, 0, 0, 0);
      }
    }
  }
}

template <int DT, int D, int BQ>
__device__ __forceinline__ void stage_store(char* __restrict__ buf, const uint4 (&st)[AttnCfg<DT, D, BQ>::TPT][8]) {
  using C = AttnCfg<DT, D, BQ>;
  constexpr int CPR = D / 8;
  char* kl = buf;
  char* vl = buf + C::KBYTES;
#pragma unroll
  for (int u = 0; u < C::TPT; ++u) {
    const int task = threadIdx.x + u * C::NT;
    if (task >= C::TASKS) continue;
    if (task < D) {
      const int dch = task % CPR;
      const int ch = task / CPR;
      const int c = ch >> 1, h = ch & 1;
      const uint32_t* w = reinterpret_cast<const uint32_t*>(&st[u][0]);  // w[4 e + m]: key e, channels 2m, 2m+1
#pragma unroll
      for (int s = 0; s < 8; ++s) {  // channel 8 dch + s
        const int m = s >> 1;
        uint32_t o[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const uint32_t a = w[4 * (2 * qq) + m], b = w[4 * (2 * qq + 1) + m];
          o[qq] = (s & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<uint4*>(vl + (8 * dch + s) * C::VROW + (16 * c + 8 * h) * 2) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
      const int t = task - D;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int ci = t + r * D;
        const int row = ci / CPR, col = ci % CPR;
        *reinterpret_cast<uint4*>(kl + row * C::KROW + col * 16) = st[u][r];
      }
    }
  }
}

template <int DT, int D, int BQ>
__global__ __launch_bounds__(BQ * 2) void attn_fwd_staged_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ kidx, const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float c_log2,
    void* __restrict__ o, float* __restrict__ lse) {
  using C = AttnCfg<DT, D, BQ>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

  const int tile = xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nqb;
  const int qb = tile - bh * nqb;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(kcnt[tile], 0), nkb);
  const int32_t* list = kidx + (size_t)tile * nkb;

  const size_t head_off = (size_t)bh * N * D * C::ES;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;

  // Q^T fragments: lane holds query 32 wave + ln, channels 16 s + 8 hf .. + 7.
  const int qrow = qb * BQ + wave * 32 + ln;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint4 x = qrow < N ? load8_bf16<DT>(qbase + ((size_t)qrow * D + 16 * s + 8 * hf) * C::ES) : make_uint4(0, 0, 0, 0);
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[r][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's partial sum (its 32 of the 64 keys of each block)
  const bool ragged = (N % BK) != 0;

  uint4 st[C::TPT][8];
  if (cnt > 0) {
    stage_load<DT, D, BQ>(kbase, vbase, min(max(list[0], 0), nkb - 1), N, st);
    stage_store<DT, D, BQ>(smem, st);
  }
  __syncthreads();

  for (int t = 0; t < cnt; ++t) {
    const int kb = min(max(list[t], 0), nkb - 1);  // clamped: no load leaves K or V
    if (t + 1 < cnt) stage_load<DT, D, BQ>(kbase, vbase, min(max(list[t + 1], 0), nkb - 1), N, st);
    const char* kl = smem + (t & 1) * C::BUF;
    const char* vl = kl + C::KBYTES;

    // S^T = K Q^T for keys 0..31 (s0) and 32..63 (s1)
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kl + ln * C::KROW + (16 * s + 8 * hf) * 2);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kl + (32 + ln) * C::KROW + (16 * s + 8 * hf) * 2);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
    }
    // element i of s0 is key 8 (i / 4) + 4 hf + i % 4; of s1 the same plus 32
    if (ragged && kb == nkb - 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (key >= N) s0[i] = -INFINITY;
        if (key + 32 >= N) s1[i] = -INFINITY;
      }
    }
    float mx = s0[0];
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = partner32_max(mx);
    const float m_new = fmaxf(m_run, mx * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c_log2, -m_new));
      s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c_log2, -m_new));
      rs += s0[i] + s1[i];
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int r = 0; r < D / 32; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[r][i] *= alpha;

    // P^T as the B operand: key chunk c = 2 t + u takes elements 8u .. 8u+7 of tile t
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint4 a, b;
      a.x = pack_bf16(s0[8 * u + 0], s0[8 * u + 1]);
      a.y = pack_bf16(s0[8 * u + 2], s0[8 * u + 3]);
      a.z = pack_bf16(s0[8 * u + 4], s0[8 * u + 5]);
      a.w = pack_bf16(s0[8 * u + 6], s0[8 * u + 7]);
      b.x = pack_bf16(s1[8 * u + 0], s1[8 * u + 1]);
      b.y = pack_bf16(s1[8 * u + 2], s1[8 * u + 3]);
      b.z = pack_bf16(s1[8 * u + 4], s1[8 * u + 5]);
      b.w = pack_bf16(s1[8 * u + 6], s1[8 * u + 7]);
      pb[u] = __builtin_bit_cast(bf16x8, a);
      pb[2 + u] = __builtin_bit_cast(bf16x8, b);
    }
#pragma unroll
    for (int r = 0; r < D / 32; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vl + (32 * r + ln) * C::VROW + (16 * c + 8 * hf) * 2);
        oacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c], oacc[r], 0, 0, 0);
      }

    if (t + 1 < cnt) stage_store<DT, D, BQ>(smem + ((t + 1) & 1) * C::BUF, st);
    __syncthreads();
  }

  // epilogue: O = O^T / l, staged through LDS for row-contiguous stores
  const float l_tot = partner32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  char* ol = smem + wave * 32 * C::OROW;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * r + 8 * a + 4 * hf;  // channels ch .. ch+3 of query ln
      const float x0 = oacc[r][4 * a] * inv, x1 = oacc[r][4 * a + 1] * inv;
      const float x2 = oacc[r][4 * a + 2] * inv, x3 = oacc[r][4 * a + 3] * inv;
      if constexpr (DT == kBF16) {
        *reinterpret_cast<uint2*>(ol + ln * C::OROW + ch * 2) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
      } else {
        *reinterpret_cast<float4*>(ol + ln * C::OROW + ch * 4) = make_float4(x0, x1, x2, x3);
      }
    }
  __syncthreads();
  constexpr int CH16 = D * C::ES / 16;  // 16-byte chunks per output row
  char* obase = static_cast<char*>(o) + head_off;
  for (int e = lane; e < 32 * CH16; e += 64) {
    const int r = e / CH16, cc = e % CH16;
    const int qr = qb * BQ + wave * 32 + r;
    if (qr < N)
      *reinterpret_cast<uint4*>(obase + (size_t)qr * D * C::ES + cc * 16) =
          *reinterpret_cast<const uint4*>(ol + r * C::OROW + cc * 16);
  }
  if (lse != nullptr && hf == 0 && qrow < N) {
    lse[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------- window-transposed rows

// Token of row s of the window-transposed order, whose runs of nw = N / w rows hold the tokens at
// one position inside their windows of w tokens: (s mod nw) w + s / nw.
__device__ __forceinline__ int wt_token(int s, int nw, int w) { return (s % nw) * w + s / nw; }

// dma_tile for rows 64 kb .. 64 kb + 63 of the window-transposed order. With nw >= 64 a block
// spans at most two runs: row i is token ((r0 + i) mod nw) w + p0 (+1 after the wrap), with
// p0, r0 the run and offset of the block's first row. Rows past N are clamped to row N - 1.
template <int D, int BQ>
__device__ __forceinline__ void dma_tile_wt(const char* __restrict__ base, int kb, int N, int nw, int w, int wave,
                                            const uint32_t (&off)[DCfg<D, BQ>::PER_WAVE], lchar* dst) {
  using C = DCfg<D, BQ>;
  const int s0 = kb * BK;
  const int p0 = s0 / nw, r0 = s0 - p0 * nw;
  const bool ragged = s0 + BK > N;
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) {
    const int i = (int)(off[u] / C::ROWB);
    const uint32_t choff = off[u] % C::ROWB;
    int tok;
    if (!ragged) {
      const int x = r0 + i;
      const bool wrap = x >= nw;
      tok = (wrap ? x - nw : x) * w + p0 + (wrap ? 1 : 0);
    } else {
      tok = wt_token(min(s0 + i, N - 1), nw, w);
    }
    // a 32-bit lane offset from the uniform head base (one head's rows stay below 4 GiB), kept
    // 32-bit by the empty asm so that the copy takes the base from SGPRs
    uint32_t o = (uint32_t)tok * C::ROWB + choff;
    asm volatile("" : "+v"(o));
    __builtin_amdgcn_global_load_lds(base + o, dst + (wave * C::PER_WAVE + u) * 1024, 16, 0, 0);
  }
}

// ---------------------------------------------------------------- bf16 kernel

// Main loop as a two-stage software pipeline over the kept list. Step t computes the scores of
// block t + 1 on the matrix cores while the vector units turn the scores of block t into P and
// the matrix cores then add P V of block t: the three are independent, so they share one basic
// block and the compiler interleaves them. K therefore runs one block ahead of V in LDS: at step
// t, K(t+1) and V(t) are resident and the DMA fills K(t+2) and V(t+1) into the buffers that
// K(t) and V(t-1) left. The running maximum is raised after P V of block t, from the scores of
// block t + 1, so the rare rescale branch closes the step instead of splitting it.
//
// WT: the rows (queries and keys) are those of the window-transposed order (windows of wt_w
// tokens, wt_nw = N / wt_w >= 64 of them), read from and written to Q, K, V, O and LSE in the
// original token order.
template <int D, int BQ, bool WT = false>
__global__ __launch_bounds__(BQ * 2, 2) void attn_fwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ kidx, const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float c_log2,
    void* __restrict__ o, float* __restrict__ lse, int wt_nw, int wt_w) {
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char kbuf_[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf_[2 * C::TILE];
  lchar* const kb0 = (lchar*)kbuf_;
  lchar* const kb1 = kb0 + C::TILE;
  lchar* const vb0 = (lchar*)vbuf_;
  lchar* const vb1 = vb0 + C::TILE;

  const int tile = xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nqb;
  const int qb = tile - bh * nqb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: SGPR
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(kcnt[tile], 0), nkb);
  const int32_t* list = kidx + (size_t)tile * nkb;
  // list entries are clamped to [0, nKB) so that no load leaves K or V
  auto blk = [&](int i) { return min(max(list[i], 0), nkb - 1); };

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;

  uint32_t doff[C::PER_WAVE];
  dma_offsets<D, BQ>(wave, lane, doff);
  // K or V block kb into dst: contiguous rows, or rows of the window-transposed order
  auto copy = [&](const char* base, int kb, lchar* dst) {
    if constexpr (WT) dma_tile_wt<D, BQ>(base, kb, N, wt_nw, wt_w, wave, doff, dst);
    else dma_tile<D, BQ>(base, kb, N, wave, lane, doff, dst);
  };
  if (cnt > 0) {
    copy(kbase, blk(0), kb0);
    copy(vbase, blk(0), vb0);
  }
  if (cnt > 1) copy(kbase, blk(1), kb1);

  // Q^T fragments (B operand of S^T): query 32 wave + ln, channels 16 s + 8 hf .. + 7
  const int qrow = qb * BQ + wave * 32 + ln;
  const bool qvalid = qrow < N;
  const int qtok = WT && qvalid ? wt_token(qrow, wt_nw, wt_w) : qrow;  // the row's token
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint4 x = qvalid ? *reinterpret_cast<const uint4*>(qbase + ((size_t)qtok * D + 16 * s + 8 * hf) * 2)
                           : make_uint4(0, 0, 0, 0);
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }

  // lane-constant LDS offsets of the K and V^T fragments within a tile
  int koff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = ln * C::ROWB + (((2 * s + hf) ^ sw) << 4);
  }
  int voff[D / 32][2];
  {
    const int i16 = lane & 15, grp = lane >> 4;
    const int half = grp >> 1, gsub = grp & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * u + 4 * half + (i16 >> 2);
      const int sw = kv_swz<D>(row);
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
        const int chunk = 4 * r + 2 * gsub + ((i16 & 3) >> 1);
        voff[r][u] = row * C::ROWB + ((chunk ^ sw) << 4) + (i16 & 1) * 8;
      }
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[r][i] = 0.f;
  float m_run = -INFINITY;  // running max in the scaled log2 domain, shared by the lane pair
  float l_run = 0.f;        // this lane's part of the running sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T of the key block in kt (64 keys x 32 queries as two 32 x 32 tiles)
  auto scores = [&](const lchar* kt, f32x16 (&sc)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[0][i] = 0.f;
      sc[1][i] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s] + 32 * C::ROWB);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], sc[1], 0, 0, 0);
    }
  };
  // keys past N (only in the ragged last key block kb) get score -inf
  auto mask_tail = [&](f32x16 (&sc)[2], int kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (key >= N) sc[0][i] = -INFINITY;
      if (key + 32 >= N) sc[1][i] = -INFINITY;
    }
  };
  // maximum over the block's 64 keys of each query, scaled to the log2 domain
  auto block_max = [&](const f32x16 (&sc)[2]) {
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m4[c] = fmaxf(sc[0][c], sc[1][c]);
#pragma unroll
    for (int i = 4; i < 16; ++i) m4[i & 3] = fmaxf(fmaxf(m4[i & 3], sc[0][i]), sc[1][i]);
    const float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    return partner32_max(mx) * c_log2;
  };
  // Rescale only when some row's maximum grew by more than 2^8: until then exp2 values stay
  // below 256, and O and l keep a common, slightly stale reference, which divides out exactly.
  auto raise_max = [&](float mx) {
    if (__ballot(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < D / 32; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[r][i] *= alpha;
      m_run = m_new;
    }
  };
  // P^T of the block (B operand of the PV product) and its row sum; key chunk c = 2 t + u takes
  // elements 8u .. 8u+7 of tile t, and the row sum adds the same bf16 values the product uses.
  // Then O^T += V^T P^T with V^T fragments read from the tile vt by transpose reads.
  auto accumulate = [&](const f32x16 (&sc)[2], lchar* vt) {
    bf16x8 pb[4];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sc[0][8 * u + 2 * e], c_log2, -m_run)),
                          __builtin_amdgcn_exp2f(fmaf(sc[0][8 * u + 2 * e + 1], c_log2, -m_run)));
        w1[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sc[1][8 * u + 2 * e], c_log2, -m_run)),
                          __builtin_amdgcn_exp2f(fmaf(sc[1][8 * u + 2 * e + 1], c_log2, -m_run)));
        rs[(e & 1) * 2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0[e]), ones, rs[(e & 1) * 2], false);
        rs[(e & 1) * 2 + 1] =
            __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1[e]), ones, rs[(e & 1) * 2 + 1], false);
      }
      pb[u] = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      pb[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) v4i16*>(vt + voff[r][0] + c * 16 * C::ROWB));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) v4i16*>(vt + voff[r][1] + c * 16 * C::ROWB));
        const v8i16 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pb[c], oacc[r], 0, 0, 0);
      }
  };

  const bool ragged_last = cnt > 0 && (N % BK) != 0 && blk(cnt - 1) == nkb - 1;
  // Step t. NEXT: 0 = no block t + 1 (last step), 1 = full block t + 1, 2 = ragged block t + 1.
  // kn / vc hold K(t+1) / V(t); kf / vf receive K(t+2) / V(t+1).
  auto step = [&](int t, const f32x16 (&sc)[2], f32x16 (&sn)[2], const lchar* kn, lchar* vc, lchar* kf, lchar* vf,
                  auto next_tag) {
    constexpr int NEXT = decltype(next_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K(t+1) and V(t) are resident; every wave is done with K(t) and V(t-1)
    // the DMA for K(t+2) and V(t+1) is issued behind the score MFMAs, so that the waves released
    // by the barrier start on the matrix cores instead of queueing their copies first
    const int blk2 = t + 2 < cnt ? blk(t + 2) : -1;
    const int blk1 = t + 1 < cnt ? blk(t + 1) : -1;
    if constexpr (NEXT != 0) {
      scores(kn, sn);
      if constexpr (NEXT == 2) mask_tail(sn, blk1);
    }
    if (blk2 >= 0) copy(kbase, blk2, kf);
    if (blk1 >= 0) copy(vbase, blk1, vf);
    accumulate(sc, vc);
    if constexpr (NEXT != 0) raise_max(block_max(sn));
  };

  using last = std::integral_constant<int, 0>;
  using full = std::integral_constant<int, 1>;
  using rag = std::integral_constant<int, 2>;
  if (cnt > 0) {
    f32x16 sa[2], sb[2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    scores(kb0, sa);
    if (ragged_last && cnt == 1) mask_tail(sa, blk(0));
    raise_max(block_max(sa));
    // steps whose next block is a full one, unrolled by two so that S alternates between sa
    // and sb and the buffers between their even / odd roles without copies
    const int nfull = ragged_last ? cnt - 2 : cnt - 1;
    int t = 0;
    for (; t + 1 < nfull; t += 2) {
      step(t, sa, sb, kb1, vb0, kb0, vb1, full{});
      step(t + 1, sb, sa, kb0, vb1, kb1, vb0, full{});
    }
    if (t < nfull) {
      step(t, sa, sb, kb1, vb0, kb0, vb1, full{});
      ++t;
#pragma unroll
      for (int h = 0; h < 2; ++h) sa[h] = sb[h];
    }
    // at most two steps remain: one whose next block is the ragged last block, and the last one
    const bool odd = (t & 1) != 0;
    if (t + 1 < cnt) {
      step(t, sa, sb, odd ? kb0 : kb1, odd ? vb1 : vb0, odd ? kb1 : kb0, odd ? vb0 : vb1, rag{});
      ++t;
#pragma unroll
      for (int h = 0; h < 2; ++h) sa[h] = sb[h];
    }
    const bool odd2 = (t & 1) != 0;
    step(t, sa, sb, odd2 ? kb0 : kb1, odd2 ? vb1 : vb0, odd2 ? kb1 : kb0, odd2 ? vb0 : vb1, last{});
  }
  __syncthreads();

  // epilogue: O = O^T / l, staged through LDS (two waves per buffer pair) for row-contiguous stores
  const float l_tot = partner32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  lchar* ol = ((wave & 1) ? vb0 : kb0) + (wave >> 1) * 32 * C::OROW;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * r + 8 * a + 4 * hf;
      const u32x2 w = {pack_bf16(oacc[r][4 * a] * inv, oacc[r][4 * a + 1] * inv),
                       pack_bf16(oacc[r][4 * a + 2] * inv, oacc[r][4 * a + 3] * inv)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(ol + ln * C::OROW + ch * 2) = w;
    }
  __syncthreads();
  constexpr int CH16 = D * 2 / 16;
  char* obase = static_cast<char*>(o) + head_off;
#pragma unroll
  for (int e = lane; e < 32 * CH16; e += 64) {
    const int r = e / CH16, cc = e % CH16;
    const int qr = qb * BQ + wave * 32 + r;
    if (qr < N) {
      const int tok = WT ? wt_token(qr, wt_nw, wt_w) : qr;
      *reinterpret_cast<u32x4*>(obase + (size_t)tok * D * 2 + cc * 16) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(ol + r * C::OROW + cc * 16);
    }
  }
  if (lse != nullptr && hf == 0 && qvalid) {
    lse[(size_t)bh * N + qtok] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_compact(const uint8_t* mask, int rows, int nkb, int32_t* kidx, int32_t* kcnt, hipStream_t stream) {
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, mask, rows, nkb, kidx, kcnt);
  return hipGetLastError();
}

template <int DT, int D, int BQ>
static hipError_t launch_attn_t(const void* q, const void* k, const void* v, const int32_t* kidx,
                                const int32_t* kcnt, int BH, int N, int nqb, int nkb, float c_log2, void* o,
                                float* lse, hipStream_t stream) {
  if constexpr (DT == kBF16) {
    hipLaunchKernelGGL((attn_fwd_kernel<D, BQ>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D, BQ>::NT), 0, stream,
                       q, k, v, kidx, kcnt, N, nqb, nkb, c_log2, o, lse, 0, 0);
  } else {
    hipLaunchKernelGGL((attn_fwd_staged_kernel<DT, D, BQ>), dim3((unsigned)(BH * nqb)), dim3(AttnCfg<DT, D, BQ>::NT),
                       0, stream, q, k, v, kidx, kcnt, N, nqb, nkb, c_log2, o, lse);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const void* q, const void* k, const void* v, int dtype, const int32_t* kidx,
                       const int32_t* kcnt, int BH, int N, int d, int Bq, double scale, void* o, float* lse,
                       hipStream_t stream) {
  const int nqb = (N + Bq - 1) / Bq;
  const int nkb = (N + BK - 1) / BK;
  const float c_log2 = (float)(scale * 1.4426950408889634);
#define SA_ATTN_CASE(DT_, D_, BQ_)                                                               \
  if (dtype == DT_ && d == D_ && Bq == BQ_)                                                      \
    return launch_attn_t<DT_, D_, BQ_>(q, k, v, kidx, kcnt, BH, N, nqb, nkb, c_log2, o, lse, stream);
  SA_ATTN_CASE(kBF16, 128, 128)
  SA_ATTN_CASE(kBF16, 128, 64)
  SA_ATTN_CASE(kBF16, 64, 128)
  SA_ATTN_CASE(kBF16, 64, 64)
  SA_ATTN_CASE(kF32, 128, 128)
  SA_ATTN_CASE(kF32, 128, 64)
  SA_ATTN_CASE(kF32, 64, 128)
  SA_ATTN_CASE(kF32, 64, 64)
#undef SA_ATTN_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_window(const void* q, const void* k, const void* v, const int32_t* kidx, const int32_t* kcnt,
                              int BH, int N, int d, int Bq, double scale, int window, void* o, float* lse,
                              hipStream_t stream) {
  const int nqb = (N + Bq - 1) / Bq;
  const int nkb = (N + BK - 1) / BK;
  const float c_log2 = (float)(scale * 1.4426950408889634);
  const int nw = N / window;
#define SA_WT_CASE(D_, BQ_)                                                                                  \
  if (d == D_ && Bq == BQ_) {                                                                                \
    hipLaunchKernelGGL((attn_fwd_kernel<D_, BQ_, true>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D_, BQ_>::NT), 0, \
                       stream, q, k, v, kidx, kcnt, N, nqb, nkb, c_log2, o, lse, nw, window);               \
    return hipGetLastError();                                                                                \
  }
  SA_WT_CASE(128, 128)
  SA_WT_CASE(128, 64)
  SA_WT_CASE(64, 128)
  SA_WT_CASE(64, 64)
#undef SA_WT_CASE
  return hipErrorInvalidValue;
}

}  // namespace sa
