// Block-sparse flash attention forward (gfx950: bf16 MFMA for bf16 inputs, fp32 MFMA for fp32 inputs, fp32 online softmax).
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
// The bf16 kernel copies K/V blocks HBM -> LDS with DMA loads and reads V^T with transpose reads,
// in a two-stage software pipeline (scores of the next block overlap the softmax and P V of the
// current one). fp32 inputs run the same scheme on the fp32 matrix instruction, with nothing
// rounded to bf16.
#include <type_traits>

#include "attn_tiles.h"

namespace sa {

constexpr int kPairMaxKB = 4096;  // key blocks per head of the paired 64-query walk

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

// ---------------------------------------------------------------- fp32 kernel

// fp32 inputs keep their precision: both products run on the fp32 matrix instruction
// (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation) and P stays fp32, so no input or
// probability is rounded to bf16. Keys pass through LDS 32 at a time (half a key block); K rows
// are padded by one float so that the 32 rows of an operand read fall in distinct banks.
// Operand layout of the 32x32x2 product: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32];
// its result register i holds C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32], the layout of the bf16
// 32x32x16 product above. So S^T (32 keys x 32 queries) = K Q^T leaves lane (ln, hf) the scores of
// query ln against keys 8 (i / 4) + 4 hf + i % 4, and step i of O^T += V^T P^T pairs K index hf
// with exactly that key on both operands.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ kidx, const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float c_log2,
    float* __restrict__ o, float* __restrict__ lse, const int32_t* __restrict__ row_order) {
  constexpr int NT = BQ * 2;
  constexpr int HK = 32;     // keys per LDS stage
  constexpr int KP = D + 1;  // padded K row (floats)
  __shared__ float ks[HK * KP];
  __shared__ __attribute__((aligned(16))) float vs[HK * D];

  const int tile = row_order ? min(max(row_order[blockIdx.x], 0), (int)gridDim.x - 1)
                            : xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nqb;
  const int qb = tile - bh * nqb;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  const int cnt = min(max(kcnt[tile], 0), nkb);
  const int32_t* list = kidx + (size_t)tile * nkb;
  const size_t head = (size_t)bh * N * D;
  const float* qh = q + head;
  const float* kh = k + head;
  const float* vh = v + head;

  const int qrow = qb * BQ + wave * 32 + ln;
  const bool qvalid = qrow < N;
  float qf[D / 2];  // B operand of step c: Q[qrow][2 c + hf]
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = qvalid ? qh[(size_t)qrow * D + 2 * c + hf] : 0.f;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[r][i] = 0.f;
  float m_run = -INFINITY;  // running max (scaled log2 domain), shared by the lane pair
  float l_run = 0.f;        // this lane's part of the running sum

  for (int t = 0; t < cnt; ++t) {
    const int kb = min(max(list[t], 0), nkb - 1);  // clamped: no load leaves K or V
    for (int h = 0; h < 2; ++h) {
      const int key0 = kb * BK + h * HK;
      if (key0 >= N) break;  // the second half of a ragged last block can be empty
      __syncthreads();       // every wave is done with the previous stage
      for (int e = threadIdx.x; e < HK * D / 4; e += NT) {
        const int r = e / (D / 4), c4 = (e % (D / 4)) * 4;
        const int key = key0 + r;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < N) {
          kv = *reinterpret_cast<const float4*>(kh + (size_t)key * D + c4);
          vv = *reinterpret_cast<const float4*>(vh + (size_t)key * D + c4);
        }
        float* kd = ks + r * KP + c4;
        kd[0] = kv.x;
        kd[1] = kv.y;
        kd[2] = kv.z;
        kd[3] = kv.w;
        *reinterpret_cast<float4*>(vs + r * D + c4) = vv;
      }
      __syncthreads();

      f32x16 sc;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 2; ++c)
        sc = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[ln * KP + 2 * c + hf], qf[c], sc, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (key0 + 8 * (i >> 2) + 4 * hf + (i & 3) >= N) sc[i] = -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      // key0 < N is held by lane hf = 0, register 0, so the pair's maximum is finite
      const float m_new = fmaxf(m_run, partner32_max(mx) * c_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c_log2, -m_new));
        rs += sc[i];
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[r][i] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
          oacc[r] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + 32 * r + ln], sc[i], oacc[r], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: lane (ln, hf) holds channels 32 r + 8 a + 4 hf .. + 3 of query ln
  const float l_tot = partner32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    float* orow = o + head + (size_t)qrow * D;
#pragma unroll
    for (int r = 0; r < D / 32; ++r)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<float4*>(orow + 32 * r + 8 * a + 4 * hf) =
            make_float4(oacc[r][4 * a] * inv, oacc[r][4 * a + 1] * inv, oacc[r][4 * a + 2] * inv,
                        oacc[r][4 * a + 3] * inv);
    if (lse != nullptr && hf == 0)
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

// K or V block kb into dst: contiguous rows (dma_tile) or rows of the window-transposed order.
template <int D, int BQ, bool WT>
__device__ __forceinline__ void copy_tile(const char* __restrict__ base, int kb, int N, int nw, int w, int wave,
                                          int lane, const uint32_t (&off)[DCfg<D, BQ>::PER_WAVE], lchar* dst) {
  if constexpr (WT) dma_tile_wt<D, BQ>(base, kb, N, nw, w, wave, off, dst);
  else dma_tile_rsrc<D, BQ>(base, kb, N, wave, off, dst);
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
//
// WIN: no kept lists. Row r attends to exactly the rows of its own window of `win` consecutive
// rows (windows [c win, (c + 1) win), the last one cut at N), the SQuad local pass; with WT the
// rows are those of the window-transposed order, where the tokens at one position inside their
// windows form runs of wt_nw rows, so win = wt_nw gives the SQuad global pass. A query block
// visits the contiguous range of key blocks that covers its rows' windows, and keys outside a
// query's window get score -inf element by element.
//
// PAIR (BQ = 128): the rows are those of 64-query blocks, taken two at a time. Workgroup (b, h, q)
// computes 64-query rows 2 q (waves 0, 1) and 2 q + 1 (waves 2, 3) of the nqb64 rows per head, and
// walks the union of their kept lists (at most kPairMaxKB key blocks per row), every union entry
// carrying whether each row keeps it. A wave scores a block its row does not keep at -inf, which
// adds exactly nothing to its softmax, so each row's result is bit-identical to that of the
// one-row walk over its own list, while one 4-wave workgroup of 64 KiB of LDS serves 128 queries
// (two per CU, two waves per SIMD) instead of a 2-wave workgroup serving 64 (one wave per SIMD).
template <int D, int BQ, bool WT = false, bool WIN = false, bool PAIR = false>
__global__ __launch_bounds__(BQ * 2, 2) void attn_fwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const int32_t* __restrict__ kidx, const int32_t* __restrict__ kcnt, int N, int nqb, int nkb, float c_log2,
    void* __restrict__ o, float* __restrict__ lse, int wt_nw, int wt_w, int win,
    const int32_t* __restrict__ row_order, int nqb64 = 0) {
  static_assert(!PAIR || (BQ == 128 && !WT && !WIN), "the paired walk runs two 64-query rows per 4-wave workgroup");
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char kbuf_[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf_[2 * C::TILE];
  lchar* const kb0 = (lchar*)kbuf_;
  lchar* const kb1 = kb0 + C::TILE;
  lchar* const vb0 = (lchar*)vbuf_;
  lchar* const vb1 = vb0 + C::TILE;

  // row_order (optional): the row of each workgroup; entries are clamped to the grid
  const int tile = row_order ? min(max(row_order[blockIdx.x], 0), (int)gridDim.x - 1)
                            : xcd_chunk_row(blockIdx.x, gridDim.x);
  const int bh = tile / nqb;
  const int qb = tile - bh * nqb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: SGPR
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  int cnt, kb_first = 0;
  const int32_t* list = kidx + (size_t)tile * nkb;
  // PAIR: the union list in LDS, entries kb | (row 2q keeps it) << 14 | (row 2q + 1 keeps it) << 15
  const __attribute__((address_space(3))) uint16_t* ulist = nullptr;
  const int half = wave >> 1;  // PAIR: the row of this wave within the pair
  int pair_cnt = 0;
  if constexpr (PAIR) {
    __shared__ uint32_t pmask[2][kPairMaxKB / 32];
    __shared__ uint16_t ul_[kPairMaxKB];
    __shared__ int ucnt;
    const int nw = (nkb + 31) >> 5;
    const int rA = 2 * qb, rB = 2 * qb + 1;
    const int32_t* la = kidx + ((size_t)bh * nqb64 + rA) * nkb;
    const int32_t* lb = kidx + ((size_t)bh * nqb64 + rB) * nkb;
    const int ca = min(max(kcnt[(size_t)bh * nqb64 + rA], 0), nkb);
    const int cb = rB < nqb64 ? min(max(kcnt[(size_t)bh * nqb64 + rB], 0), nkb) : 0;
    for (int i = threadIdx.x; i < 2 * nw; i += BQ * 2) pmask[i / nw][i % nw] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < ca; i += BQ * 2) {
      const int e = min(max(la[i], 0), nkb - 1);
      atomicOr(&pmask[0][e >> 5], 1u << (e & 31));
    }
    for (int i = threadIdx.x; i < cb; i += BQ * 2) {
      const int e = min(max(lb[i], 0), nkb - 1);
      atomicOr(&pmask[1][e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    if (wave == 0) {
      int run = 0;
      for (int w0 = 0; w0 < nw; w0 += 64) {
        const int w = w0 + lane;
        const uint32_t a = w < nw ? pmask[0][w] : 0u, b = w < nw ? pmask[1][w] : 0u;
        uint32_t u = a | b;
        const int c = __popc(u);
        int pre = c;  // inclusive prefix over the lanes
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const int t = __shfl_up(pre, m, 64);
          if (lane >= m) pre += t;
        }
        int pos = run + pre - c;
        while (u) {
          const int bit = __ffs(u) - 1;
          u &= u - 1u;
          ul_[pos++] = (uint16_t)((w * 32 + bit) | (((a >> bit) & 1u) << 14) | (((b >> bit) & 1u) << 15));
        }
        run += __shfl(pre, 63, 64);
      }
      if (lane == 0) ucnt = run;
    }
    __syncthreads();
    ulist = (const __attribute__((address_space(3))) uint16_t*)ul_;
    pair_cnt = __builtin_amdgcn_readfirstlane(ucnt);
  }
  if constexpr (WIN) {
    // key blocks from the start of the first row's window to the end of the last row's window
    const int r0 = qb * BQ, r1 = min(N, r0 + BQ) - 1;
    const int wend = min(N, (r1 / win + 1) * win);
    kb_first = (r0 / win) * win / BK;
    cnt = (wend - 1) / BK - kb_first + 1;
  } else if constexpr (PAIR) {
    cnt = pair_cnt;
  } else {
    cnt = min(max(kcnt[tile], 0), nkb);
  }
  // list entries are clamped to [0, nKB) so that no load leaves K or V
  auto blk = [&](int i) {
    if constexpr (WIN) return kb_first + i;
    else if constexpr (PAIR) return (int)(ulist[i] & 0x0fffu);
    else return min(max(list[i], 0), nkb - 1);
  };
  // PAIR: whether this wave's row keeps union entry e (an entry as stored, or -1 past the end)
  auto keeps = [&](int e) { return e >= 0 && ((e >> (14 + half)) & 1) != 0; };

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;

  uint32_t doff[C::PER_WAVE];
  dma_offsets<D, BQ>(wave, lane, doff);
  // K or V block kb into dst: contiguous rows, or rows of the window-transposed order
  auto copy = [&](const char* base, int kb, lchar* dst) {
    copy_tile<D, BQ, WT>(base, kb, N, wt_nw, wt_w, wave, lane, doff, dst);
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
  // running max in the scaled log2 domain, shared by the lane pair. With WIN a query can meet
  // blocks whose keys all lie outside its window; a finite start keeps exp2(-inf - m) at 0 there
  // (exp2(-inf + inf) would be undefined), and the first block with a key raises it as before.
  float m_run = (WIN || PAIR) ? -3.0e38f : -INFINITY;
  float l_run = 0.f;  // this lane's part of the running sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // WIN: this lane's query row keeps key rows [wa, wa + wlen); the wave skips the element test
  // for key blocks inside the one window that holds all of its valid rows
  int wa = 0, wlen = 0, wv_lo = 1, wv_hi = 0;
  if constexpr (WIN) {
    wa = (qrow / win) * win;
    wlen = max(0, min(win, N - wa));
    const int w0 = qb * BQ + wave * 32, w1 = min(N, w0 + 32) - 1;
    if (w0 < N && w0 / win == w1 / win) {
      wv_lo = (w0 / win) * win;
      wv_hi = min(N, wv_lo + win);
    }
  }

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
  // PAIR: a block this wave's row does not keep: every score -inf
  auto mask_all = [&](f32x16 (&sc)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = -INFINITY, b = -INFINITY;
      // the empty asm keeps this a branch: as selects hoisted out of it the mask would cost
      // every block
      asm volatile("" : "+v"(a), "+v"(b));
      sc[0][i] = a;
      sc[1][i] = b;
    }
  };
  // WIN: keys outside this lane's window (and past N) get score -inf
  auto mask_win = [&](f32x16 (&sc)[2], int kb) {
    if (kb * BK >= wv_lo && kb * BK + BK <= wv_hi) return;
    const int base = kb * BK + 4 * hf - wa;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = base + 8 * (i >> 2) + (i & 3);
      if ((unsigned)off >= (unsigned)wlen) sc[0][i] = -INFINITY;
      if ((unsigned)(off + 32) >= (unsigned)wlen) sc[1][i] = -INFINITY;
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
  const bool ragged_last = cnt > 0 && (N % BK) != 0 && blk(cnt - 1) == nkb - 1;
  // Step t. NEXT: 0 = no block t + 1 (last step), 1 = full block t + 1, 2 = ragged block t + 1.
  // kn / vc hold K(t+1) / V(t); kf / vf receive K(t+2) / V(t+1).
  // Word j (0..15) of P^T packed to bf16: tile h = j & 1, elements 8 u + 2 e and 8 u + 2 e + 1 with
  // u = j >> 3, e = (j >> 1) & 3; the row sum takes the same bf16 values, into partial sum
  // (e & 1) * 2 + h (the order of the adds is that of accumulate).
  auto p_word = [&](const f32x16 (&sc)[2], int j, uint32_t (&pw)[16], float (&rs)[4]) {
    const int h = j & 1, u = j >> 3, e = (j >> 1) & 3;
    pw[j] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sc[h][8 * u + 2 * e], c_log2, -m_run)),
                      __builtin_amdgcn_exp2f(fmaf(sc[h][8 * u + 2 * e + 1], c_log2, -m_run)));
    // an empty asm on the word keeps its exps here: IR passes would otherwise sink them to the P V
    // products, past the scheduling fences
    asm volatile("" : "+v"(pw[j]));
    rs[(e & 1) * 2 + h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[j]), ones,
                                                          rs[(e & 1) * 2 + h], false);
  };
  // V^T fragments of key chunk c, channel tile r, from the tile vt (two transpose reads)
  auto vrd = [&](lchar* vt, int c, int r) {
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) v4i16*>(vt + voff[r][0] + c * 16 * C::ROWB));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) v4i16*>(vt + voff[r][1] + c * 16 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // O^T += V^T P^T for the packed words of the block in vt; va0 holds the fragments of key chunks 0
  // and 1, read earlier, and chunk c + 2 is read while chunk c multiplies
  auto pv = [&](const uint32_t (&pw)[16], lchar* vt, bf16x8 (&va0)[2][D / 32]) {
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[u] = __builtin_bit_cast(bf16x8, make_uint4(pw[8 * u], pw[8 * u + 2], pw[8 * u + 4], pw[8 * u + 6]));
      pb[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(pw[8 * u + 1], pw[8 * u + 3], pw[8 * u + 5], pw[8 * u + 7]));
    }
    bf16x8 va[3][D / 32];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < D / 32; ++r) va[a][r] = va0[a][r];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
        if (c + 2 < 4) va[(c + 2) % 3][r] = vrd(vt, c + 2, r);
        oacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c % 3][r], pb[c], oacc[r], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (c + 2 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  // S^T of the key block in kt into sn, interleaved with the P words of sc: each pair of score
  // MFMAs is followed by two P words, and the K fragments are read two steps ahead (three slots),
  // so the vector units and the LDS reads run under the matrix products of one wave. mid(s) runs
  // after s-step s (the step's copies).
  auto scores_p = [&](const lchar* kt, f32x16 (&sn)[2], const f32x16 (&sc)[2], uint32_t (&pw)[16],
                      float (&rs)[4], auto&& mid) {
    // raised priority for this phase, whose vector work bounds it: the other wave on the SIMD,
    // usually in its P V products, then fills the matrix core around this wave's instructions
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sn[0][i] = 0.f;
      sn[1][i] = 0.f;
    }
    bf16x8 a0[3], a1[3];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      a0[s] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s]);
      a1[s] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s] + 32 * C::ROWB);
    }
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      if (s + 2 < D / 16) {
        a0[(s + 2) % 3] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s + 2]);
        a1[(s + 2) % 3] =
            *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[s + 2] + 32 * C::ROWB);
      }
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s % 3], qf[s], sn[0], 0, 0, 0);
      if (2 * s < 16) p_word(sc, 2 * s, pw, rs);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s % 3], qf[s], sn[1], 0, 0, 0);
      if (2 * s + 1 < 16) p_word(sc, 2 * s + 1, pw, rs);
      __builtin_amdgcn_sched_barrier(0);
      mid(s);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 2 * (D / 16); j < 16; ++j) p_word(sc, j, pw, rs);
    __builtin_amdgcn_s_setprio(0);
  };

  // kept-list entries t + 1 and t + 2 of step t, in scalar registers; entry t + 3 is fetched
  // during step t by a vector load (counted by vmcnt, which the next step's barrier drains), so
  // that no scalar load waits right behind the barrier
  int e1, e2;
  if constexpr (PAIR) {
    e1 = cnt > 1 ? (int)ulist[1] : -1;
    e2 = cnt > 2 ? (int)ulist[2] : -1;
  } else {
    e1 = cnt > 1 ? blk(1) : -1;
    e2 = cnt > 2 ? blk(2) : -1;
  }
  int vl = 0, lz = 0;
  asm volatile("" : "+v"(lz));  // a zero opaque to the compiler, which makes the list load a vector load
  auto step = [&](int t, const f32x16 (&sc)[2], f32x16 (&sn)[2], const lchar* kn, lchar* vc, lchar* kf, lchar* vf,
                  auto next_tag) {
    constexpr int NEXT = decltype(next_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K(t+1) and V(t) are resident; every wave is done with K(t) and V(t-1)
    // the DMA for K(t+2) and V(t+1) is issued between the score MFMAs, so that the waves released
    // by the barrier start on the matrix cores instead of queueing their copies first
    int blk1, blk2;
    bool keep1 = true;  // PAIR: this wave's row keeps block t + 1
    if constexpr (WIN) {
      blk2 = t + 2 < cnt ? blk(t + 2) : -1;
      blk1 = t + 1 < cnt ? blk(t + 1) : -1;
    } else if constexpr (PAIR) {
      // union entries (with their row bits) t + 1, t + 2 in scalar registers, t + 3 read from LDS
      if (t > 0) {
        e1 = e2;
        e2 = t + 2 < cnt ? __builtin_amdgcn_readfirstlane(vl) : -1;
      }
      if (t + 3 < cnt) vl = ulist[t + 3];
      blk1 = e1 >= 0 ? (e1 & 0x0fff) : -1;
      blk2 = e2 >= 0 ? (e2 & 0x0fff) : -1;
      keep1 = keeps(e1);
    } else {
      if (t > 0) {
        e1 = e2;
        e2 = t + 2 < cnt ? min(max(__builtin_amdgcn_readfirstlane(vl), 0), nkb - 1) : -1;
      }
      if (t + 3 < cnt) vl = list[t + 3 + lz];
      blk1 = e1;
      blk2 = e2;
    }
    uint32_t pw[16];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    auto issue_all = [&]() {
      if (blk2 >= 0) copy(kbase, blk2, kf);
      if (blk1 >= 0) copy(vbase, blk1, vf);
    };
    // the copies go out between score products: K after the second pair of s-steps' products, V
    // after three quarters of them, so their issue hides under the matrix core instead of delaying
    // the first P V products
    auto issue = [&](int s) {
      if (s == 1 && blk2 >= 0) copy(kbase, blk2, kf);
      if (s == 3 * (D / 64) - 1 && blk1 >= 0) copy(vbase, blk1, vf);
    };
    if constexpr (NEXT != 0) {
      scores_p(kn, sn, sc, pw, rs, issue);
      if constexpr (NEXT == 2) mask_tail(sn, blk1);
      if constexpr (WIN) mask_win(sn, blk1);
      if constexpr (PAIR) {
        if (!keep1) mask_all(sn);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) p_word(sc, j, pw, rs);
    }
    // the V^T fragments of the first two key chunks are read before anything else of the P V half
    bf16x8 va0[2][D / 32];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < D / 32; ++r) va0[a][r] = vrd(vc, a, r);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT == 0) issue_all();
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    pv(pw, vc, va0);
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
    if constexpr (WIN) mask_win(sa, blk(0));
    if constexpr (PAIR) {
      if (!keeps((int)ulist[0])) mask_all(sa);
    }
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

// Launch order of the attention rows: order[w] is the row that workgroup w computes. Workgroups
// reach XCD w % 8 in order of w, each XCD walking its rows in the order xcd_chunk_row gives.
// Over a grid of many rounds that order stays (its chunks keep neighbouring rows, and the key
// blocks they share, within one XCD's L2). Over a short grid (fewer than kLptRows rows, under 16
// rounds of the 512 workgroups that fit the chip) the last round's rows decide the time, so each
// XCD takes its rows longest list first (equal lengths in the default order): workgroup 8 l + x
// gets the row of rank l among XCD x's rows, ranked by descending count. Rows past the whole
// XCD shares keep their default place.
constexpr int kLptRows = 8192;
__global__ __launch_bounds__(1024) void row_order_kernel(const int32_t* __restrict__ kcnt, int rows,
                                                         int32_t* __restrict__ order) {
  const int per = rows >> 3;
  if (rows >= kLptRows) {
    for (int w = blockIdx.x * 1024 + threadIdx.x; w < rows; w += gridDim.x * 1024) order[w] = xcd_chunk_row(w, rows);
    return;
  }
  __shared__ int cl[kLptRows / 8];
  const int x = blockIdx.x;
  for (int l = threadIdx.x; l < per; l += 1024) cl[l] = kcnt[xcd_chunk_row(8 * l + x, rows)];
  __syncthreads();
  for (int l = threadIdx.x; l < per; l += 1024) {
    const int c = cl[l];
    int rank = 0;
    for (int j = 0; j < per; ++j) rank += (cl[j] > c) | ((cl[j] == c) & (j < l));
    order[8 * rank + x] = xcd_chunk_row(8 * l + x, rows);
  }
  if (x == 0)
    for (int w = per * 8 + threadIdx.x; w < rows; w += 1024) order[w] = w;
}

hipError_t launch_row_order(const int32_t* kcnt, int rows, int32_t* order, hipStream_t stream) {
  const unsigned grid = rows >= kLptRows ? (unsigned)((rows + 1023) / 1024) : 8u;
  hipLaunchKernelGGL(row_order_kernel, dim3(grid), dim3(1024), 0, stream, kcnt, rows, order);
  return hipGetLastError();
}

template <int DT, int D, int BQ>
static hipError_t launch_attn_t(const void* q, const void* k, const void* v, const int32_t* kidx,
                                const int32_t* kcnt, int BH, int N, int nqb, int nkb, float c_log2, void* o,
                                float* lse, const int32_t* row_order, hipStream_t stream) {
  if constexpr (DT == kBF16) {
    if constexpr (BQ == 64 && D == 128) {
      // pairs of 64-query rows on the 4-wave kernel (the rows' order does not apply). With d = 64
      // the one-row kernel's 32 KiB of LDS already lets five 2-wave workgroups share a CU, and
      // the union's extra blocks then cost more than the pairing gains.
      if (nkb <= kPairMaxKB) {
        const int nqb128 = (N + 127) / 128;
        hipLaunchKernelGGL((attn_fwd_kernel<D, 128, false, false, true>), dim3((unsigned)(BH * nqb128)),
                           dim3(DCfg<D, 128>::NT), 0, stream, q, k, v, kidx, kcnt, N, nqb128, nkb, c_log2, o, lse, 0,
                           0, 0, nullptr, nqb);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((attn_fwd_kernel<D, BQ>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D, BQ>::NT), 0, stream,
                       q, k, v, kidx, kcnt, N, nqb, nkb, c_log2, o, lse, 0, 0, 0, row_order);
  } else {
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, BQ>), dim3((unsigned)(BH * nqb)), dim3(BQ * 2), 0, stream,
                       static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v), kidx,
                       kcnt, N, nqb, nkb, c_log2, static_cast<float*>(o), lse, row_order);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const void* q, const void* k, const void* v, int dtype, const int32_t* kidx,
                       const int32_t* kcnt, int BH, int N, int d, int Bq, double scale, void* o, float* lse,
                       hipStream_t stream, const int32_t* row_order) {
  const int nqb = (N + Bq - 1) / Bq;
  const int nkb = (N + BK - 1) / BK;
  const float c_log2 = (float)(scale * 1.4426950408889634);
#define SA_ATTN_CASE(DT_, D_, BQ_)                                                               \
  if (dtype == DT_ && d == D_ && Bq == BQ_)                                                      \
    return launch_attn_t<DT_, D_, BQ_>(q, k, v, kidx, kcnt, BH, N, nqb, nkb, c_log2, o, lse, row_order, stream);
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
                       stream, q, k, v, kidx, kcnt, N, nqb, nkb, c_log2, o, lse, nw, window, 0, nullptr);   \
    return hipGetLastError();                                                                                \
  }
  SA_WT_CASE(128, 128)
  SA_WT_CASE(128, 64)
  SA_WT_CASE(64, 128)
  SA_WT_CASE(64, 64)
#undef SA_WT_CASE
  return hipErrorInvalidValue;
}

// SQuad passes, token-exact, without lists. WT = false: row t attends to the rows of its window
// of `window` tokens. WT = true: in the window-transposed order read in place, row s attends to
// the rows of its run of N / window (the tokens at its position inside their windows).
template <int D, int BQ, bool WT>
static hipError_t launch_squad_t(const void* q, const void* k, const void* v, int BH, int N, int nqb, int nkb,
                                 float c_log2, int window, void* o, float* lse, hipStream_t stream) {
  const int nw = WT ? N / window : 0;
  const int32_t* none = nullptr;
  hipLaunchKernelGGL((attn_fwd_kernel<D, BQ, WT, true>), dim3((unsigned)(BH * nqb)), dim3(DCfg<D, BQ>::NT), 0, stream,
                     q, k, v, none, none, N, nqb, nkb, c_log2, o, lse, nw, WT ? window : 0, WT ? nw : window, none);
  return hipGetLastError();
}

hipError_t launch_attn_squad(const void* q, const void* k, const void* v, int BH, int N, int d, int Bq, double scale,
                             int window, bool global_pass, void* o, float* lse, hipStream_t stream) {
  const int nqb = (N + Bq - 1) / Bq;
  const int nkb = (N + BK - 1) / BK;
  const float c_log2 = (float)(scale * 1.4426950408889634);
#define SA_SQ_CASE(D_, BQ_)                                                                                   \
  if (d == D_ && Bq == BQ_)                                                                                   \
    return global_pass ? launch_squad_t<D_, BQ_, true>(q, k, v, BH, N, nqb, nkb, c_log2, window, o, lse, stream) \
                       : launch_squad_t<D_, BQ_, false>(q, k, v, BH, N, nqb, nkb, c_log2, window, o, lse, stream);
  SA_SQ_CASE(128, 128)
  SA_SQ_CASE(128, 64)
  SA_SQ_CASE(64, 128)
  SA_SQ_CASE(64, 64)
#undef SA_SQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace sa
