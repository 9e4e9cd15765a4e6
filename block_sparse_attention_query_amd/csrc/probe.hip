// Probe-fitted residual correction of the sparse attention output (gfx950).
//
// Page "Partition the Support, Reconstruct the Residual: Training-Free Sparse Attention for Video
// Generation and World Models" (physicalainews.jp), original abstract: a small set of exact query
// rows calibrates, for each call, an affine correction from the sparse output within the output
// subspace that the probe residuals span. Per (b, h):
//   1. probes: P query blocks at evenly spaced positions among the full query blocks;
//   2. their exact (dense) attention over all N keys, split over S key-block ranges (so that a few
//      probe blocks still fill the GPU) whose partial results are merged by log-sum-exp;
//   3. X = [O_sparse, 1] and R = O_exact - O_sparse on the probe rows, G = X^T X and C = X^T R
//      (float64);
//   4. A = (G + mu I)^-1 C with mu = ridge * trace(G) / (d + 1), by Cholesky factorisation;
//   4b. with a rank below d, A <- A V_r V_r^T: V_r the eigenvectors of R^T R for its rank largest
//      eigenvalues (the principal directions of the probe residuals);
//   5. O <- O + [O, 1] A on every row, in place.
// Kernels: probe_partial (MFMA, the forward's tile layout), probe_combine, probe_gram (fp64 MFMA),
// probe_chol and probe_subst (fp64), probe_subspace (fp32 Jacobi, with a rank below d) and
// probe_apply (bf16 MFMA, HBM-bound).
#include <algorithm>
#include <type_traits>

#include "attn_tiles.h"

namespace sa {

__host__ __device__ inline int probe_block(int p, int P, int nqb, int N, int BQ) {
  const int full = (N % BQ == 0) ? nqb : max(nqb - 1, 1);
  const int i = (int)((2LL * p + 1) * full / (2LL * P));  // floor((p + 1/2) full / P)
  return min(full - 1, i);
}

// Number S of key-block ranges of the probes' dense attention. The BH P S workgroups run in
// rounds of 512 (two per CU); S minimises rounds x key blocks per range (the smaller S on a tie),
// with at most 24 ranges (each adds a partial output to write and merge) and at least 4 key
// blocks per range.
inline int probe_splits(int BH, int P, int nkb) {
  const long long units = (long long)BH * P;
  const int smax = std::max(1, std::min(24, nkb / 4));
  int best = 1;
  long long best_cost = -1;
  for (int S = 1; S <= smax; ++S) {
    const long long cost = ((units * S + 511) / 512) * ((nkb + S - 1) / S);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = S;
    }
  }
  return best;
}

// ---------------------------------------------------------------- 2a. partial dense attention

// One workgroup per (bh, range s, probe p), BQ / 32 waves of 32 queries, over key blocks
// [s nkb / S, (s + 1) nkb / S). The S^T = K Q^T and O^T += V^T P^T products, the tile layout and
// the two-stage software pipeline are the forward kernel's (step t computes the scores of block
// t + 1 while P V of block t accumulates; K runs one block ahead of V in LDS); every key block of
// the range is kept. Writes, per query, the unnormalised output sum_u 2^(c s_u - m) V_u (fp32),
// its reference m (log2 domain) and the sum l of the same weights. Partial index: (bh S + s) P + p.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? 2 : 1) void probe_partial_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                                  const void* __restrict__ v, int N, int nqb, int nkb,
                                                                  int P, int S, float c_log2, float* __restrict__ part_o,
                                                                  float* __restrict__ part_ml) {
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char kbuf_[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf_[2 * C::TILE];
  lchar* const kb0 = (lchar*)kbuf_;
  lchar* const kb1 = kb0 + C::TILE;
  lchar* const vb0 = (lchar*)vbuf_;
  lchar* const vb1 = vb0 + C::TILE;

  // the P probes of one range run on one XCD and share its L2 for the key / value blocks
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int p = unit % P;
  const int s = (unit / P) % S;
  const int bh = unit / (P * S);
  const int qb = probe_block(p, P, nqb, N, BQ);
  const int first = (int)((long long)s * nkb / S);
  const int cnt = (int)((long long)(s + 1) * nkb / S) - first;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;
  auto blk = [&](int i) { return first + i; };

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;
  uint32_t doff[C::PER_WAVE];
  dma_offsets<D, BQ>(wave, lane, doff);
  if (cnt > 0) {
    dma_tile<D, BQ>(kbase, blk(0), N, wave, lane, doff, kb0);
    dma_tile<D, BQ>(vbase, blk(0), N, wave, lane, doff, vb0);
  }
  if (cnt > 1) dma_tile<D, BQ>(kbase, blk(1), N, wave, lane, doff, kb1);
  // Q^T fragments: query 32 wave + ln, channels 16 j + 8 hf .. + 7 (rows past N are zero)
  const int qrow = qb * BQ + wave * 32 + ln;
  const bool qvalid = qrow < N;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    qf[j] = __builtin_bit_cast(bf16x8, qvalid ? *reinterpret_cast<const uint4*>(qbase + ((size_t)qrow * D + 16 * j + 8 * hf) * 2)
                                              : make_uint4(0, 0, 0, 0));
  int koff[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) koff[j] = ln * C::ROWB + (((2 * j + hf) ^ sw) << 4);
  }
  // V^T fragment offsets: the transpose read of lane i16 of group (half, gsub) covers key row
  // 16 c + 8 u + 4 half + i16 / 4 and channel chunk 4 r + 2 gsub + (i16 % 4) / 2; the chunk
  // swizzle depends on the row modulo 16 only, so the offsets of c > 0 add 16 c rows.
  int voff[D / 32][2];
  {
    const int i16 = lane & 15, grp = lane >> 4;
    const int half = grp >> 1, gsub = grp & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = 8 * u + 4 * half + (i16 >> 2);
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
        const int chunk = 4 * r + 2 * gsub + ((i16 & 3) >> 1);
        voff[r][u] = row * C::ROWB + ((chunk ^ kv_swz<D>(row)) << 4) + (i16 & 1) * 8;
      }
    }
  }
  f32x16 oacc[D / 32];
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[r][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  auto scores = [&](const lchar* kt, f32x16 (&sc)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[0][i] = 0.f;
      sc[1][i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[j]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[j] + 32 * C::ROWB);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[j], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[j], sc[1], 0, 0, 0);
    }
  };
  auto mask_tail = [&](f32x16 (&sc)[2], int kb) {  // keys past N in the ragged last block
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
      if (key >= N) sc[0][i] = -INFINITY;
      if (key + 32 >= N) sc[1][i] = -INFINITY;
    }
  };
  auto block_max = [&](const f32x16 (&sc)[2]) {
    float m4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m4[c] = fmaxf(sc[0][c], sc[1][c]);
#pragma unroll
    for (int i = 4; i < 16; ++i) m4[i & 3] = fmaxf(fmaxf(m4[i & 3], sc[0][i]), sc[1][i]);
    const float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
    return partner32_max(mx) * c_log2;
  };
  auto raise_max = [&](float mx) {  // lazy rescale: weights stay below 2^8 between raises
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
    if constexpr (NEXT != 0) {
      scores(kn, sn);
      if constexpr (NEXT == 2) mask_tail(sn, blk(t + 1));
    }
    if (t + 2 < cnt) dma_tile<D, BQ>(kbase, blk(t + 2), N, wave, lane, doff, kf);
    if (t + 1 < cnt) dma_tile<D, BQ>(vbase, blk(t + 1), N, wave, lane, doff, vf);
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
  // element i of oacc[r] is channel 32 r + 8 (i / 4) + 4 hf + i % 4 of query 32 wave + ln
  const size_t qo = (size_t)unit * BQ + wave * 32 + ln;
  float* po = part_o + qo * D;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<float4*>(po + 32 * r + 8 * a + 4 * hf) =
          make_float4(oacc[r][4 * a], oacc[r][4 * a + 1], oacc[r][4 * a + 2], oacc[r][4 * a + 3]);
  const float l_tot = partner32_sum(l_run);
  if (hf == 0) *reinterpret_cast<float2*>(part_ml + qo * 2) = make_float2(m_run, l_tot);
}

// ---------------------------------------------------------------- 2b. merge of the ranges

// One thread per (bh, probe, query, 4 channels): O = sum_s o_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
// with M = max_s m_s. Output rows are ordered [bh][probe][query].
__global__ __launch_bounds__(256) void probe_combine_kernel(const float* __restrict__ part_o,
                                                            const float* __restrict__ part_ml, long long rows, int P,
                                                            int S, int BQ, int D, float* __restrict__ exact) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = D / 4;
  if (e >= rows * per_row) return;
  const int c4 = (int)(e % per_row);
  const long long row = e / per_row;
  const long long qq = row % BQ, pu = row / BQ;
  const long long p = pu % P, bh = pu / P;
  auto part = [&](int s) { return ((bh * S + s) * P + p) * BQ + qq; };
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[part(s) * 2]);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M > -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const long long r = part(s);
      const float w = __builtin_amdgcn_exp2f(part_ml[r * 2] - M);
      L += part_ml[r * 2 + 1] * w;
      const float4 x = *reinterpret_cast<const float4*>(part_o + r * D + 4 * c4);
      acc.x += x.x * w;
      acc.y += x.y * w;
      acc.z += x.z * w;
      acc.w += x.w * w;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(exact + row * D + 4 * c4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

// ---------------------------------------------------------------- 3. [G | C] = X^T [X | R]

// Z = [X | R] on the probe rows, X = [O_sparse, 1] (bf16 output widened to float64, rows past
// the sequence zero) and R = O_exact - O_sparse; [G | C] = X^T Z is a (D + 1) x (2 D + 1) float64
// product over the m = P BQ probe rows, on the matrix cores (v_mfma_f64_16x16x4f64: lane j holds
// A[j % 16][j / 16] and B[j / 16][j % 16] of a 16x4 / 4x16 step; element i of the result is
// C[4 i + j / 16][j % 16]). Grid (BH, ceil(grows / 16)): a workgroup of 4 waves computes the
// 16 rows i0 .. i0 + 15 of Z^T Z (A = Z[:, i0 .. i0 + 15]^T), its waves splitting the 16-column
// tiles; Z is staged through LDS 16 probe rows at a time, the next stage prefetched in registers.
// grows = D + 1 gives [G | C]; grows = 2 D + 1 gives all of Z^T Z, whose last D rows and columns
// hold R^T R for the residual subspace.
template <int D>
struct GramCfg {
  static constexpr int n = D + 1, W = 2 * D + 1;
  static constexpr int NJ = (W + 15) / 16;        // 16-column tiles of [G | C]
  static constexpr int ZW = NJ * 16;              // staged columns (zero past W)
  static constexpr int ZS = ZW + 2;               // LDS row stride (doubles)
  static constexpr int CH = 16;                   // probe rows per stage
  static constexpr int EPT = (CH * ZW + 255) / 256;
  static constexpr int TPW = (NJ + 3) / 4;        // column tiles per wave
};

template <int D>
__global__ __launch_bounds__(256) void probe_gram_kernel(const uint16_t* __restrict__ o, const float* __restrict__ exact,
                                                         int N, int nqb, int BQ, int P, int grows,
                                                         double* __restrict__ gram) {
  using G = GramCfg<D>;
  constexpr int n = G::n, W = G::W, NJ = G::NJ, ZW = G::ZW, ZS = G::ZS, CH = G::CH, EPT = G::EPT, TPW = G::TPW;
  __shared__ double z[CH * ZS];
  __shared__ int ptok[1024];  // first token of each probe block
  const int bh = blockIdx.x, i0 = blockIdx.y * 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int p = tid; p < P; p += 256) ptok[p] = probe_block(p, P, nqb, N, BQ) * BQ;
  __syncthreads();
  const uint16_t* oh = o + (size_t)bh * N * D;
  const float* eh = exact + (size_t)bh * P * BQ * D;
  const int m = P * BQ;
  // Z[pr][col] for the stage: both loads of every element are issued unconditionally (clamped
  // addresses) so that they overlap, and the element is selected afterwards.
  double pre[EPT];
  auto fetch = [&](int r0) {
    uint16_t ov[EPT];
    float ev[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = tid + 256 * u;
      const int pr = min(r0 + e / ZW, m - 1), col = e % ZW;
      const int p = pr / BQ, qq = pr - p * BQ;
      const int tok = min(ptok[p] + qq, N - 1);
      const int ch = col < D ? col : (col >= n && col < W ? col - n : 0);
      ov[u] = oh[(size_t)tok * D + ch];
      ev[u] = eh[((size_t)p * BQ + qq) * D + ch];
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = tid + 256 * u;
      const int pr = r0 + e / ZW, col = e % ZW;
      const int p = min(pr, m - 1) / BQ;
      const bool valid = e < CH * ZW && pr < m && ptok[p] + (min(pr, m - 1) - p * BQ) < N;
      const double x = (double)__uint_as_float((uint32_t)ov[u] << 16);
      const double z = col < D ? x : (col == D ? 1.0 : (col < W ? (double)ev[u] - x : 0.0));
      pre[u] = valid ? z : 0.0;
    }
  };
  typedef double f64x4 __attribute__((ext_vector_type(4)));
  f64x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int jr = lane & 15, jk = lane >> 4;
  fetch(0);
  for (int r0 = 0; r0 < m; r0 += CH) {
    __syncthreads();  // the previous stage has been consumed
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = tid + 256 * u;
      if (e < CH * ZW) z[(e / ZW) * ZS + e % ZW] = pre[u];
    }
    __syncthreads();
    if (r0 + CH < m) fetch(r0 + CH);
#pragma unroll
    for (int s = 0; s < CH / 4; ++s) {
      const double a = z[(4 * s + jk) * ZS + i0 + jr];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int jt = wave + 4 * t;
        if (jt < NJ)
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, z[(4 * s + jk) * ZS + 16 * jt + jr], acc[t], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int jt = wave + 4 * t;
    const int col = 16 * jt + jr;
    if (jt < NJ && col < W) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = i0 + 4 * i + jk;
        if (row < grows) gram[((size_t)bh * grows + row) * W + col] = acc[t][i];
      }
    }
  }
}

// ---------------------------------------------------------------- 4. ridge solve

// Two kernels, float64 throughout.
//
// probe_chol: one workgroup of 1024 threads per head factorises G + mu I = L L^T by right-looking
// Cholesky steps on the unscaled trailing matrix (M' = M - m_k m_k^T / m_kk over the rows and
// columns past k, L[:, k] = m_k / sqrt(m_kk)). Every element of the lower triangle stays in the
// register of the thread that owns it (column-major packed index E, owner E mod 1024, so that a
// wave's slot covers one or two columns and drops out as a whole once the factorisation has
// passed them); step k only publishes column k through LDS (double-buffered, one barrier per
// step). The factor is written out as a square array whose rows are padded to whole row blocks,
// L below the diagonal, L^T above it and zeros in the padding, so that both substitutions read
// contiguous row segments, followed by the n reciprocals 1 / L[r][r].
//
// probe_subst: grid (heads, D / 32), 256 threads; each workgroup copies the factor to LDS and
// solves 32 of the D right-hand-side columns, which stay in registers: thread (c, rs) holds rows
// rs + 8 u of column c. Forward (L Y = C) and back (L^T A = Y) substitution run over blocks of 8
// rows: the block's values of each column go through LDS once, every thread finishes the whole
// block for its column (a small triangle, computed redundantly instead of a second barrier),
// then updates its own later (earlier) rows. Writes A (fp32 [D + 1][D]), A[0:D]^T as bf16 [D][D]
// (the apply kernel's operand) and the bias row A[D] (fp32).
template <int D>
struct SolveCfg {
  static constexpr int n = D + 1, W = 2 * D + 1;
  static constexpr int NT = 1024;                      // factorisation threads
  static constexpr int CW = 32;                        // right-hand-side columns per workgroup
  static constexpr int ST = 256;                       // substitution threads
  static constexpr int RS = ST / CW;                   // row sets (= rows per block)
  static constexpr int RPER = (n + RS - 1) / RS;       // rows per thread (= row blocks)
  static constexpr int SS = RPER * RS;                 // padded row stride of the factor (doubles)
  static constexpr int FAC = (n * SS + n + 1) & ~1;   // factor + reciprocals, doubles per head (even)
  static constexpr int TRI = n * (n + 1) / 2;          // lower triangle
  static constexpr int EPT = (TRI + NT - 1) / NT;      // factor elements per thread
  static constexpr int TS = D + 8;                     // bf16 row stride of the transposed copy
  static constexpr size_t CHOL_LDS = (size_t)n * SS * 8 + 2 * n * 8 + n * 8;
  static constexpr size_t SUBST_LDS = (size_t)FAC * 8 + 2 * RS * CW * 8;
  static_assert(D % CW == 0, "column groups");
  static_assert((size_t)CW * TS * 2 <= (size_t)n * SS * 8, "transposed copy must fit in the factor's space");
  static_assert(CHOL_LDS <= 160 * 1024 - 1024 && SUBST_LDS <= 160 * 1024, "LDS budget");
};

template <int D>
__global__ __launch_bounds__(1024) void probe_chol_kernel(const double* __restrict__ gram, int grows, double ridge,
                                                          double* __restrict__ fac) {
  using S = SolveCfg<D>;
  constexpr int n = S::n, W = S::W, NT = S::NT, SS = S::SS, TRI = S::TRI, EPT = S::EPT;
  extern __shared__ __attribute__((aligned(16))) double sm[];
  double* Lf = sm;               // n x SS: L (lower), L^T (upper), zero padding
  double* col = Lf + n * SS;     // 2 x n: column k of the trailing matrix
  double* invd = col + 2 * n;    // n: 1 / L[r][r]
  __shared__ double red[NT / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* g = gram + (size_t)bh * grows * W;

  for (int e = tid; e < n * SS; e += NT) Lf[e] = 0.0;
  double tr = 0.0;
  for (int r = tid; r < n; r += NT) tr += g[(size_t)r * W + r];
  for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o, 64);
  if (lane == 0) red[wave] = tr;
  __syncthreads();
  tr = 0.0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) tr += red[w];
  const double mu = ridge * tr / n;

  // owned elements of the lower triangle, column-major: column c starts at c n - c (c - 1) / 2
  // (ec = -1: none)
  int er[EPT], ec[EPT];
  double m[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int e = tid + NT * j;
    er[j] = 0;
    ec[j] = -1;
    m[j] = 0.0;
    if (e < TRI) {
      auto start = [](int c) { return c * n - c * (c - 1) / 2; };
      const float b2 = 2.f * n + 1.f;
      int c = (int)((b2 - sqrtf(b2 * b2 - 8.f * (float)e)) * 0.5f);
      c = c < 0 ? 0 : (c > n - 1 ? n - 1 : c);
      while (c > 0 && start(c) > e) --c;
      while (c < n - 1 && start(c + 1) <= e) ++c;
      const int r = c + e - start(c);
      er[j] = r;
      ec[j] = c;
      m[j] = g[(size_t)r * W + c] + (r == c ? mu : 0.0);
    }
  }
  for (int k = 0; k < n; ++k) {
    double* cb = col + (k & 1) * n;
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (ec[j] == k) cb[er[j]] = m[j];  // column k after step k - 1
    __syncthreads();
    const double dk = cb[k];  // > 0: G + mu I is positive definite for mu > 0
    // 1 / sqrt(dk): the hardware estimate and one Newton step
    double rsq = __builtin_amdgcn_rsq(dk);
    rsq = rsq * fma(-0.5 * dk * rsq, rsq, 1.5);
    const double inv = rsq * rsq;
    // slots of finished columns are skipped (wave-uniform); the live slots' loads are all issued
    // before the first use
    bool act[EPT];
    double va[EPT], vb[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      act[j] = __ballot(ec[j] >= k) != 0;
      va[j] = 0.0;
      vb[j] = 0.0;
      if (act[j]) {
        va[j] = cb[er[j]];
        vb[j] = cb[ec[j] < 0 ? 0 : ec[j]];
      }
    }
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (act[j]) {
        const double upd = fma(-va[j] * inv, vb[j], m[j]);
        m[j] = ec[j] > k ? upd : (ec[j] == k ? m[j] * rsq : m[j]);
      }
    }
  }
  __syncthreads();  // the zero fill is complete
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if (ec[j] >= 0) {
      Lf[er[j] * SS + ec[j]] = m[j];
      Lf[ec[j] * SS + er[j]] = m[j];
      if (er[j] == ec[j]) invd[er[j]] = 1.0 / m[j];
    }
  }
  __syncthreads();
  double* fo = fac + (size_t)bh * S::FAC;
  for (int e = tid; e < n * SS; e += NT) fo[e] = Lf[e];
  for (int e = tid; e < n; e += NT) fo[n * SS + e] = invd[e];
}

template <int D>
__global__ __launch_bounds__(256) void probe_subst_kernel(const double* __restrict__ gram, int grows,
                                                          const double* __restrict__ fac, float* __restrict__ a_out,
                                                          __bf16* __restrict__ at_out, float* __restrict__ bias_out) {
  using S = SolveCfg<D>;
  constexpr int n = S::n, W = S::W, CW = S::CW, RS = S::RS, RPER = S::RPER, SS = S::SS;
  extern __shared__ __attribute__((aligned(16))) double sm[];
  double* Lf = sm;               // n x SS
  double* invd = Lf + n * SS;    // n
  double* ytmp = sm + S::FAC;    // 2 x RS x CW: one row block of the right-hand sides
  const int bh = blockIdx.x, c0 = blockIdx.y * CW, tid = threadIdx.x;
  const double* g = gram + (size_t)bh * grows * W;
  {
    const double2* src = reinterpret_cast<const double2*>(fac + (size_t)bh * S::FAC);
    double2* dst = reinterpret_cast<double2*>(sm);
    for (int e = tid; e < S::FAC / 2; e += S::ST) dst[e] = src[e];
  }
  const int c = tid % CW, rs = tid / CW;
  double y[RPER];
#pragma unroll
  for (int u = 0; u < RPER; ++u) {
    const int row = rs + RS * u;
    y[u] = row < n ? g[(size_t)row * W + n + c0 + c] : 0.0;
  }
  __syncthreads();
  // Forward substitution L Y = C. Before block K the register array is rotated left by K: y[p]
  // holds row rs + RS (K + p) for p < RPER - K, the finished rows sit behind them, and after the
  // last block every row is back at y[u].
  for (int K = 0; K < RPER; ++K) {
    double* yt = ytmp + (K & 1) * RS * CW;
    if (K * RS + rs < n) yt[rs * CW + c] = y[0];
    __syncthreads();
    double yv[RS], yf[RS];
#pragma unroll
    for (int l = 0; l < RS; ++l) yv[l] = yt[l * CW + c];
#pragma unroll
    for (int l = 0; l < RS; ++l) {
      const int row = K * RS + l;
      const int rc = row < n ? row : n - 1;
      const double* lr = Lf + rc * SS + K * RS;
      double s = yv[l];
#pragma unroll
      for (int l2 = 0; l2 < l; ++l2) s = fma(-lr[l2], yf[l2], s);
      yf[l] = row < n ? s * invd[rc] : 0.0;
    }
    double own = 0.0;
#pragma unroll
    for (int l = 0; l < RS; ++l)
      if (l == rs) own = yf[l];
#pragma unroll
    for (int p0 = 1; p0 < RPER; p0 += 2) {
      // two rows at a time: their loads overlap, and the pin below keeps the next pair's loads
      // from being issued ahead (register pressure)
      double s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = p0 + h, row = rs + RS * (K + p);
        s[h] = 0.0;
        if (p < RPER && p < RPER - K && row < n) {
          const double* lr = Lf + row * SS + K * RS;
          s[h] = y[p];
#pragma unroll
          for (int l = 0; l < RS; ++l) s[h] = fma(-lr[l], yf[l], s[h]);
        }
      }
      asm volatile("" : "+v"(s[0]), "+v"(s[1])::"memory");
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = p0 + h, row = rs + RS * (K + p);
        if (p < RPER && p < RPER - K && row < n) y[p] = s[h];
      }
    }
#pragma unroll
    for (int p = 0; p + 1 < RPER; ++p) y[p] = y[p + 1];
    y[RPER - 1] = own;
  }
  __syncthreads();  // the last forward block's values are read before the buffers are reused
  // Back substitution L^T A = Y, blocks K = RPER - 1 .. 0 at steps j = RPER - 1 - K. Before step
  // j the array is rotated right by j: y[RPER - 1] holds row rs + RS K and y[p] row rs + RS (p - j)
  // for j <= p < RPER - 1. Row `row` of the square array holds L^T[row][col] for col > row.
  for (int j = 0; j < RPER; ++j) {
    const int K = RPER - 1 - j;
    double* yt = ytmp + (j & 1) * RS * CW;
    if (K * RS + rs < n) yt[rs * CW + c] = y[RPER - 1];
    __syncthreads();
    double yv[RS], yf[RS];
#pragma unroll
    for (int l = 0; l < RS; ++l) yv[l] = yt[l * CW + c];
#pragma unroll
    for (int l = RS - 1; l >= 0; --l) {
      const int row = K * RS + l;
      const int rc = row < n ? row : n - 1;
      const double* lr = Lf + rc * SS + K * RS;
      double s = yv[l];
#pragma unroll
      for (int l2 = l + 1; l2 < RS; ++l2) s = fma(-lr[l2], yf[l2], s);
      yf[l] = row < n ? s * invd[rc] : 0.0;
    }
    double own = 0.0;
#pragma unroll
    for (int l = 0; l < RS; ++l)
      if (l == rs) own = yf[l];
#pragma unroll
    for (int p0 = 0; p0 + 1 < RPER; p0 += 2) {
      double s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = p0 + h;
        s[h] = 0.0;
        if (p + 1 < RPER && p >= j) {
          const int row = rs + RS * (p - j);  // a row of an earlier block, < n
          const double* lr = Lf + row * SS + K * RS;
          s[h] = y[p];
#pragma unroll
          for (int l = 0; l < RS; ++l) s[h] = fma(-lr[l], yf[l], s[h]);
        }
      }
      asm volatile("" : "+v"(s[0]), "+v"(s[1])::"memory");
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int p = p0 + h;
        if (p + 1 < RPER && p >= j) y[p] = s[h];
      }
    }
#pragma unroll
    for (int p = RPER - 1; p > 0; --p) y[p] = y[p - 1];
    y[0] = own;
  }
  // outputs: A rows from registers; A^T in bf16 through a transposed LDS copy
  __syncthreads();
  __bf16* tl = reinterpret_cast<__bf16*>(Lf);
#pragma unroll
  for (int u = 0; u < RPER; ++u) {
    const int row = rs + RS * u;
    if (row < n) a_out[((size_t)bh * n + row) * D + c0 + c] = (float)y[u];
    if (row < D) tl[c * S::TS + row] = (__bf16)y[u];
    if (row == D) bias_out[(size_t)bh * D + c0 + c] = (float)y[u];
  }
  __syncthreads();
  for (int e = tid; e < CW * (D / 8); e += S::ST) {
    const int cc = e / (D / 8), ch = e % (D / 8);
    *reinterpret_cast<uint4*>(at_out + ((size_t)bh * D + c0 + cc) * D + ch * 8) =
        *reinterpret_cast<const uint4*>(tl + cc * S::TS + ch * 8);
  }
}

// ---------------------------------------------------------------- 4b. residual subspace

// The map confined to the output subspace observed in the probe residuals: A <- A V_r V_r^T with
// V_r the eigenvectors of R^T R (the last D rows and columns of Z^T Z) for its `rank` largest
// eigenvalues. One workgroup of 512 threads per head; R^T R and the eigenvector matrix sit in LDS
// as fp32 (rows padded by one float). Cyclic Jacobi: each sweep runs D - 1 rounds of D / 2
// disjoint pairs (the round-robin pairing: index 0 fixed, the others rotated by one per round);
// a round computes every pair's rotation (c, s) annihilating S[p][q], then rotates rows p and q
// of S for all pairs, then columns p and q of S and of V (S <- J^T S J, V <- V J). Sweeps stop when
// the off-diagonal mass is below 1e-12 of the total, after at most kJacobiSweeps. Eigenvalue i
// ranks by (descending S[i][i], index); the projector P = sum over the kept i of v_i v_i^T replaces
// S, A (fp32, from the substitution) replaces V, and A P is written back as A, A^T (bf16) and the
// bias row, the formats of the substitution kernel.
constexpr int kJacobiSweeps = 20;
template <int D>
struct SubCfg {
  static constexpr int NT = 512, P = D + 1;
  static constexpr size_t LDS = (size_t)2 * D * P * 4 + (size_t)(D + 2 * (D / 2) + 32) * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((size_t)(D + 1) * D <= (size_t)D * P, "A must fit in the eigenvector space");
};

template <int D>
__global__ __launch_bounds__(512) void probe_subspace_kernel(const double* __restrict__ gram, int rank,
                                                             float* __restrict__ a_io, __bf16* __restrict__ at_out,
                                                             float* __restrict__ bias_out) {
  using C = SubCfg<D>;
  constexpr int n = D + 1, W = 2 * D + 1, P = C::P, NT = C::NT, NP = D / 2;
  extern __shared__ __attribute__((aligned(16))) float sub_sm[];
  float* S = sub_sm;               // D x P
  float* V = S + D * P;            // D x P
  float* lam = V + D * P;          // D
  float* rc = lam + D;             // NP rotation cosines
  float* rsn = rc + NP;            // NP rotation sines
  float* red = rsn + NP;           // 32 partial sums
  const int bh = blockIdx.x, tid = threadIdx.x;
  const double* g = gram + ((size_t)bh * W + n) * W + n;  // R^T R, row stride W
  for (int e = tid; e < D * D; e += NT) {
    const int i = e / D, j = e % D;
    S[i * P + j] = (float)g[(size_t)i * W + j];
    V[i * P + j] = i == j ? 1.f : 0.f;
  }
  __syncthreads();
  // players of round k: 0, then 1 + (t - 1 + k) mod (D - 1) for t = 1 .. D - 1; pair i takes the
  // players at positions i and D - 1 - i
  auto player = [&](int t, int k) { return t == 0 ? 0 : 1 + (t - 1 + k) % (D - 1); };
  for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
    for (int k = 0; k < D - 1; ++k) {
      if (tid < NP) {
        const int a = player(tid, k), b = player(D - 1 - tid, k);
        const int p = min(a, b), q = max(a, b);
        const float spp = S[p * P + p], sqq = S[q * P + q], spq = S[p * P + q];
        float c = 1.f, sn = 0.f;
        if (fabsf(spq) > 1e-30f && fabsf(spq) > 1e-9f * sqrtf(fabsf(spp * sqq))) {
          const float tau = (sqq - spp) / (2.f * spq);
          const float t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
          c = 1.f / sqrtf(1.f + t * t);
          sn = t * c;
        }
        rc[tid] = c;
        rsn[tid] = sn;
      }
      __syncthreads();
      for (int e = tid; e < NP * D; e += NT) {  // rows p, q of S
        const int i = e / D, j = e % D;
        const int a = player(i, k), b = player(D - 1 - i, k);
        const int p = min(a, b), q = max(a, b);
        const float c = rc[i], sn = rsn[i];
        const float x = S[p * P + j], y = S[q * P + j];
        S[p * P + j] = c * x - sn * y;
        S[q * P + j] = sn * x + c * y;
      }
      __syncthreads();
      for (int e = tid; e < NP * D; e += NT) {  // columns p, q of S and V
        const int i = e % NP, j = e / NP;
        const int a = player(i, k), b = player(D - 1 - i, k);
        const int p = min(a, b), q = max(a, b);
        const float c = rc[i], sn = rsn[i];
        const float x = S[j * P + p], y = S[j * P + q];
        S[j * P + p] = c * x - sn * y;
        S[j * P + q] = sn * x + c * y;
        const float u = V[j * P + p], w = V[j * P + q];
        V[j * P + p] = c * u - sn * w;
        V[j * P + q] = sn * u + c * w;
      }
      __syncthreads();
    }
    // off-diagonal mass against the total
    float off = 0.f, tot = 0.f;
    for (int e = tid; e < D * D; e += NT) {
      const float x = S[(e / D) * P + e % D];
      tot += x * x;
      if (e / D != e % D) off += x * x;
    }
    for (int m = 32; m > 0; m >>= 1) {
      off += __shfl_xor(off, m);
      tot += __shfl_xor(tot, m);
    }
    if ((tid & 63) == 0) {
      red[tid >> 6] = off;
      red[16 + (tid >> 6)] = tot;
    }
    __syncthreads();
    float o2 = 0.f, t2 = 0.f;
    for (int w = 0; w < NT / 64; ++w) {
      o2 += red[w];
      t2 += red[16 + w];
    }
    __syncthreads();
    if (o2 <= 1e-12f * t2) break;  // uniform: every thread read the same sums
  }
  if (tid < D) lam[tid] = S[tid * P + tid];
  __syncthreads();
  // kept eigenvectors: rank by (descending eigenvalue, index)
  bool keep_i = false;
  if (tid < D) {
    int r = 0;
    const float li = lam[tid];
    for (int j = 0; j < D; ++j) r += (lam[j] > li || (lam[j] == li && j < tid)) ? 1 : 0;
    keep_i = r < rank;
  }
  __syncthreads();
  if (tid < D) lam[tid] = keep_i ? 1.f : 0.f;  // lam now flags the kept eigenvectors
  __syncthreads();
  for (int e = tid; e < D * D; e += NT) {  // projector into S
    const int a = e / D, b = e % D;
    float x = 0.f;
    for (int i = 0; i < D; ++i) x = fmaf(V[a * P + i] * lam[i], V[b * P + i], x);
    S[a * P + b] = x;
  }
  __syncthreads();
  float* A = V;  // (D + 1) x D, row stride D
  float* ah = a_io + (size_t)bh * n * D;
  for (int e = tid; e < n * D; e += NT) A[e] = ah[e];
  __syncthreads();
  for (int e = tid; e < n * D; e += NT) {
    const int row = e / D, col = e % D;
    float x = 0.f;
    for (int a = 0; a < D; ++a) x = fmaf(A[row * D + a], S[a * P + col], x);
    ah[e] = x;
    if (row < D) at_out[((size_t)bh * D + col) * D + row] = (__bf16)x;
    else bias_out[(size_t)bh * D + col] = x;
  }
}

// ---------------------------------------------------------------- 5. O <- O + O A[0:D] + A[D]

// Grid BH x ceil(N / ROWS): each workgroup (4 waves) keeps A[0:D]^T (bf16) of its head in LDS and
// walks ROWS token rows in tiles of 64. Per tile, C^T = A^T O^T runs on bf16 MFMA with fp32
// accumulation (32 x 32 output tiles: channels x tokens), then O + C + bias is rounded to bf16
// and stored in place, staged through LDS for row-contiguous stores.
template <int D>
__global__ __launch_bounds__(256) void probe_apply_kernel(uint16_t* __restrict__ o, const __bf16* __restrict__ at_g,
                                                          const float* __restrict__ bias_g, int N, int tph, int rows) {
  constexpr int ROWB = 2 * D, PADB = ROWB + 16;  // padded LDS rows: 16-byte row reads spread over banks
  constexpr int CPR = ROWB / 16;                 // 16-byte chunks per row
  constexpr int NT = D / 32;
  constexpr int TPW = 2 * NT / 4;                // 32 x 32 output tiles per wave
  static_assert((2 * NT) % 4 == 0, "tiles must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) char at[D * PADB];  // at[n][k] = A[k][n]
  __shared__ __attribute__((aligned(16))) char ot[64 * PADB]; // O tile [token][channel]
  __shared__ float bias[D];
  const int bh = blockIdx.x / tph;
  const int t0 = (blockIdx.x % tph) * rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  const char* ag = reinterpret_cast<const char*>(at_g + (size_t)bh * D * D);
  for (int e = tid; e < D * CPR; e += 256)
    *reinterpret_cast<uint4*>(at + (e / CPR) * PADB + (e % CPR) * 16) = *reinterpret_cast<const uint4*>(ag + e * 16);
  for (int e = tid; e < D; e += 256) bias[e] = bias_g[(size_t)bh * D + e];
  char* oh = reinterpret_cast<char*>(o + (size_t)bh * N * D);
  const int t1 = min(N, t0 + rows);
  // the next 64-row tile of O is loaded into registers while the current one is processed
  constexpr int PF = 64 * CPR / 256;  // 16-byte pieces per thread
  static_assert((64 * CPR) % 256 == 0, "whole pieces per thread");
  uint4 nx[PF];
  auto load = [&](int r0) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int e = tid + 256 * u, r = e / CPR, c = e % CPR;
      nx[u] = r0 + r < t1 ? *reinterpret_cast<const uint4*>(oh + (size_t)(r0 + r) * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  if (t0 < t1) load(t0);
  for (int r0 = t0; r0 < t1; r0 += 64) {
    __syncthreads();  // the previous tile's stores have read ot; A^T is resident
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int e = tid + 256 * u, r = e / CPR, c = e % CPR;
      *reinterpret_cast<uint4*>(ot + r * PADB + c * 16) = nx[u];
    }
    __syncthreads();
    if (r0 + 64 < t1) load(r0 + 64);
    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = wave + 4 * u, rt = tt & 1, ct = tt >> 1;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][i] = 0.f;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(ot + (32 * rt + ln) * PADB + (16 * j + 8 * hf) * 2);
        const bf16x8 y = *reinterpret_cast<const bf16x8*>(at + (32 * ct + ln) * PADB + (16 * j + 8 * hf) * 2);
        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, acc[u], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done reading O as an operand
    // element i of acc[u]: channel 32 ct + 8 (i / 4) + 4 hf + i % 4 of token 32 rt + ln; each
    // LDS cell is read and rewritten by the one lane that owns it
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = wave + 4 * u, rt = tt & 1, ct = tt >> 1;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ch = 32 * ct + 8 * a + 4 * hf;
        uint2* cell = reinterpret_cast<uint2*>(ot + (32 * rt + ln) * PADB + ch * 2);
        const uint2 w = *cell;
        const float x0 = bf16_lo(w.x) + acc[u][4 * a] + bias[ch];
        const float x1 = bf16_hi(w.x) + acc[u][4 * a + 1] + bias[ch + 1];
        const float x2 = bf16_lo(w.y) + acc[u][4 * a + 2] + bias[ch + 2];
        const float x3 = bf16_hi(w.y) + acc[u][4 * a + 3] + bias[ch + 3];
        *cell = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
      }
    }
    __syncthreads();
    for (int e = tid; e < 64 * CPR; e += 256) {
      const int r = e / CPR, c = e % CPR;
      if (r0 + r < N)
        *reinterpret_cast<uint4*>(oh + (size_t)(r0 + r) * ROWB + c * 16) = *reinterpret_cast<const uint4*>(ot + r * PADB + c * 16);
    }
  }
}

// ---------------------------------------------------------------- workspace and launcher

namespace {
constexpr int kApplyRows = 256;
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
struct ProbeWs {
  size_t part_o, part_ml, exact, gram, fac, amat, at, bias, total;
};
ProbeWs probe_ws_layout(int BH, int N, int d, int Bq, int P) {
  const int nkb = (N + BK - 1) / BK;
  const size_t units = (size_t)BH * P * probe_splits(BH, P, nkb);
  ProbeWs w{};
  size_t off = 0;
  w.part_o = off;
  off += al256(units * Bq * d * 4);
  w.part_ml = off;
  off += al256(units * Bq * 2 * 4);
  w.exact = off;
  off += al256((size_t)BH * P * Bq * d * 4);
  w.gram = off;
  off += al256((size_t)BH * (2 * d + 1) * (2 * d + 1) * 8);  // Z^T Z (rows past d + 1 only with a rank)
  w.fac = off;
  off += al256((size_t)BH * (d == 128 ? SolveCfg<128>::FAC : SolveCfg<64>::FAC) * 8);
  w.amat = off;
  off += al256((size_t)BH * (d + 1) * d * 4);
  w.at = off;
  off += al256((size_t)BH * d * d * 2);
  w.bias = off;
  off += al256((size_t)BH * d * 4);
  w.total = off;
  return w;
}
}  // namespace

size_t probe_workspace_bytes(int BH, int N, int d, int Bq, int P) { return probe_ws_layout(BH, N, d, Bq, P).total; }

template <int D, int BQ>
static hipError_t launch_probe_t(const void* q, const void* k, const void* v, void* o, int BH, int N, float scale,
                                 int P, double ridge, int rank, float* a_user, float* exact_user, void* ws,
                                 hipStream_t stream) {
  const int nqb = (N + BQ - 1) / BQ, nkb = (N + BK - 1) / BK;
  const int S = probe_splits(BH, P, nkb);
  const ProbeWs w = probe_ws_layout(BH, N, D, BQ, P);
  char* base = static_cast<char*>(ws);
  float* part_o = reinterpret_cast<float*>(base + w.part_o);
  float* part_ml = reinterpret_cast<float*>(base + w.part_ml);
  float* exact = exact_user ? exact_user : reinterpret_cast<float*>(base + w.exact);
  double* gram = reinterpret_cast<double*>(base + w.gram);
  double* fac = reinterpret_cast<double*>(base + w.fac);
  float* amat = a_user ? a_user : reinterpret_cast<float*>(base + w.amat);
  __bf16* at = reinterpret_cast<__bf16*>(base + w.at);
  float* bias = reinterpret_cast<float*>(base + w.bias);

  const float c_log2 = scale * 1.4426950408889634f;
  const size_t units = (size_t)BH * P * S;
  hipLaunchKernelGGL((probe_partial_kernel<D, BQ>), dim3((unsigned)units), dim3(DCfg<D, BQ>::NT), 0, stream, q, k, v, N,
                     nqb, nkb, P, S, c_log2, part_o, part_ml);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)BH * P * BQ;
  hipLaunchKernelGGL(probe_combine_kernel, dim3((unsigned)((rows * (D / 4) + 255) / 256)), dim3(256), 0, stream, part_o,
                     part_ml, rows, P, S, BQ, D, exact);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool project = rank < D;
  const int grows = project ? 2 * D + 1 : D + 1;
  hipLaunchKernelGGL((probe_gram_kernel<D>), dim3((unsigned)BH, (unsigned)((grows + 15) / 16)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(o), exact, N, nqb, BQ, P, grows, gram);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  using SC = SolveCfg<D>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&probe_chol_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)SC::CHOL_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((probe_chol_kernel<D>), dim3((unsigned)BH), dim3(SC::NT), SC::CHOL_LDS, stream, gram, grows, ridge,
                     fac);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&probe_subst_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)SC::SUBST_LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((probe_subst_kernel<D>), dim3((unsigned)BH, (unsigned)(D / SC::CW)), dim3(SC::ST), SC::SUBST_LDS,
                     stream, gram, grows, fac, amat, at, bias);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (project) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&probe_subspace_kernel<D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)SubCfg<D>::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((probe_subspace_kernel<D>), dim3((unsigned)BH), dim3(SubCfg<D>::NT), SubCfg<D>::LDS, stream,
                       gram, rank, amat, at, bias);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int tph = (N + kApplyRows - 1) / kApplyRows;
  hipLaunchKernelGGL((probe_apply_kernel<D>), dim3((unsigned)(BH * tph)), dim3(256), 0, stream,
                     static_cast<uint16_t*>(o), at, bias, N, tph, kApplyRows);
  return hipGetLastError();
}

hipError_t launch_probe(const void* q, const void* k, const void* v, void* o, int BH, int N, int d, int Bq,
                        double scale, int P, double ridge, int rank, float* a_user, float* exact_user, void* ws,
                        hipStream_t stream) {
  const float sc = (float)scale;
#define SA_PROBE_CASE(D_, BQ_)                                                                                   \
  if (d == D_ && Bq == BQ_)                                                                                      \
    return launch_probe_t<D_, BQ_>(q, k, v, o, BH, N, sc, P, ridge, rank, a_user, exact_user, ws, stream);
  SA_PROBE_CASE(128, 128)
  SA_PROBE_CASE(128, 64)
  SA_PROBE_CASE(64, 128)
  SA_PROBE_CASE(64, 64)
#undef SA_PROBE_CASE
  return hipErrorInvalidValue;
}

}  // namespace sa
