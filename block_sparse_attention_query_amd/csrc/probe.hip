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
//   5. O <- O + [O, 1] A on every row, in place.
// Kernels: probe_partial (MFMA, the forward's tile layout), probe_combine, probe_gram (fp64),
// probe_solve (fp64, one workgroup per head) and probe_apply (bf16 MFMA, HBM-bound).
#include <algorithm>

#include "attn_tiles.h"

namespace sa {

__host__ __device__ inline int probe_block(int p, int P, int nqb, int N, int BQ) {
  const int full = (N % BQ == 0) ? nqb : max(nqb - 1, 1);
  const int i = (int)((2LL * p + 1) * full / (2LL * P));  // floor((p + 1/2) full / P)
  return min(full - 1, i);
}

// Number of key-block ranges of the probes' dense attention: about 1024 workgroups in all, with
// at least 4 key blocks per range.
inline int probe_splits(int BH, int P, int nkb) {
  const long long units = (long long)BH * P;
  const int want = (int)std::max(1LL, (1024 + units - 1) / units);
  return std::max(1, std::min(want, nkb / 4));
}

// ---------------------------------------------------------------- 2a. partial dense attention

// One workgroup per (bh, range s, probe p), BQ / 32 waves of 32 queries, over key blocks
// [s nkb / S, (s + 1) nkb / S). The S^T = K Q^T and O^T += V^T P^T products and the tile layout
// are the forward kernel's; every key block of the range is kept. Writes, per query, the
// unnormalised output sum_u 2^(c s_u - m) V_u (fp32), its reference m (log2 domain) and the
// sum l of the same weights. Partial index: (bh S + s) P + p.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, 2) void probe_partial_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                                  const void* __restrict__ v, int N, int nqb, int nkb,
                                                                  int P, int S, float c_log2, float* __restrict__ part_o,
                                                                  float* __restrict__ part_ml) {
  using C = DCfg<D, BQ>;
  __shared__ __attribute__((aligned(1024))) char buf0_[2 * C::TILE];
  __shared__ __attribute__((aligned(1024))) char buf1_[2 * C::TILE];
  lchar* const buf0 = (lchar*)buf0_;
  lchar* const buf1 = (lchar*)buf1_;

  // the P probes of one range run on one XCD and share its L2 for the key / value blocks
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  const int p = unit % P;
  const int s = (unit / P) % S;
  const int bh = unit / (P * S);
  const int qb = probe_block(p, P, nqb, N, BQ);
  const int kb0 = (int)((long long)s * nkb / S), kb1 = (int)((long long)(s + 1) * nkb / S);
  const int cnt = kb1 - kb0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31;
  const int hf = lane >> 5;

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;
  uint32_t doff[C::PER_WAVE];
  dma_offsets<D, BQ>(wave, lane, doff);
  if (cnt > 0) {
    dma_tile<D, BQ>(kbase, kb0, N, wave, lane, doff, buf0);
    dma_tile<D, BQ>(vbase, kb0, N, wave, lane, doff, buf0 + C::TILE);
  }
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

  for (int t = 0; t < cnt; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block t is resident; every wave is done with block t - 1
    if (t + 1 < cnt) {
      lchar* nb = (t & 1) ? buf0 : buf1;
      dma_tile<D, BQ>(kbase, kb0 + t + 1, N, wave, lane, doff, nb);
      dma_tile<D, BQ>(vbase, kb0 + t + 1, N, wave, lane, doff, nb + C::TILE);
    }
    const lchar* kt = (t & 1) ? buf1 : buf0;
    lchar* vt = ((t & 1) ? buf1 : buf0) + C::TILE;
    const int kb = kb0 + t;
    f32x16 s0, s1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[j]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koff[j] + 32 * C::ROWB);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[j], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[j], s1, 0, 0, 0);
    }
    if (kb * BK + BK > N) {  // keys past N in the ragged last block
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (key >= N) s0[i] = -INFINITY;
        if (key + 32 >= N) s1[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
    mx = partner32_max(mx) * c_log2;
    if (__ballot(mx > m_run + 8.f)) {  // lazy rescale: weights stay below 2^8 between raises
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < D / 32; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[r][i] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[4];
    float rs = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t w0[4], w1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s0[8 * u + 2 * e], c_log2, -m_run)),
                          __builtin_amdgcn_exp2f(fmaf(s0[8 * u + 2 * e + 1], c_log2, -m_run)));
        w1[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s1[8 * u + 2 * e], c_log2, -m_run)),
                          __builtin_amdgcn_exp2f(fmaf(s1[8 * u + 2 * e + 1], c_log2, -m_run)));
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0[e]), ones, rs, false);
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1[e]), ones, rs, false);
      }
      pb[u] = __builtin_bit_cast(bf16x8, make_uint4(w0[0], w0[1], w0[2], w0[3]));
      pb[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(w1[0], w1[1], w1[2], w1[3]));
    }
    l_run += rs;
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

// Grid (BH, ceil((D + 1) / 32)): rows i0 .. i0 + 31 of the (D + 1) x (2 D + 1) matrix [G | C],
// summed in float64 over the probe rows that lie inside the sequence. X = [O_sparse, 1] from the
// bf16 output, R = O_exact - O_sparse.
template <int D>
__global__ __launch_bounds__(256) void probe_gram_kernel(const uint16_t* __restrict__ o, const float* __restrict__ exact,
                                                         int N, int nqb, int BQ, int P, double* __restrict__ gram) {
  constexpr int W = 2 * D + 1;      // columns of [G | C]
  constexpr int CH = 16;            // probe rows per LDS stage
  constexpr int JPT = (W + 7) / 8;  // columns per thread
  __shared__ double z[CH][W + 1];   // [X | R] of CH probe rows
  const int bh = blockIdx.x;
  const int i = blockIdx.y * 32 + (threadIdx.x & 31);
  const int jg = threadIdx.x >> 5;  // this thread's columns: jg, jg + 8, ...
  double acc[JPT];
#pragma unroll
  for (int t = 0; t < JPT; ++t) acc[t] = 0.0;
  const int m = P * BQ;
  for (int r0 = 0; r0 < m; r0 += CH) {
    __syncthreads();
    for (int e = threadIdx.x; e < CH * (D + 1); e += 256) {
      const int rr = e / (D + 1), c = e % (D + 1);
      const int pr = r0 + rr;
      const int p = pr / BQ, qq = pr % BQ;
      double xs = 0.0, xe = 0.0;
      if (pr < m) {
        const int tok = probe_block(p, P, nqb, N, BQ) * BQ + qq;
        if (tok < N) {
          if (c < D) {
            xs = (double)__uint_as_float((uint32_t)o[((size_t)bh * N + tok) * D + c] << 16);
            xe = (double)exact[(((size_t)bh * P + p) * BQ + qq) * D + c];
          } else {
            xs = 1.0;
          }
        }
      }
      z[rr][c] = xs;
      if (c < D) z[rr][D + 1 + c] = xe - xs;
    }
    __syncthreads();
    if (i <= D) {
#pragma unroll 1
      for (int rr = 0; rr < CH; ++rr) {
        const double xi = z[rr][i];
#pragma unroll
        for (int t = 0; t < JPT; ++t) {
          const int j = jg + 8 * t;
          if (j < W) acc[t] = fma(xi, z[rr][j], acc[t]);
        }
      }
    }
  }
  if (i <= D) {
#pragma unroll
    for (int t = 0; t < JPT; ++t) {
      const int j = jg + 8 * t;
      if (j < W) gram[((size_t)bh * (D + 1) + i) * W + j] = acc[t];
    }
  }
}

// ---------------------------------------------------------------- 4. ridge solve

// One workgroup (4 waves) per head, float64. The lower triangle of G + mu I is factorised in
// packed storage (row r at offset r (r + 1) / 2; the pivots are kept apart) by right-looking
// Cholesky steps, then the D right-hand sides C are solved 64 columns at a time (lane = column)
// by blocked forward and back substitution: 32-row blocks, whose updates from the solved rows use
// all four waves and whose diagonal triangles use one. Writes A (fp32 [D + 1][D]), A[0:D]^T as
// bf16 [D][D] (the apply kernel's operand) and the bias row A[D] (fp32).
template <int D>
__global__ __launch_bounds__(256) void probe_solve_kernel(const double* __restrict__ gram, double ridge,
                                                          float* __restrict__ a_out, __bf16* __restrict__ at_out,
                                                          float* __restrict__ bias_out) {
  constexpr int n = D + 1, W = 2 * D + 1, G = 64, YS = G + 1, RB = 32;
  extern __shared__ __attribute__((aligned(16))) double sm[];
  double* L = sm;                    // n (n + 1) / 2, packed lower triangle
  double* Y = sm + n * (n + 1) / 2;  // n x YS, right-hand sides / solution columns
  __shared__ double piv[n];
  __shared__ double red[256];
  const int bh = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const double* g = gram + (size_t)bh * n * W;
  auto at = [](int r, int c) { return r * (r + 1) / 2 + c; };

  for (int r = wave; r < n; r += 4)
    for (int c = lane; c <= r; c += 64) L[at(r, c)] = g[(size_t)r * W + c];
  double tr = 0.0;
  for (int r = tid; r < n; r += 256) tr += g[(size_t)r * W + r];
  red[tid] = tr;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const double mu = ridge * red[0] / n;
  for (int r = tid; r < n; r += 256) L[at(r, r)] += mu;
  __syncthreads();

  for (int kk = 0; kk < n; ++kk) {
    const double pk = sqrt(L[at(kk, kk)]);  // > 0: G + mu I is positive definite for mu > 0
    if (tid == 0) piv[kk] = pk;
    const double inv = 1.0 / pk;
    for (int r = kk + 1 + tid; r < n; r += 256) L[at(r, kk)] *= inv;
    __syncthreads();
    for (int r = kk + 1 + wave; r < n; r += 4) {
      const double lr = L[at(r, kk)];
      for (int c = kk + 1 + lane; c <= r; c += 64) L[at(r, c)] -= lr * L[at(c, kk)];
    }
    __syncthreads();
  }

  for (int c0 = 0; c0 < D; c0 += G) {
    for (int r = wave; r < n; r += 4) Y[r * YS + lane] = c0 + lane < D ? g[(size_t)r * W + n + c0 + lane] : 0.0;
    __syncthreads();
    // forward substitution L y = c
    for (int r0 = 0; r0 < n; r0 += RB) {
      const int rb = min(RB, n - r0);
      if (r0 > 0) {
        for (int i = wave; i < rb; i += 4) {
          const int row = r0 + i;
          double s = 0.0;
          for (int j = 0; j < r0; ++j) s = fma(L[at(row, j)], Y[j * YS + lane], s);
          Y[row * YS + lane] -= s;
        }
        __syncthreads();
      }
      if (wave == 0) {
        for (int i = 0; i < rb; ++i) {
          const int row = r0 + i;
          double s = Y[row * YS + lane];
          for (int j = r0; j < row; ++j) s -= L[at(row, j)] * Y[j * YS + lane];
          Y[row * YS + lane] = s / piv[row];
        }
      }
      __syncthreads();
    }
    // back substitution L^T a = y
    for (int r1 = n; r1 > 0; r1 -= RB) {
      const int r0 = max(0, r1 - RB);
      if (r1 < n) {
        for (int i = wave; i < r1 - r0; i += 4) {
          const int row = r0 + i;
          double s = 0.0;
          for (int j = r1; j < n; ++j) s = fma(L[at(j, row)], Y[j * YS + lane], s);
          Y[row * YS + lane] -= s;
        }
        __syncthreads();
      }
      if (wave == 0) {
        for (int row = r1 - 1; row >= r0; --row) {
          double s = Y[row * YS + lane];
          for (int j = row + 1; j < r1; ++j) s -= L[at(j, row)] * Y[j * YS + lane];
          Y[row * YS + lane] = s / piv[row];
        }
      }
      __syncthreads();
    }
    if (c0 + lane < D) {
      for (int r = wave; r < n; r += 4) a_out[((size_t)bh * n + r) * D + c0 + lane] = (float)Y[r * YS + lane];
      if (wave == 0) bias_out[(size_t)bh * D + c0 + lane] = (float)Y[D * YS + lane];
    }
    for (int c = wave; c < G && c0 + c < D; c += 4)
      for (int r = lane; r < D; r += 64) at_out[((size_t)bh * D + c0 + c) * D + r] = (__bf16)Y[r * YS + c];
    __syncthreads();
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
  for (int r0 = t0; r0 < t1; r0 += 64) {
    __syncthreads();  // the previous tile's stores have read ot; A^T is resident
    for (int e = tid; e < 64 * CPR; e += 256) {
      const int r = e / CPR, c = e % CPR;
      *reinterpret_cast<uint4*>(ot + r * PADB + c * 16) =
          r0 + r < N ? *reinterpret_cast<const uint4*>(oh + (size_t)(r0 + r) * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
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
  size_t part_o, part_ml, exact, gram, amat, at, bias, total;
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
  off += al256((size_t)BH * (d + 1) * (2 * d + 1) * 8);
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
                                 int P, double ridge, float* a_user, float* exact_user, void* ws, hipStream_t stream) {
  const int nqb = (N + BQ - 1) / BQ, nkb = (N + BK - 1) / BK;
  const int S = probe_splits(BH, P, nkb);
  const ProbeWs w = probe_ws_layout(BH, N, D, BQ, P);
  char* base = static_cast<char*>(ws);
  float* part_o = reinterpret_cast<float*>(base + w.part_o);
  float* part_ml = reinterpret_cast<float*>(base + w.part_ml);
  float* exact = exact_user ? exact_user : reinterpret_cast<float*>(base + w.exact);
  double* gram = reinterpret_cast<double*>(base + w.gram);
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
  hipLaunchKernelGGL((probe_gram_kernel<D>), dim3((unsigned)BH, (unsigned)((D + 1 + 31) / 32)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(o), exact, N, nqb, BQ, P, gram);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr int n = D + 1;
  const size_t smem = ((size_t)n * (n + 1) / 2 + (size_t)n * 65) * sizeof(double);
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&probe_solve_kernel<D>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((probe_solve_kernel<D>), dim3((unsigned)BH), dim3(256), smem, stream, gram, ridge, amat, at, bias);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int tph = (N + kApplyRows - 1) / kApplyRows;
  hipLaunchKernelGGL((probe_apply_kernel<D>), dim3((unsigned)(BH * tph)), dim3(256), 0, stream,
                     static_cast<uint16_t*>(o), at, bias, N, tph, kApplyRows);
  return hipGetLastError();
}

hipError_t launch_probe(const void* q, const void* k, const void* v, void* o, int BH, int N, int d, int Bq,
                        double scale, int P, double ridge, float* a_user, float* exact_user, void* ws,
                        hipStream_t stream) {
  const float sc = (float)scale;
  if (d == 128 && Bq == 128) return launch_probe_t<128, 128>(q, k, v, o, BH, N, sc, P, ridge, a_user, exact_user, ws, stream);
  if (d == 128 && Bq == 64) return launch_probe_t<128, 64>(q, k, v, o, BH, N, sc, P, ridge, a_user, exact_user, ws, stream);
  if (d == 64 && Bq == 128) return launch_probe_t<64, 128>(q, k, v, o, BH, N, sc, P, ridge, a_user, exact_user, ws, stream);
  if (d == 64 && Bq == 64) return launch_probe_t<64, 64>(q, k, v, o, BH, N, sc, P, ridge, a_user, exact_user, ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
