// Semantic-aware permutation with centroid Top-p and attention over variable-size blocks (gfx950).
//
// Page "Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via Semantic-Aware
// Permutation" (gist.science summary), section "2. 手法":
//   A. k-means clusters of Q and of K; tokens permuted so that every cluster is contiguous; the
//      output, permuted back, equals attention in the original order.
//   B. scores between cluster centroids, clusters taken in descending order of estimated score
//      until the running sum reaches p.
//   C. attention over variable-size blocks: dense contiguous queries, sparse key/value loads.
// Kernels:
//   km_init / km_assign / km_rank / km_scan / km_scatter / km_update   Lloyd's k-means; the
//       assignment runs on bf16 MFMA with every centroid split into a high and a low bf16 part
//       (about 16 mantissa bits), the permutation is a stable counting sort, and the update is a
//       float64 mean over each cluster's contiguous run of the permuted order (deterministic).
//   cluster_select    float64 centroid scores, size-weighted softmax, sort, Top-p cut.
//   permute_rows      gather (or scatter) of [N, d] rows by a permutation.
//   cluster_tiles     query tiles of up to BQ rows inside each query cluster.
//   attn_var          flash attention of one query tile over the concatenated keys of its kept
//                     key clusters: every lane's DMA fetches its own key row, so 64-key tiles are
//                     filled across cluster boundaries and only the stream's last tile is partial.
#include <algorithm>

#include "attn_tiles.h"

namespace sa {

constexpr int KM_MAXC = 1024;  // clusters per head
constexpr int KM_CH = 256;     // tokens per chunk of the counting sort

// Exclusive prefix sum of v over the NT threads of the workgroup; returns this thread's prefix
// and writes the total to *total. scratch holds NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) scratch[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = scratch[w];
    if (w < wave) base += s;
    tot += s;
  }
  *total = tot;
  __syncthreads();  // scratch may be reused by the caller
  return base + inc - v;
}

// ---------------------------------------------------------------- k-means

// Operands of the assignment for centroid c of head bh: high and low bf16 parts (padded rows
// past C are zero) and the fp32 squared norm (+inf for padded rows, which are never chosen).
// Called by every thread of the workgroup; threads 0 .. D - 1 hold channel vch.
template <int D, int NT>
__device__ __forceinline__ void km_write_operands(const float vch, int bh, int c, int C, int CP, __bf16* chi,
                                                  __bf16* clo, float* cn, float* red) {
  const int ch = threadIdx.x;
  float sq = 0.f;
  if (ch < D) {
    const __bf16 hi = (__bf16)vch;
    const __bf16 lo = (__bf16)(vch - (float)hi);
    chi[((size_t)bh * CP + c) * D + ch] = hi;
    clo[((size_t)bh * CP + c) * D + ch] = lo;
    sq = vch * vch;
  }
  for (int o = 32; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 64);
  if ((ch & 63) == 0) red[ch >> 6] = sq;
  __syncthreads();
  if (ch == 0) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += red[w];
    cn[(size_t)bh * CP + c] = c < C ? s : INFINITY;
  }
}

// Grid (BH, CP), D threads: centroid c starts at token floor((2c + 1) N / (2C)), or at init.
template <int D>
__global__ __launch_bounds__(D) void km_init_kernel(const uint16_t* __restrict__ x, const float* __restrict__ init,
                                                    int N, int C, int CP, float* __restrict__ cen,
                                                    __bf16* __restrict__ chi, __bf16* __restrict__ clo,
                                                    float* __restrict__ cn) {
  __shared__ float red[D / 64];
  const int bh = blockIdx.x, c = blockIdx.y, ch = threadIdx.x;
  float v = 0.f;
  if (c < C) {
    if (init != nullptr) {
      v = init[((size_t)bh * C + c) * D + ch];
    } else {
      const long long tok = ((2LL * c + 1) * N) / (2LL * C);
      v = __uint_as_float((uint32_t)x[((size_t)bh * N + tok) * D + ch] << 16);
    }
    cen[((size_t)bh * C + c) * D + ch] = v;
  }
  km_write_operands<D, D>(v, bh, c, C, CP, chi, clo, cn, red);
}

// Grid (BH, ceil(N / 256)), 4 waves of 64 tokens (two sets of 32). Centroids stream through LDS
// 64 at a time; per 32-centroid tile, S^T = (C_hi + C_lo) X^T on bf16 MFMA (element i of lane j:
// centroid 8 (i / 4) + 4 (j / 32) + i % 4 of the tile, token j % 32), then dist = |c|^2 - 2 <x, c>.
// Each lane visits its centroids in ascending order and keeps the first strict minimum; the two
// halves of a token's centroids are merged with the lower index on equality.
template <int D>
__global__ __launch_bounds__(256) void km_assign_kernel(const uint16_t* __restrict__ x, const __bf16* __restrict__ chi,
                                                        const __bf16* __restrict__ clo, const float* __restrict__ cn,
                                                        int N, int CP, int32_t* __restrict__ labels) {
  constexpr int CT = 64;               // centroids per LDS stage
  constexpr int RB = 2 * D + 16;       // padded LDS row (bytes)
  __shared__ __attribute__((aligned(16))) char hs[CT * RB];
  __shared__ __attribute__((aligned(16))) char ls[CT * RB];
  __shared__ float cns[KM_MAXC];
  const int bh = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 31, hf = lane >> 5;
  for (int c = tid; c < CP; c += 256) cns[c] = cn[(size_t)bh * CP + c];
  const uint16_t* xh = x + (size_t)bh * N * D;
  bf16x8 xf[2][D / 16];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int t = blockIdx.y * 256 + wave * 64 + s * 32 + ln;
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
      xf[s][j] = __builtin_bit_cast(bf16x8, t < N ? *reinterpret_cast<const uint4*>(xh + (size_t)t * D + 16 * j + 8 * hf)
                                                  : make_uint4(0, 0, 0, 0));
  }
  float best[2] = {INFINITY, INFINITY};
  int bidx[2] = {0, 0};
  const char* hg = reinterpret_cast<const char*>(chi + (size_t)bh * CP * D);
  const char* lg = reinterpret_cast<const char*>(clo + (size_t)bh * CP * D);
  for (int c0 = 0; c0 < CP; c0 += CT) {
    const int rows = min(CT, CP - c0);
    __syncthreads();  // the previous stage has been read (and cns is resident)
    for (int e = tid; e < rows * (2 * D / 16); e += 256) {
      const int r = e / (2 * D / 16), k = e % (2 * D / 16);
      *reinterpret_cast<uint4*>(hs + r * RB + k * 16) = *reinterpret_cast<const uint4*>(hg + (size_t)(c0 + r) * 2 * D + k * 16);
      *reinterpret_cast<uint4*>(ls + r * RB + k * 16) = *reinterpret_cast<const uint4*>(lg + (size_t)(c0 + r) * 2 * D + k * 16);
    }
    __syncthreads();
    for (int ct = 0; ct < rows; ct += 32) {
      f32x16 acc[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[s][i] = 0.f;
#pragma unroll
      for (int j = 0; j < D / 16; ++j) {
        const int off = (ct + ln) * RB + (16 * j + 8 * hf) * 2;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(hs + off);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(ls + off);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xf[s][j], acc[s], 0, 0, 0);
          acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xf[s][j], acc[s], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = c0 + ct + 8 * (i >> 2) + 4 * hf + (i & 3);
        const float cnv = cns[c];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float dv = fmaf(-2.f, acc[s][i], cnv);
          if (dv < best[s]) {
            best[s] = dv;
            bidx[s] = c;
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float pb = __shfl_xor(best[s], 32, 64);
    const int pi = __shfl_xor(bidx[s], 32, 64);
    if (pb < best[s] || (pb == best[s] && pi < bidx[s])) bidx[s] = pi;
    const int t = blockIdx.y * 256 + wave * 64 + s * 32 + ln;
    if (hf == 0 && t < N) labels[(size_t)bh * N + t] = bidx[s];
  }
}

// Counting sort, pass 1. Grid (BH, ceil(N / 256)): for every token, the number of earlier tokens
// of its chunk with the same label; per chunk, the count of every label (all C of them), stored
// label-major (hist[bh][label][chunk]) so that each label's counts are contiguous for pass 2.
__global__ __launch_bounds__(KM_CH) void km_rank_kernel(const int32_t* __restrict__ labels, int N, int C, int nch,
                                                       int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  constexpr int NW = KM_CH / 64;
  __shared__ int lab[KM_CH];
  __shared__ int cnt[NW][KM_MAXC];  // per-wave label counts
  const int bh = blockIdx.x, ch = blockIdx.y, tid = threadIdx.x, wave = tid >> 6;
  const int t = ch * KM_CH + tid;
  for (int c = tid; c < C; c += KM_CH)
#pragma unroll
    for (int w = 0; w < NW; ++w) cnt[w][c] = 0;
  const int my = t < N ? labels[(size_t)bh * N + t] : -1;
  lab[tid] = my;
  __syncthreads();
  // earlier lanes of this wave with the same label, then the counts of the earlier waves
  int r = 0;
  for (int u = wave * 64; u < tid; ++u) r += lab[u] == my;
  if (t < N) atomicAdd(&cnt[wave][my], 1);  // counts only: the order of the additions does not matter
  __syncthreads();
  if (t < N) {
    for (int w = 0; w < wave; ++w) r += cnt[w][my];
    rank[(size_t)bh * N + t] = r;
  }
  int32_t* hh = hist + (size_t)bh * C * nch + ch;
  for (int c = tid; c < C; c += KM_CH) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n += cnt[w][c];
    hh[(size_t)c * nch] = n;
  }
}

// Pass 2a. Grid (BH, ceil(C / 16)), 16 waves, one label per wave: exclusive prefix of the label's
// chunk counts over the chunks, in place (lane l owns a contiguous run of chunks: its run sum, a
// wave scan of the sums, then the run rewritten), and the label total into offsets[label].
__global__ __launch_bounds__(1024) void km_scan_kernel(int32_t* __restrict__ hist, int C, int nch,
                                                      int32_t* __restrict__ offsets) {
  const int bh = blockIdx.x, lane = threadIdx.x & 63;
  const int c = blockIdx.y * 16 + (threadIdx.x >> 6);
  if (c >= C) return;  // whole waves
  int32_t* h = hist + ((size_t)bh * C + c) * nch;
  const int per = (nch + 63) / 64;
  const int k0 = min(nch, lane * per), k1 = min(nch, k0 + per);
  int sum = 0;
  for (int k = k0; k < k1; ++k) sum += h[k];
  int inc = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  int run = inc - sum;
  for (int k = k0; k < k1; ++k) {
    const int v = h[k];
    h[k] = run;
    run += v;
  }
  if (lane == 63) offsets[(size_t)bh * (C + 1) + c] = inc;
}

// Pass 2b. Grid BH, 1024 threads (thread = label): offsets[c] = the exclusive prefix of the label
// totals, offsets[C] = N; and the order in which the centroid update visits the clusters, largest
// first (ties to the lower label): ord[bh][r] = the label of rank r, ord[bh][r] = r for the
// padding ranks C <= r < CP. One workgroup sums one cluster, so the largest clusters set the
// update's time unless they start first.
__global__ __launch_bounds__(KM_MAXC) void km_offsets_kernel(int C, int CP, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ ord) {
  __shared__ int scratch[KM_MAXC / 64];
  __shared__ int sz[KM_MAXC];
  const int bh = blockIdx.x, c = threadIdx.x;
  int32_t* off = offsets + (size_t)bh * (C + 1);
  const int v = c < C ? off[c] : 0;
  if (c < C) sz[c] = v;
  int total;
  const int ex = block_exclusive_scan<KM_MAXC>(v, scratch, &total);
  if (c < C) off[c] = ex;
  if (c == 0) off[C] = total;
  __syncthreads();  // sz is complete
  if (c < C) {
    int r = 0;
    for (int j = 0; j < C; ++j) r += (sz[j] > v) | ((sz[j] == v) & (j < c));
    ord[(size_t)bh * CP + r] = c;
  } else if (c < CP) {
    ord[(size_t)bh * CP + c] = c;
  }
}

// Pass 3. Grid (BH, ceil(N / 256)): perm[offsets[l] + chunk base[l] + rank] = token.
__global__ __launch_bounds__(KM_CH) void km_scatter_kernel(const int32_t* __restrict__ labels,
                                                          const int32_t* __restrict__ rank,
                                                          const int32_t* __restrict__ hist,
                                                          const int32_t* __restrict__ offsets, int N, int C, int nch,
                                                          int32_t* __restrict__ perm) {
  const int bh = blockIdx.x, ch = blockIdx.y;
  const int t = ch * KM_CH + threadIdx.x;
  if (t >= N) return;
  const int l = labels[(size_t)bh * N + t];
  const int pos = offsets[(size_t)bh * (C + 1) + l] + hist[((size_t)bh * C + l) * nch + ch] + rank[(size_t)bh * N + t];
  perm[(size_t)bh * N + pos] = t;
}

// Grid (BH, CP), 256 threads: centroid c = the float64 mean of its tokens (an empty cluster keeps
// its centroid), then its MFMA operands. Thread (r, cs) sums channels 8 cs .. 8 cs + 7 (one
// 16-byte load per row) over the members o0 + r, o0 + r + RS, ... of the cluster's run of the
// permuted order, eight rows in flight; the RS partial sums of a channel are added in the order
// of r, so the result is deterministic.
// Workgroup (bh, r) takes cluster ord[bh][r], so that the grid's first round holds the largest
// clusters of every head.
template <int D>
__global__ __launch_bounds__(256) void km_update_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ ord, int N, int C, int CP,
                                                        float* __restrict__ cen, __bf16* __restrict__ chi,
                                                        __bf16* __restrict__ clo, float* __restrict__ cn) {
  constexpr int LPR = D / 8;    // lanes per row: 16 bytes (8 channels) each
  constexpr int RS = 256 / LPR;  // row slots: members o0 + r, o0 + r + RS, ... go to slot r
  __shared__ double part[RS][D];
  __shared__ float red[4];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int c = min(max(ord[(size_t)bh * CP + blockIdx.y], 0), CP - 1);
  const int r = tid / LPR, cs = tid % LPR;
  int o0 = 0, o1 = 0;
  if (c < C) {
    o0 = offsets[(size_t)bh * (C + 1) + c];
    o1 = offsets[(size_t)bh * (C + 1) + c + 1];
  }
  const char* xh = reinterpret_cast<const char*>(x) + (size_t)bh * N * D * 2 + cs * 16;
  const int32_t* pp = perm + (size_t)bh * N;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  auto add = [&](const uint4 w) {
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)__uint_as_float(q[e] << 16);
      acc[2 * e + 1] += (double)__uint_as_float(q[e] & 0xffff0000u);
    }
  };
  int m = o0 + r;
  for (; m + 7 * RS < o1; m += 8 * RS) {  // eight gathered rows in flight
    uint4 b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) b[u] = *reinterpret_cast<const uint4*>(xh + (size_t)pp[m + u * RS] * D * 2);
#pragma unroll
    for (int u = 0; u < 8; ++u) add(b[u]);
  }
  for (; m < o1; m += RS) add(*reinterpret_cast<const uint4*>(xh + (size_t)pp[m] * D * 2));
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r][cs * 8 + e] = acc[e];
  __syncthreads();
  float v = 0.f;
  const int ch = tid;
  if (tid < D && c < C) {
    float* cp = cen + ((size_t)bh * C + c) * D + ch;
    if (o1 > o0) {
      double sm = part[0][ch];
#pragma unroll
      for (int h = 1; h < RS; ++h) sm += part[h][ch];
      v = (float)(sm / (double)(o1 - o0));
      *cp = v;
    } else {
      v = *cp;
    }
  }
  km_write_operands<D, 256>(v, bh, c, C, CP, chi, clo, cn, red);
}

// ---------------------------------------------------------------- centroid Top-p

// Grid (BH, Cq), 256 threads. Row i: S_ij = scale <cq_i, ck_j> (float64), weights
// n_j exp(S_ij - max) over the non-empty key clusters, probabilities = weights / their sum;
// bitonic sort by (probability descending, index ascending); the kept length is
// min(#non-empty, max(1, m*)) with m* the first prefix whose sequential running sum reaches p.
__global__ __launch_bounds__(256) void cluster_select_kernel(const float* __restrict__ cq, const float* __restrict__ ck,
                                                             const int32_t* __restrict__ koff, int Cq, int Ck, int d,
                                                             double scale, double p, double* __restrict__ probs,
                                                             uint8_t* __restrict__ mask) {
  __shared__ double qrow[128];
  __shared__ double pv[KM_MAXC];
  __shared__ int pi[KM_MAXC];
  __shared__ double red[4];
  __shared__ int keep_len;
  const int bh = blockIdx.x, i = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < d; e += 256) qrow[e] = (double)cq[((size_t)bh * Cq + i) * d + e];
  int np = 1;
  while (np < Ck) np <<= 1;
  __syncthreads();
  double lmax = -INFINITY;
  for (int j = tid; j < Ck; j += 256) {
    const float* kr = ck + ((size_t)bh * Ck + j) * d;
    double s = 0.0;
    for (int e = 0; e < d; ++e) s = fma(qrow[e], (double)kr[e], s);
    s *= scale;
    const int n = koff[(size_t)bh * (Ck + 1) + j + 1] - koff[(size_t)bh * (Ck + 1) + j];
    pv[j] = n > 0 ? s : -INFINITY;
    lmax = fmax(lmax, pv[j]);
  }
  for (int o = 32; o > 0; o >>= 1) lmax = fmax(lmax, __shfl_xor(lmax, o, 64));
  if (lane == 0) red[wave] = lmax;
  __syncthreads();
  const double M = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double lsum = 0.0;
  for (int j = tid; j < Ck; j += 256) {
    const int n = koff[(size_t)bh * (Ck + 1) + j + 1] - koff[(size_t)bh * (Ck + 1) + j];
    const double w = n > 0 ? (double)n * exp(pv[j] - M) : 0.0;
    pv[j] = w;
    lsum += w;
  }
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o, 64);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  const double tot = (red[0] + red[1]) + (red[2] + red[3]);
  for (int j = tid; j < np; j += 256) {
    if (j < Ck) {
      pv[j] /= tot;
      if (probs != nullptr) probs[((size_t)bh * Cq + i) * Ck + j] = pv[j];
    } else {
      pv[j] = -1.0;  // padding sorts last
    }
    pi[j] = j;
  }
  // bitonic sort into descending probability, ascending index on equality
  for (int k = 2; k <= np; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      __syncthreads();
      for (int e = tid; e < np; e += 256) {
        const int f = e ^ jj;
        if (f > e) {
          const bool up = (e & k) == 0;  // this run is ordered "first before"
          const double a = pv[e], b = pv[f];
          const int ia = pi[e], ib = pi[f];
          const bool a_first = a > b || (a == b && ia < ib);
          if (a_first != up) {
            pv[e] = b;
            pv[f] = a;
            pi[e] = ib;
            pi[f] = ia;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int nnz = 0, mstar = Ck;
    double run = 0.0;
    bool hit = p <= 0.0;
    if (hit) mstar = 0;
    for (int s = 0; s < Ck; ++s) {
      if (pv[s] > 0.0) ++nnz;
      if (!hit) {
        run += pv[s];
        if (run >= p) {
          hit = true;
          mstar = s + 1;
        }
      }
    }
    keep_len = min(nnz, max(1, mstar));
  }
  uint8_t* mrow = mask + ((size_t)bh * Cq + i) * Ck;
  for (int j = tid; j < Ck; j += 256) mrow[j] = 0;
  __syncthreads();
  for (int s = tid; s < keep_len; s += 256) mrow[pi[s]] = 1;
}

// ---------------------------------------------------------------- permutation of rows

// One thread per 16-byte piece: out[t'] = x[perm[t']] (gather) or out[perm[t']] = x[t'] (scatter).
__global__ __launch_bounds__(256) void permute_rows_kernel(const char* __restrict__ x, const int32_t* __restrict__ perm,
                                                           int N, int row_bytes, int inverse, long long pieces,
                                                           char* __restrict__ out) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= pieces) return;
  const int per = row_bytes / 16;
  const long long row = e / per;
  const int k = (int)(e % per);
  const long long bh = row / N;
  const int t = (int)(row % N);
  const long long src = inverse ? row : bh * N + perm[row];
  const long long dst = inverse ? bh * N + perm[row] : row;
  (void)t;
  *reinterpret_cast<uint4*>(out + dst * row_bytes + k * 16) = *reinterpret_cast<const uint4*>(x + src * row_bytes + k * 16);
}

// ---------------------------------------------------------------- variable-size blocks

// Grid BH, 1024 threads (thread = query cluster): query tiles (cluster, first row, rows) of at
// most BQ rows inside every cluster of the permuted query order.
__global__ __launch_bounds__(KM_MAXC) void cluster_tiles_kernel(const int32_t* __restrict__ qoff, int Cq, int BQ,
                                                               int max_tiles, int4* __restrict__ tiles,
                                                               int32_t* __restrict__ ntiles) {
  __shared__ int scratch[KM_MAXC / 64];
  const int bh = blockIdx.x, i = threadIdx.x;
  int o0 = 0, n = 0;
  if (i < Cq) {
    o0 = qoff[(size_t)bh * (Cq + 1) + i];
    n = qoff[(size_t)bh * (Cq + 1) + i + 1] - o0;
  }
  const int nt = (n + BQ - 1) / BQ;
  int total;
  const int base = block_exclusive_scan<KM_MAXC>(nt, scratch, &total);
  for (int t = 0; t < nt; ++t)
    tiles[(size_t)bh * max_tiles + base + t] = make_int4(i, o0 + t * BQ, min(BQ, n - t * BQ), 0);
  if (i == 0) ntiles[bh] = total;
}

// Key tile t of the stream: var_rows gives the key row behind each of the lane's DMA pieces
// (stream position pos lies in the range e with cum[e] <= pos < cum[e + 1]; the lane's cursor
// cur[u] only moves forward because positions grow with t).
template <int D, int BQ>
__device__ __forceinline__ void var_rows(int t, int L, const __attribute__((address_space(3))) int* cum,
                                         const __attribute__((address_space(3))) int* rstart, int trow0,
                                         int (&cur)[DCfg<D, BQ>::PER_WAVE], int (&row)[DCfg<D, BQ>::PER_WAVE]) {
  using C = DCfg<D, BQ>;
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) {
    const int pos = min(t * BK + trow0 + u * (1024 / C::ROWB), L - 1);
    while (cum[cur[u] + 1] <= pos) ++cur[u];
    row[u] = rstart[cur[u]] + pos - cum[cur[u]];
  }
}

// Copy of one tensor's rows of a key tile (K or V) into dst: var_rows gives the row behind each of
// the lane's DMA pieces.
template <int D, int BQ>
__device__ __forceinline__ void var_dma1(const char* __restrict__ base, int N, const int (&row)[DCfg<D, BQ>::PER_WAVE],
                                         int trow0, int c0, int wave, lchar* dst) {
  using C = DCfg<D, BQ>;
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) {
    // piece u fills tile row trow0 + u (1024 / ROWB), swizzled chunk slot c0
    const uint32_t choff = (uint32_t)((c0 ^ kv_swz<D>(trow0 + u * (1024 / C::ROWB))) << 4);
    // a 32-bit lane offset from the uniform head base (one head's rows stay below 4 GiB); the
    // empty asm keeps the compiler from widening it to a 64-bit per-lane address
    uint32_t off = (uint32_t)min(max(row[u], 0), N - 1) * C::ROWB + choff;
    asm volatile("" : "+v"(off));
    __builtin_amdgcn_global_load_lds(base + off, dst + (wave * C::PER_WAVE + u) * 1024, 16, 0, 0);
  }
}

// One workgroup per query tile (i, qs, qc) of head bh. The key stream of cluster i is the
// concatenation, in ascending cluster order, of the key ranges [koff[j], koff[j + 1]) of its kept
// clusters j; cum[] holds the stream position where each range starts. Key tile t covers stream
// positions 64 t .. 64 t + 63: the DMA lane that fills row r of the tile follows a cursor through
// the ranges (positions only grow, so it never moves back) to key row rstart[e] + pos - cum[e] of
// the key-permuted order, which kperm (when given) maps to the original token. Positions past
// the stream's end are clamped to its last key and get score -inf.
// The main loop is the forward kernel's two-stage software pipeline: step t computes the scores
// of tile t + 1 while the vector units turn the scores of tile t into P and the matrix cores add
// P V of tile t, so K runs one tile ahead of V. The V rows of tile t + 1 are the rows its K copy
// used a step earlier, so one cursor set serves both; the row indices of tile t + 2 are loaded
// one step before their copy is issued.
template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2, BQ == 128 ? 2 : 1) void attn_var_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                             const void* __restrict__ v, int N,
                                                             const int4* __restrict__ tiles,
                                                             const int32_t* __restrict__ ntiles, int max_tiles,
                                                             const int32_t* __restrict__ koff, int Cq, int Ck,
                                                             const int32_t* __restrict__ kidx,
                                                             const int32_t* __restrict__ kcnt,
                                                             const int32_t* __restrict__ qperm,
                                                             const int32_t* __restrict__ kperm, float c_log2,
                                                             void* __restrict__ o, float* __restrict__ lse) {
  using C = DCfg<D, BQ>;
  constexpr int NT = C::NT;
  __shared__ __attribute__((aligned(1024))) char kb0_[C::TILE];
  __shared__ __attribute__((aligned(1024))) char kb1_[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vb0_[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vb1_[C::TILE];
  __shared__ int rstart[KM_MAXC];
  __shared__ int cum[KM_MAXC + 1];
  __shared__ int scratch[NT / 64];
  lchar* const kb0 = (lchar*)kb0_;
  lchar* const kb1 = (lchar*)kb1_;
  lchar* const vb0 = (lchar*)vb0_;
  lchar* const vb1 = (lchar*)vb1_;

  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / max_tiles, tile = w % max_tiles;
  if (tile >= ntiles[bh]) return;  // uniform over the workgroup
  const int4 tl = tiles[(size_t)bh * max_tiles + tile];
  const int ci = tl.x, qs = tl.y, qc = tl.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x, lane = tid & 63, ln = lane & 31, hf = lane >> 5;

  // the key ranges of the kept clusters and their stream positions
  const int cnt = kcnt[(size_t)bh * Cq + ci];
  const int32_t* list = kidx + ((size_t)bh * Cq + ci) * Ck;
  const int32_t* ko = koff + (size_t)bh * (Ck + 1);
  constexpr int PT = (KM_MAXC + NT - 1) / NT;
  int sz[PT], lsum = 0;
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = tid * PT + u;
    sz[u] = 0;
    if (e < cnt) {
      const int j = list[e];
      rstart[e] = ko[j];
      sz[u] = ko[j + 1] - ko[j];
    }
    lsum += sz[u];
  }
  int L;
  int run = block_exclusive_scan<NT>(lsum, scratch, &L);
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int e = tid * PT + u;
    if (e < cnt) cum[e] = run;
    run += sz[u];
  }
  if (tid == 0) cum[cnt] = L;
  __syncthreads();
  const int ntk = (L + BK - 1) / BK;

  const size_t head_off = (size_t)bh * N * D * 2;
  const char* qbase = static_cast<const char*>(q) + head_off;
  const char* kbase = static_cast<const char*>(k) + head_off;
  const char* vbase = static_cast<const char*>(v) + head_off;
  // this lane's DMA pieces: piece u fills 16 bytes of tile row trow0 + u (1024 / ROWB) at chunk
  // slot c0 (1024-byte stretches hold whole rows, so the slot is the same for every piece)
  const int trow0 = (wave * C::PER_WAVE * 1024 + lane * 16) / C::ROWB;
  const int c0 = ((lane * 16) % C::ROWB) >> 4;
  int cur[C::PER_WAVE];
#pragma unroll
  for (int u = 0; u < C::PER_WAVE; ++u) cur[u] = 0;
  typedef __attribute__((address_space(3))) const int lint;
  lint* cum_l = (lint*)cum;
  lint* rst_l = (lint*)rstart;
  const int32_t* kp_h = kperm != nullptr ? kperm + (size_t)bh * N : nullptr;
  // rk: rows of the next K tile to copy (tile t + 2 inside step t); rv: rows of the next V tile
  int rk[C::PER_WAVE], rv[C::PER_WAVE];
  if (ntk > 0) {
    var_rows<D, BQ>(0, L, cum_l, rst_l, trow0, cur, rk);
    if (kp_h != nullptr) {
#pragma unroll
      for (int u = 0; u < C::PER_WAVE; ++u) rk[u] = kp_h[rk[u]];
    }
    var_dma1<D, BQ>(kbase, N, rk, trow0, c0, wave, kb0);
    var_dma1<D, BQ>(vbase, N, rk, trow0, c0, wave, vb0);
  }
  if (ntk > 1) {
    var_rows<D, BQ>(1, L, cum_l, rst_l, trow0, cur, rk);
    if (kp_h != nullptr) {
#pragma unroll
      for (int u = 0; u < C::PER_WAVE; ++u) rk[u] = kp_h[rk[u]];
    }
    var_dma1<D, BQ>(kbase, N, rk, trow0, c0, wave, kb1);
#pragma unroll
    for (int u = 0; u < C::PER_WAVE; ++u) rv[u] = rk[u];
  }
  if (ntk > 2) {
    var_rows<D, BQ>(2, L, cum_l, rst_l, trow0, cur, rk);
    if (kp_h != nullptr) {
#pragma unroll
      for (int u = 0; u < C::PER_WAVE; ++u) rk[u] = kp_h[rk[u]];  // in flight until step 0
    }
  }

  // query rows: permuted position qrow; with qperm, Q, O and LSE live in the original token order
  // and row qrow is token qperm[qrow]
  const int32_t* qp_h = qperm != nullptr ? qperm + (size_t)bh * N : nullptr;
  const int qrow = qs + wave * 32 + ln;
  const bool qvalid = wave * 32 + ln < qc;
  const int qtok = qvalid && qp_h != nullptr ? min(max(qp_h[qrow], 0), N - 1) : qrow;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    qf[j] = __builtin_bit_cast(bf16x8, qvalid ? *reinterpret_cast<const uint4*>(qbase + ((size_t)qtok * D + 16 * j + 8 * hf) * 2)
                                              : make_uint4(0, 0, 0, 0));
  int koffs[D / 16];
  {
    const int sw = kv_swz<D>(ln);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) koffs[j] = ln * C::ROWB + (((2 * j + hf) ^ sw) << 4);
  }
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
      const bf16x8 a0 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j]);
      const bf16x8 a1 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j] + 32 * C::ROWB);
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[j], sc[0], 0, 0, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[j], sc[1], 0, 0, 0);
    }
  };
  // stream positions past the end (only in the last tile) get score -inf
  auto mask_tail = [&](f32x16 (&sc)[2], int t) {
    if (t * BK + BK > L) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = t * BK + 8 * (i >> 2) + 4 * hf + (i & 3);
        if (pos >= L) sc[0][i] = -INFINITY;
        if (pos + 32 >= L) sc[1][i] = -INFINITY;
      }
    }
  };
  auto block_max = [&](const f32x16 (&sc)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(sc[0][i], sc[1][i]));
    return partner32_max(mx) * c_log2;
  };
  auto raise_max = [&](float mx) {
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
  };
  // word j (0..15) of P^T packed to bf16: tile h = j & 1, elements 8 u + 2 e and 8 u + 2 e + 1 with
  // u = j >> 3, e = (j >> 1) & 3; the row sum adds the same bf16 values, into partial sum
  // (e & 1) * 2 + h
  auto p_word = [&](const f32x16 (&sc)[2], int j, uint32_t (&pw)[16], float (&rs)[4]) {
    const int h = j & 1, u = j >> 3, e = (j >> 1) & 3;
    pw[j] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(sc[h][8 * u + 2 * e], c_log2, -m_run)),
                      __builtin_amdgcn_exp2f(fmaf(sc[h][8 * u + 2 * e + 1], c_log2, -m_run)));
    asm volatile("" : "+v"(pw[j]));  // keeps the exps here instead of sunk to the P V products
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
  // O^T += V^T P^T; va0 holds key chunk 0's fragments, read earlier, and chunk c + 1 is read while
  // chunk c multiplies
  auto pv = [&](const uint32_t (&pw)[16], lchar* vt, bf16x8 (&va0)[D / 32]) {
    bf16x8 pb[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[u] = __builtin_bit_cast(bf16x8, make_uint4(pw[8 * u], pw[8 * u + 2], pw[8 * u + 4], pw[8 * u + 6]));
      pb[2 + u] = __builtin_bit_cast(bf16x8, make_uint4(pw[8 * u + 1], pw[8 * u + 3], pw[8 * u + 5], pw[8 * u + 7]));
    }
    bf16x8 va[2][D / 32];
#pragma unroll
    for (int r = 0; r < D / 32; ++r) va[0][r] = va0[r];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int r = 0; r < D / 32; ++r) {
        if (c + 1 < 4) va[(c + 1) & 1][r] = vrd(vt, c + 1, r);
        oacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[c & 1][r], pb[c], oacc[r], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (c + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
  };
  // S^T of the tile in kt into sn, interleaved with the P words of sc (two words after each pair of
  // score MFMAs, K fragments read two steps ahead); mid(s) runs after s-step s. The phase is bound
  // by vector issue, so it runs at raised priority: the other wave on the SIMD, usually in its P V
  // products, fills the matrix core around it.
  auto scores_p = [&](const lchar* kt, f32x16 (&sn)[2], const f32x16 (&sc)[2], uint32_t (&pw)[16], float (&rs)[4],
                      auto&& mid) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sn[0][i] = 0.f;
      sn[1][i] = 0.f;
    }
    bf16x8 a0[3], a1[3];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      a0[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j]);
      a1[j] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j] + 32 * C::ROWB);
    }
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      if (j + 2 < D / 16) {
        a0[(j + 2) % 3] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j + 2]);
        a1[(j + 2) % 3] =
            *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(kt + koffs[j + 2] + 32 * C::ROWB);
      }
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[j % 3], qf[j], sn[0], 0, 0, 0);
      if (2 * j < 16) p_word(sc, 2 * j, pw, rs);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[j % 3], qf[j], sn[1], 0, 0, 0);
      if (2 * j + 1 < 16) p_word(sc, 2 * j + 1, pw, rs);
      __builtin_amdgcn_sched_barrier(0);
      mid(j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 2 * (D / 16); j < 16; ++j) p_word(sc, j, pw, rs);
    __builtin_amdgcn_s_setprio(0);
  };

  // Step t: kn / vc hold K(t+1) / V(t); kf / vf receive K(t+2) / V(t+1). NEXT: 1 = a full tile
  // t + 1; 2 = one of the closing steps: tile t + 1 may be the stream's last tile (masked past its
  // end) or absent.
  auto step = [&](int t, const f32x16 (&sc)[2], f32x16 (&sn)[2], const lchar* kn, lchar* vc, lchar* kf, lchar* vf,
                  auto next_tag) {
    constexpr int NEXT = decltype(next_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K(t+1) and V(t) are resident; every wave is done with K(t) and V(t-1)
    const bool next = NEXT == 1 || (NEXT == 2 && t + 1 < ntk);
    // the copies of K(t+2) and V(t+1) go out between the score products (K after the second
    // s-step, V after three quarters of them), where their issue hides under the matrix core
    auto issue = [&](int j) {
      if (j == 1 && t + 2 < ntk) var_dma1<D, BQ>(kbase, N, rk, trow0, c0, wave, kf);
      if (j == 3 * (D / 64) - 1 && t + 1 < ntk) var_dma1<D, BQ>(vbase, N, rv, trow0, c0, wave, vf);
    };
    uint32_t pw[16];
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    if (next) {
      scores_p(kn, sn, sc, pw, rs, issue);
      if constexpr (NEXT == 2) mask_tail(sn, t + 1);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) p_word(sc, j, pw, rs);
      issue(1);
      issue(3 * (D / 64) - 1);
    }
#pragma unroll
    for (int u = 0; u < C::PER_WAVE; ++u) rv[u] = rk[u];
    if (t + 3 < ntk) {
      var_rows<D, BQ>(t + 3, L, cum_l, rst_l, trow0, cur, rk);
      if (kp_h != nullptr) {
#pragma unroll
        for (int u = 0; u < C::PER_WAVE; ++u) rk[u] = kp_h[rk[u]];  // lands with this step's copies
      }
    }
    // the first V^T fragments are read before anything else of the P V half is issued
    bf16x8 va0[D / 32];
#pragma unroll
    for (int r = 0; r < D / 32; ++r) va0[r] = vrd(vc, 0, r);
    __builtin_amdgcn_sched_barrier(0);
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    pv(pw, vc, va0);
    if (next) raise_max(block_max(sn));
  };

  using full = std::integral_constant<int, 1>;
  using closing = std::integral_constant<int, 2>;
  if (ntk > 0) {
    f32x16 sa[2], sb[2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    scores(kb0, sa);
    mask_tail(sa, 0);
    raise_max(block_max(sa));
    // pairs of steps whose next tiles are both before the last one (S alternates between sa and
    // sb, the buffers between their even and odd roles); t stays even
    int t = 0;
    for (; t + 3 < ntk; t += 2) {
      step(t, sa, sb, kb1, vb0, kb0, vb1, full{});
      step(t + 1, sb, sa, kb0, vb1, kb1, vb0, full{});
    }
    // one to three closing steps, one code path: buffers chosen by parity, S moved into sa
    for (; t < ntk; ++t) {
      const bool odd = (t & 1) != 0;
      step(t, sa, sb, odd ? kb0 : kb1, odd ? vb1 : vb0, odd ? kb1 : kb0, odd ? vb0 : vb1, closing{});
#pragma unroll
      for (int h = 0; h < 2; ++h) sa[h] = sb[h];
    }
  }
  __syncthreads();  // every wave is done with the K / V buffers before they stage the output

  // epilogue: O = O^T / l, staged through LDS (two waves per buffer) for row-contiguous stores
  const float l_tot = partner32_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  lchar* ol = ((wave & 1) ? vb0 : kb0) + (wave >> 1) * 32 * C::OROW;
#pragma unroll
  for (int r = 0; r < D / 32; ++r)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ch = 32 * r + 8 * a + 4 * hf;
      const u32x2 wv = {pack_bf16(oacc[r][4 * a] * inv, oacc[r][4 * a + 1] * inv),
                        pack_bf16(oacc[r][4 * a + 2] * inv, oacc[r][4 * a + 3] * inv)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(ol + ln * C::OROW + ch * 2) = wv;
    }
  __syncthreads();
  constexpr int CH16 = D * 2 / 16;
  char* obase = static_cast<char*>(o) + head_off;
#pragma unroll
  for (int e = lane; e < 32 * CH16; e += 64) {
    const int r = e / CH16, cc = e % CH16;
    if (wave * 32 + r < qc) {
      const int pos = qs + wave * 32 + r;
      const int tok = qp_h != nullptr ? min(max(qp_h[pos], 0), N - 1) : pos;
      *reinterpret_cast<u32x4*>(obase + (size_t)tok * D * 2 + cc * 16) =
          *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(ol + r * C::OROW + cc * 16);
    }
  }
  if (lse != nullptr && hf == 0 && qvalid)
    lse[(size_t)bh * N + qtok] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------- workspaces and launchers

namespace {
size_t al256(size_t x) { return (x + 255) / 256 * 256; }
int pad32(int c) { return (c + 31) / 32 * 32; }
}  // namespace

size_t kmeans_workspace_bytes(int BH, int N, int d, int C) {
  const size_t CP = (size_t)pad32(C), nch = (size_t)(N + KM_CH - 1) / KM_CH;
  return 2 * al256((size_t)BH * CP * d * 2) + al256((size_t)BH * CP * 4) + al256((size_t)BH * N * 4) +
         al256((size_t)BH * nch * C * 4) + al256((size_t)BH * CP * 4);
}

hipError_t launch_kmeans(const void* x, int BH, int N, int d, int C, int iters, const float* init, float* cen,
                         int32_t* labels, int32_t* perm, int32_t* offsets, void* ws, hipStream_t stream) {
  const int CP = pad32(C), nch = (N + KM_CH - 1) / KM_CH;
  char* p = static_cast<char*>(ws);
  __bf16* chi = reinterpret_cast<__bf16*>(p);
  p += al256((size_t)BH * CP * d * 2);
  __bf16* clo = reinterpret_cast<__bf16*>(p);
  p += al256((size_t)BH * CP * d * 2);
  float* cn = reinterpret_cast<float*>(p);
  p += al256((size_t)BH * CP * 4);
  int32_t* rank = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)BH * N * 4);
  int32_t* hist = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)BH * nch * C * 4);
  int32_t* ord = reinterpret_cast<int32_t*>(p);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  hipError_t e;
#define SA_KM(D_)                                                                                                  \
  hipLaunchKernelGGL((km_init_kernel<D_>), dim3((unsigned)BH, (unsigned)CP), dim3(D_), 0, stream, xs, init, N, C, CP, \
                     cen, chi, clo, cn);                                                                           \
  if ((e = hipGetLastError()) != hipSuccess) return e;                                                             \
  for (int it = 0; it < iters; ++it) {                                                                             \
    hipLaunchKernelGGL((km_assign_kernel<D_>), dim3((unsigned)BH, (unsigned)((N + 255) / 256)), dim3(256), 0, stream, \
                       xs, chi, clo, cn, N, CP, labels);                                                           \
    hipLaunchKernelGGL(km_rank_kernel, dim3((unsigned)BH, (unsigned)nch), dim3(KM_CH), 0, stream, labels, N, C, nch, \
                       rank, hist);                                                                                \
    hipLaunchKernelGGL(km_scan_kernel, dim3((unsigned)BH, (unsigned)((C + 15) / 16)), dim3(1024), 0, stream, hist, C, \
                       nch, offsets);                                                                              \
    hipLaunchKernelGGL(km_offsets_kernel, dim3((unsigned)BH), dim3(KM_MAXC), 0, stream, C, CP, offsets, ord);     \
    hipLaunchKernelGGL(km_scatter_kernel, dim3((unsigned)BH, (unsigned)nch), dim3(KM_CH), 0, stream, labels, rank,  \
                       hist, offsets, N, C, nch, perm);                                                            \
    hipLaunchKernelGGL((km_update_kernel<D_>), dim3((unsigned)BH, (unsigned)CP), dim3(256), 0, stream, xs, perm,     \
                       offsets, ord, N, C, CP, cen, chi, clo, cn);                                                 \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                           \
  }
  if (d == 128) {
    SA_KM(128)
  } else if (d == 64) {
    SA_KM(64)
  } else {
    return hipErrorInvalidValue;
  }
#undef SA_KM
  return hipSuccess;
}

hipError_t launch_cluster_select(const float* cq, const float* ck, const int32_t* koff, int BH, int Cq, int Ck, int d,
                                 double scale, double p, double* probs, uint8_t* mask, hipStream_t stream) {
  hipLaunchKernelGGL(cluster_select_kernel, dim3((unsigned)BH, (unsigned)Cq), dim3(256), 0, stream, cq, ck, koff, Cq,
                     Ck, d, scale, p, probs, mask);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* x, const int32_t* perm, int BH, int N, int row_bytes, int inverse,
                               void* out, hipStream_t stream) {
  const long long pieces = (long long)BH * N * (row_bytes / 16);
  hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const char*>(x), perm, N, row_bytes, inverse, pieces, static_cast<char*>(out));
  return hipGetLastError();
}

int cluster_max_tiles(int N, int Cq, int Bq) { return (N + Bq - 1) / Bq + Cq; }

size_t cluster_fwd_workspace_bytes(int BH, int N, int Cq, int Ck, int Bq) {
  const size_t mt = (size_t)cluster_max_tiles(N, Cq, Bq);
  return al256((size_t)BH * mt * 16) + al256((size_t)BH * 4) + al256((size_t)BH * Cq * Ck * 4) +
         al256((size_t)BH * Cq * 4);
}

hipError_t launch_compact(const uint8_t* mask, int rows, int nkb, int32_t* kidx, int32_t* kcnt, hipStream_t stream);

hipError_t launch_cluster_fwd(const void* q, const void* k, const void* v, int BH, int N, int d, const int32_t* qoff,
                              int Cq, const int32_t* koff, int Ck, const uint8_t* mask, const int32_t* qperm,
                              const int32_t* kperm, int Bq, double scale, void* o, float* lse, void* ws,
                              hipStream_t stream) {
  const int mt = cluster_max_tiles(N, Cq, Bq);
  char* p = static_cast<char*>(ws);
  int4* tiles = reinterpret_cast<int4*>(p);
  p += al256((size_t)BH * mt * 16);
  int32_t* nt = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)BH * 4);
  int32_t* kidx = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)BH * Cq * Ck * 4);
  int32_t* kcnt = reinterpret_cast<int32_t*>(p);
  hipLaunchKernelGGL(cluster_tiles_kernel, dim3((unsigned)BH), dim3(KM_MAXC), 0, stream, qoff, Cq, Bq, mt, tiles, nt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_compact(mask, BH * Cq, Ck, kidx, kcnt, stream)) != hipSuccess) return e;
  const float c_log2 = (float)(scale * 1.4426950408889634);
  const dim3 grid((unsigned)((size_t)BH * mt));
#define SA_VAR(D_, BQ_)                                                                                            \
  if (d == D_ && Bq == BQ_) {                                                                                      \
    hipLaunchKernelGGL((attn_var_kernel<D_, BQ_>), grid, dim3(DCfg<D_, BQ_>::NT), 0, stream, q, k, v, N, tiles, nt,  \
                       mt, koff, Cq, Ck, kidx, kcnt, qperm, kperm, c_log2, o, lse);                                \
    return hipGetLastError();                                                                                      \
  }
  SA_VAR(128, 128)
  SA_VAR(128, 64)
  SA_VAR(64, 128)
  SA_VAR(64, 64)
#undef SA_VAR
  return hipErrorInvalidValue;
}

}  // namespace sa
