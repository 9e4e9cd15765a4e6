// Pooled probability pattern and hybrid Top-k U Top-p block mask (gfx950).
//
// Method (SpargeAttention2 page on ai-papers.net, sections "Top-kとTop-pの限界を解剖する" and
// "ハイブリッドマスキングと蒸留微調整"; Sparse VideoGen2 page, "2. 手法" B):
//   scores   S[i][j] = scale * <q_pool[i], k_pool[j]>         (float64)
//   softmax  P[i][j] = exp(S[i][j] - max_j S[i][j]) / sum      (float64, one row per query block)
//   order    descending P, the lower block index first on equal P
//   Top-k    the first k entries of the order
//   Top-p    the shortest prefix whose running sum is >= p
//   union    both are prefixes of one order, so the kept set is the first max(k, m*) entries.
//
// Everything that decides the mask is float64 so that it agrees with a float64 reference
// except for rows that sit within rounding of a threshold.
//
// Kernel 1 (scores_kernel) is a small float64 GEMM per head written straight into `probs`.
// Kernel 2 (select_kernel) takes one row per workgroup: softmax in place, then orders only the
// entries that can belong to the kept prefix, a chunked prefix sum for m*, then the mask row and
// optional lists.
#include "sa_common.h"

namespace sa {

// ---------------------------------------------------------------- kernel 1: pooled scores

constexpr int ST = 64;   // output tile edge
constexpr int SKD = 16;  // depth of one LDS stage

__global__ __launch_bounds__(256) void scores_kernel(const double* __restrict__ qp, const double* __restrict__ kp,
                                                     int nqb, int nkb, int d, double scale,
                                                     double* __restrict__ s_out) {
  __shared__ double As[SKD][ST + 1];
  __shared__ double Bs[SKD][ST + 1];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * ST;
  const int j0 = blockIdx.x * ST;
  const double* qh = qp + (size_t)bh * nqb * d;
  const double* kh = kp + (size_t)bh * nkb * d;
  const int tj = threadIdx.x & 15;  // columns j0 + tj + 16 b
  const int ti = threadIdx.x >> 4;  // rows    i0 + ti + 16 a
  double acc[4][4] = {};
  for (int d0 = 0; d0 < d; d0 += SKD) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = threadIdx.x + 256 * e;
      const int r = idx >> 4, c = idx & 15;
      As[c][r] = (i0 + r < nqb) ? qh[(size_t)(i0 + r) * d + d0 + c] : 0.0;
      Bs[c][r] = (j0 + r < nkb) ? kh[(size_t)(j0 + r) * d + d0 + c] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SKD; ++c) {
      double a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] = As[c][ti + 16 * x];
        b[x] = Bs[c][tj + 16 * x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
  double* so = s_out + (size_t)bh * nqb * nkb;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + ti + 16 * x;
    if (i >= nqb) continue;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tj + 16 * y;
      if (j < nkb) so[(size_t)i * nkb + j] = scale * acc[x][y];
    }
  }
}

// ---------------------------------------------------------------- kernel 2: row selection

__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// (P, index) a ranks before b: larger probability first, then the lower block index. P >= 0,
// so comparing IEEE bit patterns as unsigned integers orders like the values.
__device__ __forceinline__ bool ranks_before(uint64_t ka, uint32_t ia, uint64_t kb, uint32_t ib) {
  return ka > kb || (ka == kb && ia < ib);
}

constexpr int NBUCKET = 128;    // half-octave buckets of P: bucket 2o + (lower half of octave o)
constexpr int RANK_MAX = 2048;  // candidates ordered by rank counting up to this many; sorted above
constexpr double FIX = 4503599627370496.0;  // 2^52: fixed-point scale of the bucket masses

// Monotone non-increasing in P: a larger probability never lands in a later bucket.
__device__ __forceinline__ int bucket_of(uint64_t bits) {
  const int o = 1023 - (int)(bits >> 52);          // P in [2^-o, 2^(1-o)); P = 0 gives o = 1023
  const int lower = (int)((~bits >> 51) & 1ull);   // mantissa top bit clear: lower half-octave
  return min(NBUCKET - 1, 2 * max(o, 0) + lower);
}

// Dynamic LDS for a row of nkb entries (np2 = next power of two >= nkb):
//   uint64 pk[np2] | uint64 hmass[128] | uint32 hcnt[128] | uint16 cand[np2] | uint16 ord[np2] |
//   uint8 flag[np2]
// Steps: softmax in place (pk holds S, then exp, then P bits); bucket histogram of P with integer
// atomics (count and 2^-52 fixed-point mass, both order-independent); the first bucket prefix
// whose count reaches k and whose mass reaches p + 1e-12 gives a candidate set that is closed
// under ">=" and therefore holds the whole kept prefix; candidates are ordered exactly (rank
// counting, or a bitonic sort when there are many); float64 running sums over that order give m*.
__global__ __launch_bounds__(256) void select_kernel(double* __restrict__ probs, uint8_t* __restrict__ mask,
                                                     int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt,
                                                     int nkb, int np2, int k, double p) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  uint64_t* pk = reinterpret_cast<uint64_t*>(lds);
  uint64_t* hmass = pk + np2;
  uint32_t* hcnt = reinterpret_cast<uint32_t*>(hmass + NBUCKET);
  uint16_t* cand = reinterpret_cast<uint16_t*>(hcnt + NBUCKET);
  uint16_t* ord = cand + np2;
  uint8_t* flag = reinterpret_cast<uint8_t*>(ord + np2);
  __shared__ double red[8];
  __shared__ double scan[256];
  __shared__ int n_cand, b_star, m_star_s;
  __shared__ int wcnt[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t row = blockIdx.x;
  double* P = probs + row * (size_t)nkb;

  // softmax over the row (scores were written into `probs` by kernel 1)
  double mx = -INFINITY;
  for (int j = tid; j < nkb; j += 256) {
    const double sj = P[j];
    pk[j] = (uint64_t)__double_as_longlong(sj);
    mx = fmax(mx, sj);
  }
  for (int j = tid; j < np2; j += 256) flag[j] = 0;
  if (tid < NBUCKET) {
    hcnt[tid] = 0;
    hmass[tid] = 0;
  }
  if (tid == 0) {
    n_cand = 0;
    m_star_s = nkb;
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  double sum = 0.0;
  for (int j = tid; j < nkb; j += 256) {
    const double e = exp(__longlong_as_double(pk[j]) - mx);
    pk[j] = (uint64_t)__double_as_longlong(e);
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[4 + wave] = sum;
  __syncthreads();
  sum = ((red[4] + red[5]) + red[6]) + red[7];
  for (int j = tid; j < nkb; j += 256) {
    const double pj = __longlong_as_double(pk[j]) / sum;
    P[j] = pj;
    const uint64_t bits = (uint64_t)__double_as_longlong(pj);
    pk[j] = bits;
    const int b = bucket_of(bits);
    atomicAdd(&hcnt[b], 1u);
    atomicAdd(reinterpret_cast<unsigned long long*>(&hmass[b]), (unsigned long long)(pj * FIX));
  }
  __syncthreads();

  // first bucket prefix holding >= k entries and (for p > 0) mass >= p + 1e-12
  if (wave == 0) {
    const unsigned long long need = p > 0.0 ? (unsigned long long)ceil((p + 1e-12) * FIX) : 0ull;
    unsigned c0 = hcnt[2 * lane], c1 = hcnt[2 * lane + 1];
    unsigned long long m0 = hmass[2 * lane], m1 = hmass[2 * lane + 1];
    unsigned cs = c0 + c1;
    unsigned long long ms = m0 + m1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {  // inclusive scan over lanes
      const unsigned cu = __shfl_up(cs, o, 64);
      const unsigned long long mu = __shfl_up(ms, o, 64);
      if (lane >= o) {
        cs += cu;
        ms += mu;
      }
    }
    const unsigned cb = cs - c0 - c1;  // exclusive prefix before bucket 2 lane
    const unsigned long long mb = ms - m0 - m1;
    const bool ok0 = cb + c0 >= (unsigned)k && mb + m0 >= need;
    const bool ok1 = cs >= (unsigned)k && ms >= need;
    const uint64_t b0 = __ballot(ok0), b1 = __ballot(ok1);
    int bs = NBUCKET - 1;
    if (b0 | b1) {
      const int l0 = b0 ? __ffsll((unsigned long long)b0) - 1 : 64;
      const int l1 = b1 ? __ffsll((unsigned long long)b1) - 1 : 64;
      bs = min(2 * l0, 2 * l1 + 1);
    }
    if (lane == 0) b_star = bs;
  }
  __syncthreads();
  const int bs = b_star;
  for (int j = tid; j < nkb; j += 256) {
    if (bucket_of(pk[j]) <= bs) cand[atomicAdd(&n_cand, 1)] = (uint16_t)j;
  }
  __syncthreads();
  const int S = n_cand;

  // exact order of the candidates
  if (S <= RANK_MAX) {
    for (int c = tid; c < S; c += 256) {
      const uint32_t jc = cand[c];
      const uint64_t kc = pk[jc];
      int rank = 0;
      for (int x = 0; x < S; ++x) {
        const uint32_t jx = cand[x];
        rank += ranks_before(pk[jx], jx, kc, jc) ? 1 : 0;
      }
      ord[rank] = (uint16_t)jc;
    }
  } else {
    int sp2 = 1;
    while (sp2 < S) sp2 <<= 1;
    for (int c = S + tid; c < sp2; c += 256) cand[c] = 0xffff;  // padding ranks last
    __syncthreads();
    for (int size = 2; size <= sp2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (sp2 >> 1); t += 256) {
          const int lo = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
          const int hi = lo + stride;
          const uint32_t ja = cand[lo], jb = cand[hi];
          const uint64_t ka = ja == 0xffff ? 0 : pk[ja], kb = jb == 0xffff ? 0 : pk[jb];
          const bool b_first = (jb != 0xffff) && (ja == 0xffff || ranks_before(kb, jb, ka, ja));
          if (b_first == ((lo & size) == 0)) {
            cand[lo] = (uint16_t)jb;
            cand[hi] = (uint16_t)ja;
          }
        }
        __syncthreads();
      }
    }
    for (int c = tid; c < S; c += 256) ord[c] = cand[c];
  }
  __syncthreads();

  // Top-p: m* = min{m >= 1 : P_(1) + ... + P_(m) >= p}, or nkb if the sum never reaches p. The
  // candidates hold every prefix that can reach p (or all entries when the row's mass is short).
  int m_star = 0;
  if (p > 0.0) {
    const int per = (S + 255) / 256;
    const int lo = tid * per, hi = min(S, lo + per);
    double local = 0.0;
    for (int r = lo; r < hi; ++r) local += __longlong_as_double(pk[ord[r]]);
    scan[tid] = local;
    __syncthreads();
    if (wave == 0) {  // exclusive scan of the 256 chunk sums, in order
      double v[4];
      double run = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = run;
        run += scan[4 * lane + e];
      }
      double incl = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const double up = __shfl_up(incl, o, 64);
        if (lane >= o) incl += up;
      }
      double base = __shfl_up(incl, 1, 64);
      if (lane == 0) base = 0.0;
#pragma unroll
      for (int e = 0; e < 4; ++e) scan[4 * lane + e] = base + v[e];
    }
    __syncthreads();
    double c = scan[tid];
    for (int r = lo; r < hi; ++r) {
      c += __longlong_as_double(pk[ord[r]]);
      if (c >= p) {
        atomicMin(&m_star_s, r + 1);
        break;
      }
    }
    __syncthreads();
    m_star = m_star_s;
  }
  const int L = min(max(k, m_star), S);

  for (int r = tid; r < L; r += 256) flag[ord[r]] = 1;
  __syncthreads();
  uint8_t* mrow = mask + row * (size_t)nkb;
  for (int j = tid; j < nkb; j += 256) mrow[j] = flag[j];

  if (kept_idx != nullptr) {
    // ascending kept indices: one pass of 256 entries at a time, ballot prefix per wave
    int32_t* out = kept_idx + row * (size_t)nkb;
    int base = 0;
    for (int j0 = 0; j0 < nkb; j0 += 256) {
      const int j = j0 + tid;
      const bool f = j < nkb && flag[j];
      const uint64_t b = __ballot(f);
      if (lane == 0) wcnt[wave] = __popcll(b);
      __syncthreads();
      int off = base;
      for (int w = 0; w < wave; ++w) off += wcnt[w];
      if (f) out[off + __popcll(b & ((1ull << lane) - 1ull))] = j;
      for (int w = 0; w < 4; ++w) base += wcnt[w];
      __syncthreads();
    }
    if (tid == 0) kept_cnt[row] = L;
  }
}

int select_np2(int nkb) {
  int n = 1;
  while (n < nkb) n <<= 1;
  return n;
}

size_t select_lds_bytes(int np2) {
  return (size_t)np2 * 8 + NBUCKET * 8 + NBUCKET * 4 + (size_t)np2 * 2 * 2 + (size_t)np2;
}

hipError_t launch_select(const double* qp, const double* kp, int BH, int nqb, int nkb, int d, double scale,
                         int k, double p, double* probs, uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt,
                         hipStream_t stream) {
  const dim3 g1((unsigned)((nkb + ST - 1) / ST), (unsigned)((nqb + ST - 1) / ST), (unsigned)BH);
  hipLaunchKernelGGL(scores_kernel, g1, dim3(256), 0, stream, qp, kp, nqb, nkb, d, scale, probs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int np2 = select_np2(nkb);
  const size_t lds = select_lds_bytes(np2);
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)(BH * nqb)), dim3(256), lds, stream, probs, mask, kept_idx,
                     kept_cnt, nkb, np2, k, p);
  return hipGetLastError();
}

}  // namespace sa
