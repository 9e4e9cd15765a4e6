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
// Kernel 1 (scores_kernel) is a float64 GEMM per head on the matrix cores, written into `probs`.
// Kernel 2 takes the rows: select_rows_kernel one wave per row in registers, select_kernel (rows
// longer than a wave holds) one workgroup per row; softmax in place, then only the entries that can
// belong to the kept prefix are ordered, running sums give m*, then the mask row and optional lists.
// Without `probs`, select_fused_kernel does both: scores of 16 rows in LDS, then the rows' selection.
#include <algorithm>

#include "sa_common.h"

namespace sa {

// ---------------------------------------------------------------- kernel 1: pooled scores

// S = scale * Qbar Kbar^T per head in float64 on the matrix cores (v_mfma_f64_16x16x4f64). For
// that instruction lane j holds A[j % 16][j / 16] and B[j / 16][j % 16] of a 16x4 / 4x16 step, and
// element i of the result holds C[4 i + j / 16][j % 16] (lane layout checked with one-hot
// operands). A workgroup of 4 waves owns 128 query-block rows of Qbar (wave w keeps rows
// 32 w .. 32 w + 31 in registers, as two sets of 16 that share every Kbar operand read, which
// gives each wave four independent accumulation chains) and walks a chunk of 32-row tiles of Kbar. The tiles pass
// through two LDS buffers: the next tile's loads are in flight while the current one multiplies,
// and are stored to the other buffer afterwards. Two doubles of padding per row put the 32 lanes
// of each half-wave read (16 rows x 2 consecutive doubles) on distinct banks.
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
constexpr int SQ = 128;  // query-block rows per workgroup
constexpr int SK = 32;  // key-block rows per tile

template <int D>
__global__ __launch_bounds__(256, 2) void scores_kernel(const double* __restrict__ qp, const double* __restrict__ kp,
                                                        int nqb, int nkb, int tiles_per_chunk, double scale,
                                                        double* __restrict__ s_out) {
  constexpr int LROW = D + 2;
  constexpr int PER = SK * D / 2 / 256;  // 16-byte pieces of a tile per thread
  __shared__ __attribute__((aligned(16))) double kl[2][SK * LROW];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * SQ;
  const int ntile = (nkb + SK - 1) / SK;
  const int t0 = blockIdx.x * tiles_per_chunk;
  const int t1 = min(ntile, t0 + tiles_per_chunk);
  if (t0 >= t1) return;
  const double* qh = qp + (size_t)bh * nqb * D;
  const double* kh = kp + (size_t)bh * nkb * D;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, kq = lane >> 4;

  // piece u of thread tid: tile row r = e / (D / 2), doubles 2 c .. 2 c + 1, e = tid + 256 u
  f64x2 v[PER];
  auto load = [&](int t) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 2), c = e % (D / 2);
      const int j = t * SK + r;
      v[u] = j < nkb ? *reinterpret_cast<const f64x2*>(kh + (size_t)j * D + 2 * c) : (f64x2){0.0, 0.0};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + 256 * u;
      const int r = e / (D / 2), c = e % (D / 2);
      *reinterpret_cast<f64x2*>(&kl[buf][r * LROW + 2 * c]) = v[u];
    }
  };

  load(t0);
  double a[2][D / 4];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int qrow = i0 + 32 * wave + 16 * g + m;
#pragma unroll
    for (int s = 0; s < D / 4; ++s) a[g][s] = qrow < nqb ? qh[(size_t)qrow * D + 4 * s + kq] : 0.0;
  }
  store(0);
  __syncthreads();

  double* so = s_out + (size_t)bh * nqb * nkb;
  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < t1) load(t + 1);  // in flight during the products
    f64x4 acc[2][2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[g][h] = (f64x4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < D / 4; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double b = kl[buf][(16 * h + m) * LROW + 4 * s + kq];
#pragma unroll
        for (int g = 0; g < 2; ++g) acc[g][h] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[g][s], b, acc[g][h], 0, 0, 0);
      }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int col = t * SK + 16 * h + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = i0 + 32 * wave + 16 * g + 4 * i + kq;
          if (row < nqb && col < nkb) so[(size_t)row * nkb + col] = scale * acc[g][h][i];
        }
      }
    // the other buffer was last read in step t - 1, which every wave finished before the barrier
    if (t + 1 < t1) store(buf ^ 1);
    __syncthreads();
  }
}

// Key tiles per workgroup: enough workgroups for about four rounds of two per CU.
inline int scores_tiles_per_chunk(int BH, int nqb, int nkb) {
  const int ntile = (nkb + SK - 1) / SK;
  const long long pairs = (long long)BH * ((nqb + SQ - 1) / SQ);
  const int chunks = (int)std::max(1LL, std::min<long long>(ntile, (2048 + pairs - 1) / pairs));
  return (ntile + chunks - 1) / chunks;
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

// ---------------------------------------------------------------- kernel 2b: one wave per row

// Rows of up to WAVE_NKB entries take one wave each (four rows per workgroup, no workgroup
// barrier). Entry j of the row stays in lane j % 64, register slot j / 64, for the whole
// selection. Wave sums and maxima combine within each 16-lane row with DPP moves and then add the
// four row results, read from lanes 0, 16, 32 and 48, in a fixed order: every lane gets the same
// value, identical from run to run.
//
// Selection without sorting the row. Let key(P) be the IEEE bits of P (ordered like P, as P >= 0)
// and f(T) the predicate "at least k entries have key >= T and, for p > 0, their mass is >= p".
// f is monotone; with T* = max{T : f(T)} the kept prefix holds every entry whose key is above T*,
// none below it, and a leading run, in index order, of the entries whose key equals T* (the
// prefix through T* meets both thresholds; the part above T* misses one of them). T* is
// bracketed by bisection, first over the 128 half-octave bucket edges, then over key values while
// more than 64 entries lie inside the bracket [lo, hi]. The entries inside are put in exact order,
// by rank counting (at most 64 of them, one per lane) or, when the bracket has closed on a single
// value, by index, and running sums along that order give m*.
constexpr int WAVE_NKB = 2048;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] (lane ^ 1, lane ^ 2), row_ror:4, row_ror:8.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_f64(double x, int l) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_dpp(double x) {
  x += dpp_f64<DPP_XOR1>(x);
  x += dpp_f64<DPP_XOR2>(x);
  x += dpp_f64<DPP_ROR4>(x);
  x += dpp_f64<DPP_ROR8>(x);
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}
__device__ __forceinline__ double wave_max_dpp(double x) {
  x = fmax(x, dpp_f64<DPP_XOR1>(x));
  x = fmax(x, dpp_f64<DPP_XOR2>(x));
  x = fmax(x, dpp_f64<DPP_ROR4>(x));
  x = fmax(x, dpp_f64<DPP_ROR8>(x));
  return fmax(fmax(readlane_f64(x, 0), readlane_f64(x, 16)), fmax(readlane_f64(x, 32), readlane_f64(x, 48)));
}

// Smallest key of bucket b (bucket_of(key) <= b exactly when key >= bucket_floor(b)).
__device__ __forceinline__ int64_t bucket_floor(int b) {
  if (b >= NBUCKET - 1) return 0;
  const int64_t e = 1023 - (b >> 1);
  return (e << 52) | ((b & 1) ? (int64_t)0 : ((int64_t)1 << 51));
}

// Softmax and hybrid selection of one row whose scores one wave holds in registers: v[u] is the
// score of entry 64 u + lane (-inf past the end of the row). P (NULL: not written) receives the
// probabilities, mrow the mask row, out / cnt_out (both NULL or neither) the ascending kept list
// and its length. s_key and s_val are 64 entries each of LDS scratch private to the wave.
template <int R>
__device__ __forceinline__ void select_row(double (&v)[R], int nkb, int k, double p, double* __restrict__ P,
                                           uint8_t* __restrict__ mrow, int32_t* __restrict__ out,
                                           int32_t* __restrict__ cnt_out, int64_t* s_key, double* s_val) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  int64_t key[R];  // key of entry 64 u + lane, -1 past the end of the row
  {
    double mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < R; ++u) mx = fmax(mx, v[u]);
    mx = wave_max_dpp(mx);
    double sum = 0.0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (64 * u + lane < nkb) {
        v[u] = exp(v[u] - mx);
        sum += v[u];
      }
    }
    sum = wave_sum_dpp(sum);
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = 64 * u + lane;
      key[u] = -1;
      if (j < nkb) {
        const double pj = v[u] / sum;
        if (P != nullptr) P[j] = pj;
        key[u] = __double_as_longlong(pj);
      }
    }
  }

  // count and mass of the entries with key >= T (count and mass are wave-uniform)
  auto tally = [&](int64_t T, int& cnt, double& mass) {
    int c = 0;
    double m = 0.0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const bool ge = key[u] >= T;
      c += __popcll(__ballot(ge));
      m += ge ? __longlong_as_double(key[u]) : 0.0;
    }
    cnt = c;
    mass = wave_sum_dpp(m);
  };
  auto meets = [&](int cnt, double mass) { return cnt >= k && (p <= 0.0 || mass >= p); };

  int c_lo, c_hi;      // entries with key >= lo, and with key > hi
  double m_lo, m_hi;   // their masses
  tally(0, c_lo, m_lo);
  const bool keep_all = !meets(c_lo, m_lo);  // the row's mass never reaches p: m* = nkb
  int64_t lo = 0, hi = INT64_MAX;
  int n_keep = 0;      // leading entries of the bracket, in selection order, that are kept
  uint64_t kmask = 0;  // bracket positions kept when the bracket holds <= 64 entries
  int nb = 0;
  if (!keep_all) {
    c_hi = 0;
    m_hi = 0.0;
    int blo = 0, bhi = NBUCKET - 1;  // f(bucket_floor(bhi)) holds, f(bucket_floor(blo - 1)) fails
    while (blo < bhi) {
      const int mid = (blo + bhi) >> 1;
      int c;
      double m;
      tally(bucket_floor(mid), c, m);
      if (meets(c, m)) {
        bhi = mid;
        c_lo = c;
        m_lo = m;
      } else {
        blo = mid + 1;
        c_hi = c;
        m_hi = m;
      }
    }
    lo = bucket_floor(blo);
    hi = blo == 0 ? INT64_MAX : bucket_floor(blo - 1) - 1;
    while (c_lo - c_hi > 64 && lo < hi) {
      const int64_t mid = lo + ((hi - lo + 1) >> 1);
      int c;
      double m;
      tally(mid, c, m);
      if (meets(c, m)) {
        lo = mid;
        c_lo = c;
        m_lo = m;
      } else {
        hi = mid - 1;
        c_hi = c;
        m_hi = m;
      }
    }
    nb = c_lo - c_hi;
    const int need_k = max(k - c_hi, 0);
    if (nb <= 64) {
      // gather the bracket (ascending index) one entry per lane, rank it, then running sums
      int base = 0;
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const bool in = key[u] >= lo && key[u] <= hi;
        const uint64_t bal = __ballot(in);
        if (in) s_key[base + __popcll(bal & below)] = key[u];
        base += __popcll(bal);
      }
      wave_sync();
      const bool mine = lane < nb;
      const int64_t kc = mine ? s_key[lane] : -1;
      int rank = 0;
      for (int x = 0; x < nb; ++x) {
        const uint32_t xl = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)kc, x);
        const uint32_t xh = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)kc >> 32), x);
        const int64_t kx = (int64_t)(((uint64_t)xh << 32) | xl);
        rank += (kx > kc || (kx == kc && x < lane)) ? 1 : 0;
      }
      int n_p = 0;
      if (p > 0.0 && m_hi < p) {
        if (mine) s_val[rank] = __longlong_as_double(kc);
        wave_sync();
        double run = mine ? s_val[lane] : 0.0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double up = __shfl_up(run, o, 64);
          if (lane >= o) run += up;
        }
        const uint64_t hit = __ballot(mine && m_hi + run >= p);
        n_p = hit ? __ffsll((unsigned long long)hit) : nb;
      }
      n_keep = min(nb, max(need_k, n_p));
      kmask = __ballot(mine && rank < n_keep);
    } else {
      // lo == hi: every entry in the bracket has the value v, and the order among them is by index
      const double v = __longlong_as_double(lo);
      int n_p = 0;
      if (p > 0.0 && m_hi < p) n_p = v > 0.0 ? (int)min((double)nb, ceil((p - m_hi) / v)) : nb;
      n_keep = min(nb, max(need_k, n_p));
    }
  }

  int pos0 = 0, n_out = 0;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int j = 64 * u + lane;
    const bool in = key[u] >= lo && key[u] <= hi;
    const uint64_t bal = __ballot(in);
    const int pos = pos0 + __popcll(bal & below);
    pos0 += __popcll(bal);
    bool kept;
    if (keep_all) kept = j < nkb;
    else kept = key[u] > hi || (in && (nb <= 64 ? (pos < 64 && ((kmask >> pos) & 1ull) != 0) : pos < n_keep));
    if (j < nkb) mrow[j] = kept ? 1 : 0;
    if (out != nullptr) {
      const uint64_t kb = __ballot(kept);
      if (kept) out[n_out + __popcll(kb & below)] = j;
      n_out += __popcll(kb);
    }
  }
  if (out != nullptr && lane == 0) *cnt_out = n_out;
}

template <int R>
__global__ __launch_bounds__(256) void select_rows_kernel(double* __restrict__ probs, uint8_t* __restrict__ mask,
                                                          int32_t* __restrict__ kept_idx,
                                                          int32_t* __restrict__ kept_cnt, int rows, int nkb, int k,
                                                          double p) {
  __shared__ int64_t s_key[4][64];
  __shared__ double s_val[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 4 + wave;
  if (row >= (size_t)rows) return;  // whole wave leaves; nothing below synchronises the workgroup
  // kernel 1 left the scores in `probs`; the probabilities are written back in place
  double* P = probs + row * (size_t)nkb;
  double v[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int j = 64 * u + lane;
    v[u] = j < nkb ? P[j] : -INFINITY;
  }
  select_row<R>(v, nkb, k, p, P, mask + row * (size_t)nkb, kept_idx ? kept_idx + row * (size_t)nkb : nullptr,
                kept_idx ? kept_cnt + row : nullptr, s_key[wave], s_val[wave]);
}

// ---------------------------------------------------------------- fused scores + selection

// For callers that do not want the probabilities. One workgroup per group of FQ query-block rows
// of a head: the scores of the whole group stay in LDS, so they never make a round trip through
// HBM. 16 waves, so that the row phase has a wave per row. Phase 1: the group's FQ x nkb scores
// on the float64 matrix cores. Waves w and w + 8 compute the same 16-column tiles
// t = w mod 8, + 8, ..., over the first and the second half of
// the channels, and add their partial scores into the zeroed LDS rows (two float64 adds onto
// zero, so the sum does not depend on their order). Each wave keeps its half of the group's Qbar
// rows as A operands in registers and reads each tile's Kbar half-rows as B operands straight
// from memory (one head's Kbar stays in the XCD's L2), the next tile's loads in flight during the
// current tile's products. Lane (m, kq) of the v_mfma_f64_16x16x4f64 supplies row / column m at
// channels h D / 2 + KH kq .. + KH - 1 over the KH = D / 8 steps of half h, so each lane reads
// one contiguous run; even and odd steps accumulate in two chains. Phase 2: wave r takes row r
// of the group and runs the per-row softmax and selection on its scores, read from LDS.
// Workgroups take the (head, group) items in one contiguous range per XCD.
constexpr int FQ = 16;            // query-block rows per workgroup (the M of the fp64 product)
constexpr int FW = 16;            // waves per workgroup: one per row in the row phase
constexpr int FUSED_NKB = 1280;   // FQ rows of float64 scores fill the 160 KiB of LDS

inline int fused_pitch(int nkb) { return std::max(128, (nkb + 15) / 16 * 16); }

template <int D, int R>
__global__ __launch_bounds__(FW * 64, 1) void select_fused_kernel(const double* __restrict__ qp,
                                                                  const double* __restrict__ kp, int n_items,
                                                                  int nqb, int nkb, int pitch, double scale, int k,
                                                                  double p, uint8_t* __restrict__ mask,
                                                                  int32_t* __restrict__ kept_idx,
                                                                  int32_t* __restrict__ kept_cnt) {
  constexpr int KH = D / 8;  // product steps per channel half
  extern __shared__ __attribute__((aligned(16))) double s_lds[];  // [FQ][pitch] scores
  const int ngrp = (nqb + FQ - 1) / FQ;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int bh = item / ngrp;
  const int i0 = (item - bh * ngrp) * FQ;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = lane & 15, kq = lane >> 4;
  const int pw = wave & 7;                  // tiles pw, pw + 8, ...
  const int ch0 = (wave >> 3) * (D / 2) + KH * kq;  // this lane's first channel
  const double* qh = qp + (size_t)bh * nqb * D;
  const double* kh = kp + (size_t)bh * nkb * D;

  for (int e = 2 * threadIdx.x; e < FQ * pitch; e += 2 * FW * 64)
    *reinterpret_cast<f64x2*>(s_lds + e) = (f64x2){0.0, 0.0};

  // row r of base (clamped to the n rows there are), this lane's KH channels. Rows past the end
  // only feed scores that are never read: query rows past nqb and key columns past nkb.
  auto load_run = [&](const double* base, int r, int n, double (&x)[KH]) {
    const f64x2* src = reinterpret_cast<const f64x2*>(base + (size_t)min(r, n - 1) * D + ch0);
#pragma unroll
    for (int s = 0; s < KH / 2; ++s) {
      const f64x2 w = src[s];
      x[2 * s] = w[0];
      x[2 * s + 1] = w[1];
    }
  };
  double a[KH];
  load_run(qh, i0 + m, nqb, a);
  __syncthreads();  // the zeroed scores

  // tile t: this half's part of the scores of the group's rows against key blocks 16 t .. + 15
  auto tile = [&](int t, const double (&b)[KH]) {
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = acc0;
#pragma unroll
    for (int s = 0; s < KH; s += 2) {
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s + 1], b[s + 1], acc1, 0, 0, 0);
    }
    // result element i: row 4 i + kq, column 16 t + m
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __hip_atomic_fetch_add(&s_lds[(4 * i + kq) * pitch + 16 * t + m], scale * (acc0[i] + acc1[i]),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  // the next tile's loads (clamped to the last tile, so that the loop body has no branch) are
  // issued before the current tile's products and moved into place after them, so the products
  // never wait for the loads in flight
  const int ntile = (nkb + 15) / 16;
  double bc[KH], bn[KH];
  load_run(kh, 16 * min(pw, ntile - 1) + m, nkb, bc);
  for (int t = pw; t < ntile; t += 8) {
    load_run(kh, 16 * min(t + 8, ntile - 1) + m, nkb, bn);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out ahead of the products
    tile(t, bc);
    __builtin_amdgcn_sched_barrier(0);  // and the moves, which wait for them, come after
#pragma unroll
    for (int s = 0; s < KH; ++s) bc[s] = bn[s];
  }
  __syncthreads();

  const int row = i0 + wave;
  if (row >= nqb) return;  // nothing below synchronises the workgroup
  double* srow = s_lds + (size_t)wave * pitch;
  double v[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int j = 64 * u + lane;
    v[u] = j < nkb ? srow[j] : -INFINITY;
  }
  // the row's LDS becomes the wave's scratch once every lane has read it
  wave_sync();
  const size_t g = (size_t)bh * nqb + row;
  select_row<R>(v, nkb, k, p, nullptr, mask + g * nkb,
                kept_idx ? kept_idx + g * nkb : nullptr, kept_idx ? kept_cnt + g : nullptr,
                reinterpret_cast<int64_t*>(srow), srow + 64);
}

template <int D, int R>
hipError_t launch_fused(const double* qp, const double* kp, int BH, int nqb, int nkb, double scale, int k, double p,
                        uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, hipStream_t stream) {
  const int pitch = fused_pitch(nkb);
  const size_t lds = (size_t)FQ * pitch * sizeof(double);
  const auto fn = reinterpret_cast<const void*>(&select_fused_kernel<D, R>);
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int n_items = BH * ((nqb + FQ - 1) / FQ);
  hipLaunchKernelGGL((select_fused_kernel<D, R>), dim3((unsigned)n_items), dim3(FW * 64), lds, stream, qp, kp,
                     n_items, nqb, nkb, pitch, scale, k, p, mask, kept_idx, kept_cnt);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_fused(const double* qp, const double* kp, int BH, int nqb, int nkb, double scale, int k, double p,
                          uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, hipStream_t stream) {
  const int r = (nkb + 63) / 64;
#define SA_FUSED(RR) return launch_fused<D, RR>(qp, kp, BH, nqb, nkb, scale, k, p, mask, kept_idx, kept_cnt, stream)
  if (r <= 1) SA_FUSED(1);
  if (r <= 2) SA_FUSED(2);
  if (r <= 4) SA_FUSED(4);
  if (r <= 8) SA_FUSED(8);
  if (r <= 12) SA_FUSED(12);
  if (r <= 16) SA_FUSED(16);
  SA_FUSED(20);
#undef SA_FUSED
}

template <int R>
hipError_t launch_rows(double* probs, uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, int rows, int nkb, int k,
                       double p, hipStream_t stream) {
  hipLaunchKernelGGL((select_rows_kernel<R>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, probs, mask,
                     kept_idx, kept_cnt, rows, nkb, k, p);
  return hipGetLastError();
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
  // Without probs the scores stay on chip (rows of at most FUSED_NKB entries, which the host
  // checks ensure). With probs the scores pass through it: the two kernels together are faster
  // than the fused one at 720p, whose groups of 16 rows read each head's Kbar 37 times over.
  if (probs == nullptr) {
    if (nkb > FUSED_NKB) return hipErrorInvalidValue;
    if (d == 128) return dispatch_fused<128>(qp, kp, BH, nqb, nkb, scale, k, p, mask, kept_idx, kept_cnt, stream);
    return dispatch_fused<64>(qp, kp, BH, nqb, nkb, scale, k, p, mask, kept_idx, kept_cnt, stream);
  }
  const int tpc = scores_tiles_per_chunk(BH, nqb, nkb);
  const int ntile = (nkb + SK - 1) / SK;
  const dim3 g1((unsigned)((ntile + tpc - 1) / tpc), (unsigned)((nqb + SQ - 1) / SQ), (unsigned)BH);
  if (d == 128)
    hipLaunchKernelGGL((scores_kernel<128>), g1, dim3(256), 0, stream, qp, kp, nqb, nkb, tpc, scale, probs);
  else
    hipLaunchKernelGGL((scores_kernel<64>), g1, dim3(256), 0, stream, qp, kp, nqb, nkb, tpc, scale, probs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nkb <= WAVE_NKB) {
    const int rows = BH * nqb;
    const int r = (nkb + 63) / 64;  // register slots per lane
    if (r <= 1) return launch_rows<1>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 2) return launch_rows<2>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 4) return launch_rows<4>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 8) return launch_rows<8>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 12) return launch_rows<12>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 16) return launch_rows<16>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 20) return launch_rows<20>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 24) return launch_rows<24>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    if (r <= 28) return launch_rows<28>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
    return launch_rows<32>(probs, mask, kept_idx, kept_cnt, rows, nkb, k, p, stream);
  }
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
