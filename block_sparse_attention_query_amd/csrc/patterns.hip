// Fixed-pattern block masks and the window transpose of the token axis (gfx950).
//
// Patterns (SQuad page, section "手法": a local pass inside windows of w tokens and a global pass
// among the tokens at the same position inside their window; Sparse-vDiT page, section
// "3. 中核となる技術的要素": diagonal, multi-diagonal and vertical-stripe patterns). A block pair
// (i, j) is kept when some query token of block i and some key token of block j satisfy the
// pattern; each test below decides that from the two blocks' token intervals
// [qlo, qhi] and [klo, khi] alone.
#include "sa_common.h"

namespace sa {

constexpr int PAT_LOCAL = 1, PAT_GLOBAL = 2, PAT_DIAG = 4, PAT_MULTIDIAG = 8, PAT_STRIPE = 16;

__device__ __forceinline__ long long floor_div(long long x, long long p) {
  return x >= 0 ? x / p : -((-x + p - 1) / p);
}

__device__ __forceinline__ bool pattern_keep(int kinds, long long qlo, long long qhi, long long klo, long long khi,
                                             long long w, long long band, long long period) {
  bool keep = false;
  if (kinds & PAT_LOCAL)  // the two intervals share a window
    keep |= qlo / w <= khi / w && klo / w <= qhi / w;
  if (kinds & PAT_GLOBAL) {  // the arcs of positions-in-window (mod w) of the two intervals meet
    const long long lq = qhi - qlo + 1, lk = khi - klo + 1;
    if (lq >= w || lk >= w) {
      keep = true;
    } else {
      const long long a = qlo % w, b = klo % w;
      keep |= ((b - a + w) % w) < lq || ((a - b + w) % w) < lk;
    }
  }
  if (kinds & PAT_DIAG) {  // distance between the intervals
    const long long d = max(0LL, max(klo - qhi, qlo - khi));
    keep |= d <= band;
  }
  if (kinds & PAT_MULTIDIAG) {  // some shift of the key interval by a multiple of period is within band
    const long long lo = klo - qhi - band, hi = khi - qlo + band;
    keep |= floor_div(hi, period) * period >= lo;
  }
  if (kinds & PAT_STRIPE)  // the key interval holds a multiple of period
    keep |= (khi / period) * period >= klo;
  return keep;
}

// One wave per mask row (b, h, i): the mask row and, optionally, the ascending kept list.
__global__ __launch_bounds__(256) void pattern_mask_kernel(int kinds, int window, int band, int period, int rows,
                                                           int nqb, int nkb, int N, int Bq, int Bk,
                                                           uint8_t* __restrict__ mask, int32_t* __restrict__ kidx,
                                                           int32_t* __restrict__ kcnt) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int i = row % nqb;
  const long long qlo = (long long)i * Bq, qhi = min((long long)N, qlo + Bq) - 1;
  uint8_t* m = mask + (size_t)row * nkb;
  int32_t* out = kidx != nullptr ? kidx + (size_t)row * nkb : nullptr;
  int cnt = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    bool f = false;
    if (j < nkb) {
      const long long klo = (long long)j * Bk, khi = min((long long)N, klo + Bk) - 1;
      f = pattern_keep(kinds, qlo, qhi, klo, khi, window, band, period);
      m[j] = f ? 1 : 0;
    }
    if (out != nullptr) {
      const uint64_t b = __ballot(f);
      if (f) out[cnt + __popcll(b & ((1ull << lane) - 1ull))] = j;
      cnt += __popcll(b);
    }
  }
  if (out != nullptr && lane == 0) kcnt[row] = cnt;
}

// Window transpose of the token axis: with nw = N / w, forward writes out[s] = x[(s % nw) w + s / nw]
// (the tokens at one position inside their window become contiguous), inverse undoes it. One
// thread moves 16 bytes of a token row.
__global__ __launch_bounds__(256) void window_transpose_kernel(const char* __restrict__ x, char* __restrict__ out,
                                                               long long rows, int N, int w, int row_bytes,
                                                               int inverse) {
  const int vpr = row_bytes / 16;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * vpr) return;
  const long long r = e / vpr;
  const int c = (int)(e - r * vpr);
  const long long bh = r / N;
  const int s = (int)(r - bh * N);
  const int nw = N / w;
  const int src = inverse ? (s % w) * nw + s / w : (s % nw) * w + s / nw;
  *reinterpret_cast<uint4*>(out + (size_t)r * row_bytes + (size_t)c * 16) =
      *reinterpret_cast<const uint4*>(x + ((size_t)bh * N + src) * row_bytes + (size_t)c * 16);
}

hipError_t launch_pattern_mask(int kinds, int window, int band, int period, int BH, int N, int Bq, int Bk,
                               uint8_t* mask, int32_t* kidx, int32_t* kcnt, hipStream_t stream) {
  const int nqb = (N + Bq - 1) / Bq, nkb = (N + Bk - 1) / Bk;
  const int rows = BH * nqb;
  hipLaunchKernelGGL(pattern_mask_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, kinds, window, band,
                     period, rows, nqb, nkb, N, Bq, Bk, mask, kidx, kcnt);
  return hipGetLastError();
}

hipError_t launch_window_transpose(const void* x, void* out, int BH, int N, int row_bytes, int w, int inverse,
                                   hipStream_t stream) {
  const long long rows = (long long)BH * N;
  const long long threads = rows * (row_bytes / 16);
  hipLaunchKernelGGL(window_transpose_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const char*>(x), static_cast<char*>(out), rows, N, w, row_bytes, inverse);
  return hipGetLastError();
}

}  // namespace sa
