// Block mean pooling of Q and K (gfx950).
//
// Consecutive tokens form a block that is represented by one pooled vector (Sparse VideoGen2
// page, section "1. 問題定義"); the mean over the block's valid tokens is taken. The kernel is
// HBM-bound: every Q and K element is read exactly once with 16-byte coalesced loads, summed in
// float64 (exact for bf16 inputs), reduced across row groups by lane shuffles and across the
// four waves through LDS, and divided once by the valid token count. Inputs larger than the
// chip's last-level cache are read with non-temporal loads: they stream through without
// displacing cached lines and reach a higher read rate (5.8 against 5.4 TB/s at 1.5 GB); smaller
// inputs, which the cache may still hold from their producer, keep ordinary loads.
#include "sa_common.h"

namespace sa {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int DT, int D, bool NT>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                   int BH, int N, int Bq, int Bk, int nqb, int nkb,
                                                   double* __restrict__ qp, double* __restrict__ kp) {
  constexpr int ES = DT == kBF16 ? 2 : 4;  // bytes per element
  constexpr int EPV = 16 / ES;             // elements per 16-byte vector
  constexpr int VPR = D / EPV;             // vectors per token row
  constexpr int RG = 256 / VPR;            // token rows covered by one pass of the workgroup
  constexpr int MAXR = 128 / RG;           // passes for the largest block (Bq, Bk <= 128)
  __shared__ double red[4][D];             // one partial sum per wave

  int blk = blockIdx.x;
  const char* src;
  double* dst;
  int bsz, bh, i;
  if (blk < BH * nqb) {
    bh = blk / nqb;
    i = blk - bh * nqb;
    src = static_cast<const char*>(q);
    bsz = Bq;
    dst = qp + (size_t)blk * D;
  } else {
    blk -= BH * nqb;
    bh = blk / nkb;
    i = blk - bh * nkb;
    src = static_cast<const char*>(k);
    bsz = Bk;
    dst = kp + (size_t)blk * D;
  }
  const int row0 = i * bsz;
  const int nvalid = min(bsz, N - row0);
  const uint4* base = reinterpret_cast<const uint4*>(src + ((size_t)bh * N + row0) * (size_t)(D * ES));
  const int c = threadIdx.x % VPR;
  const int r0 = threadIdx.x / VPR;

  // every load of the thread is issued before the first sum
  uint4 v[MAXR];
#pragma unroll
  for (int u = 0; u < MAXR; ++u) {
    const int r = r0 + u * RG;
    if (r >= nvalid) {
      v[u] = make_uint4(0, 0, 0, 0);
    } else if constexpr (NT) {
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + (size_t)r * VPR + c);
      v[u] = make_uint4(x[0], x[1], x[2], x[3]);
    } else {
      v[u] = base[(size_t)r * VPR + c];
    }
  }
  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
#pragma unroll
  for (int u = 0; u < MAXR; ++u) {
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    if constexpr (DT == kBF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)bf16_lo(w[e]);
        acc[2 * e + 1] += (double)bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += (double)__uint_as_float(w[e]);
    }
  }
  // lanes l, l ^ VPR, l ^ 2 VPR, ... of a wave hold the same channels: sum them by shuffles, then
  // the four waves through LDS (sums of bf16 values in float64 are exact, so the order is free)
#pragma unroll
  for (int m = VPR; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += __shfl_xor(acc[e], m, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane < VPR) {
#pragma unroll
    for (int e = 0; e < EPV; ++e) red[wave][c * EPV + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const double s = (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
    dst[threadIdx.x] = s / (double)nvalid;
  }
}

// Inputs above this size (Q and K together) use non-temporal loads: 256 MiB, the size of the
// MI355X last-level cache.
constexpr size_t kStreamBytes = size_t(256) << 20;

template <int DT, int D>
static void launch_pool_t(const void* q, const void* k, int BH, int N, int Bq, int Bk, int nqb, int nkb, double* qp,
                          double* kp, hipStream_t stream) {
  const dim3 grid((unsigned)(BH * (nqb + nkb)));
  const size_t bytes = (size_t)2 * BH * N * D * (DT == kBF16 ? 2 : 4);
  if (bytes > kStreamBytes)
    hipLaunchKernelGGL((pool_kernel<DT, D, true>), grid, dim3(256), 0, stream, q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp);
  else
    hipLaunchKernelGGL((pool_kernel<DT, D, false>), grid, dim3(256), 0, stream, q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp);
}

hipError_t launch_pool(const void* q, const void* k, int dtype, int BH, int N, int d, int Bq, int Bk,
                       double* qp, double* kp, hipStream_t stream) {
  const int nqb = (N + Bq - 1) / Bq;
  const int nkb = (N + Bk - 1) / Bk;
  if (dtype == kBF16 && d == 128) launch_pool_t<kBF16, 128>(q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp, stream);
  else if (dtype == kBF16 && d == 64) launch_pool_t<kBF16, 64>(q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp, stream);
  else if (dtype == kF32 && d == 128) launch_pool_t<kF32, 128>(q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp, stream);
  else launch_pool_t<kF32, 64>(q, k, BH, N, Bq, Bk, nqb, nkb, qp, kp, stream);
  return hipGetLastError();
}

}  // namespace sa
