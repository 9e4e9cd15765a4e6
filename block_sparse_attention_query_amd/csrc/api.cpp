// C ABI entry points: host-side argument checks, shape arithmetic and kernel launches.
// Every check runs before the first HIP call, so invalid arguments enqueue nothing (and can be
// exercised on a machine without a GPU).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/sparse_attn.h"

namespace sa {
hipError_t launch_pool(const void* q, const void* k, int dtype, int BH, int N, int d, int Bq, int Bk, double* qp,
                       double* kp, hipStream_t stream);
hipError_t launch_select(const double* qp, const double* kp, int BH, int nqb, int nkb, int d, double scale, int k,
                         double p, double* probs, uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt,
                         hipStream_t stream);
hipError_t launch_compact(const uint8_t* mask, int rows, int nkb, int32_t* kidx, int32_t* kcnt, hipStream_t stream);
hipError_t launch_attn(const void* q, const void* k, const void* v, int dtype, const int32_t* kidx,
                       const int32_t* kcnt, int BH, int N, int d, int Bq, double scale, void* o, float* lse,
                       hipStream_t stream, const int32_t* row_order = nullptr);
hipError_t launch_row_order(const int32_t* kcnt, int rows, int32_t* order, hipStream_t stream);
hipError_t launch_attn_window(const void* q, const void* k, const void* v, const int32_t* kidx, const int32_t* kcnt,
                              int BH, int N, int d, int Bq, double scale, int window, void* o, float* lse,
                              hipStream_t stream);
hipError_t launch_attn_squad(const void* q, const void* k, const void* v, int BH, int N, int d, int Bq, double scale,
                             int window, bool global_pass, void* o, float* lse, hipStream_t stream);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      const uint8_t* mask, int BH, int N, int d, int Bq, double scale, void* dq, void* dk, void* dv,
                      void* ws, hipStream_t stream);
size_t bwd_workspace_bytes(int BH, int N, int Bq);
hipError_t launch_pattern_mask(int kinds, int window, int band, int period, int BH, int N, int Bq, int Bk,
                               uint8_t* mask, int32_t* kidx, int32_t* kcnt, hipStream_t stream);
hipError_t launch_window_transpose(const void* x, void* out, int BH, int N, int row_bytes, int w, int inverse,
                                   hipStream_t stream);
size_t probe_workspace_bytes(int BH, int N, int d, int Bq, int P);
hipError_t launch_probe(const void* q, const void* k, const void* v, void* o, int BH, int N, int d, int Bq,
                        double scale, int P, double ridge, int rank, float* a_user, float* exact_user, void* ws,
                        hipStream_t stream);
size_t kmeans_workspace_bytes(int BH, int N, int d, int C);
hipError_t launch_kmeans(const void* x, int BH, int N, int d, int C, int iters, const float* init, float* cen,
                         int32_t* labels, int32_t* perm, int32_t* offsets, void* ws, hipStream_t stream);
hipError_t launch_cluster_select(const float* cq, const float* ck, const int32_t* koff, int BH, int Cq, int Ck, int d,
                                 double scale, double p, double* probs, uint8_t* mask, hipStream_t stream);
hipError_t launch_permute_rows(const void* x, const int32_t* perm, int BH, int N, int row_bytes, int inverse,
                               void* out, hipStream_t stream);
int cluster_max_tiles(int N, int Cq, int Bq);
size_t cluster_fwd_workspace_bytes(int BH, int N, int Cq, int Ck, int Bq);
hipError_t launch_cluster_fwd(const void* q, const void* k, const void* v, int BH, int N, int d, const int32_t* qoff,
                              int Cq, const int32_t* koff, int Ck, const uint8_t* mask, const int32_t* qperm,
                              const int32_t* kperm, int Bq, double scale, void* o, float* lse, void* ws,
                              hipStream_t stream);
}  // namespace sa

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return SA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int cdiv(int a, int b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shapes shared by the calls; products are checked to stay within 32-bit grid limits.
int check_shape(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return fail(SA_ERR_INVALID_ARG, "B, H, N and d must be positive");
  if ((long long)B * H > 65535) return fail(SA_ERR_UNSUPPORTED, "B*H = %lld exceeds 65535", (long long)B * H);
  if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d);
  return SA_OK;
}

int check_dtype(int dtype) {
  if (dtype != SA_BF16 && dtype != SA_F32) return fail(SA_ERR_UNSUPPORTED, "dtype %d not SA_BF16 or SA_F32", dtype);
  return SA_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

extern "C" {

int sparse_attn_topk_count(double k_frac, int nkb) {
  if (!(k_frac >= 0.0 && k_frac <= 1.0) || nkb <= 0) return -1;
  double x = ceil(k_frac * (double)nkb - 1e-9);
  if (x < 0.0) x = 0.0;
  if (x > (double)nkb) x = (double)nkb;
  return (int)x;
}

const char* sparse_attn_error_string(int code) {
  switch (code) {
    case SA_OK: return "ok";
    case SA_ERR_INVALID_ARG: return "invalid argument";
    case SA_ERR_UNSUPPORTED: return "unsupported configuration";
    case SA_ERR_HIP: return "HIP error";
    default: return "unknown error code";
  }
}

const char* sparse_attn_last_error(void) { return g_last_error; }

int sparse_attn_pool_qk(const void* q, const void* k, int dtype, int B, int H, int N, int d, int Bq, int Bk,
                        double* q_pool, double* k_pool, void* stream) {
  if (!q || !k || !q_pool || !k_pool) return fail(SA_ERR_INVALID_ARG, "pool_qk: null pointer");
  int rc = check_shape(B, H, N, d);
  if (rc) return rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((Bq != 64 && Bq != 128) || (Bk != 64 && Bk != 128))
    return fail(SA_ERR_UNSUPPORTED, "pool_qk: block sizes Bq=%d Bk=%d not in {64, 128}", Bq, Bk);
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_pool) || !aligned16(k_pool))
    return fail(SA_ERR_INVALID_ARG, "pool_qk: pointers must be 16-byte aligned");
  const long long blocks = (long long)B * H * (cdiv(N, Bq) + cdiv(N, Bk));
  if (blocks > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "pool_qk: too many blocks");
  return hip_status(sa::launch_pool(q, k, dtype, B * H, N, d, Bq, Bk, q_pool, k_pool,
                                    static_cast<hipStream_t>(stream)),
                    "pool_qk launch");
}

int sparse_attn_select_mask(const double* q_pool, const double* k_pool, int B, int H, int nqb, int nkb, int d,
                            double scale, double k_frac, double p, double* probs, uint8_t* mask, int32_t* kept_idx,
                            int32_t* kept_cnt, void* stream) {
  if (!q_pool || !k_pool || !mask) return fail(SA_ERR_INVALID_ARG, "select_mask: null pointer");
  if ((kept_idx == nullptr) != (kept_cnt == nullptr))
    return fail(SA_ERR_INVALID_ARG, "select_mask: kept_idx and kept_cnt must both be given or both be NULL");
  if (nqb <= 0 || nkb <= 0) return fail(SA_ERR_INVALID_ARG, "select_mask: nqb and nkb must be positive");
  int rc = check_shape(B, H, 1, d);
  if (rc) return rc;
  if (nkb > SA_MAX_NKB) return fail(SA_ERR_UNSUPPORTED, "select_mask: nkb=%d exceeds %d", nkb, SA_MAX_NKB);
  if (!probs && nkb > SA_SELECT_FUSED_NKB)
    return fail(SA_ERR_INVALID_ARG, "select_mask: probs may be NULL only for nkb <= %d (nkb=%d)",
                SA_SELECT_FUSED_NKB, nkb);
  if ((long long)B * H * nqb > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "select_mask: too many rows");
  if ((cdiv(nqb, 64)) > 65535) return fail(SA_ERR_UNSUPPORTED, "select_mask: nqb too large");
  if (!(scale > 0.0) || !isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "select_mask: scale must be finite and > 0");
  if (!(k_frac >= 0.0 && k_frac <= 1.0)) return fail(SA_ERR_INVALID_ARG, "select_mask: k_frac must lie in [0, 1]");
  if (!(p >= 0.0 && p <= 1.0)) return fail(SA_ERR_INVALID_ARG, "select_mask: p must lie in [0, 1]");
  const int k = sparse_attn_topk_count(k_frac, nkb);
  return hip_status(sa::launch_select(q_pool, k_pool, B * H, nqb, nkb, d, scale, k, p, probs, mask, kept_idx,
                                      kept_cnt, static_cast<hipStream_t>(stream)),
                    "select_mask launch");
}

size_t sparse_attn_fwd_workspace_size(int B, int H, int N, int Bq, int Bk) {
  if (B <= 0 || H <= 0 || N <= 0 || Bq <= 0 || Bk <= 0) return 0;
  const size_t rows = (size_t)B * H * cdiv(N, Bq);
  const size_t nkb = (size_t)cdiv(N, Bk);
  return align_up(rows * nkb * sizeof(int32_t)) + align_up(rows * sizeof(int32_t));
}

namespace {
int check_fwd_common(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d, int Bq,
                     int Bk, double scale, const void* o) {
  if (!q || !k || !v || !o) return fail(SA_ERR_INVALID_ARG, "fwd: null pointer");
  int rc = check_shape(B, H, N, d);
  if (rc) return rc;
  if ((rc = check_dtype(dtype))) return rc;
  if ((Bq != 64 && Bq != 128) || Bk != 64)
    return fail(SA_ERR_UNSUPPORTED, "fwd: block sizes Bq=%d Bk=%d (need Bq in {64,128}, Bk = 64)", Bq, Bk);
  if (!(scale > 0.0) || !isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "fwd: scale must be finite and > 0");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SA_ERR_INVALID_ARG, "fwd: q, k, v and o must be 16-byte aligned");
  if ((long long)B * H * cdiv(N, Bq) > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "fwd: too many query blocks");
  return SA_OK;
}
}  // namespace

int sparse_attn_fwd_lists(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                          const int32_t* kept_cnt, int B, int H, int N, int d, int Bq, int Bk, double scale, void* o,
                          float* lse, void* stream) {
  if (!kept_idx || !kept_cnt) return fail(SA_ERR_INVALID_ARG, "fwd_lists: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, o);
  if (rc) return rc;
  return hip_status(sa::launch_attn(q, k, v, dtype, kept_idx, kept_cnt, B * H, N, d, Bq, scale, o, lse,
                                    static_cast<hipStream_t>(stream)),
                    "fwd_lists: attention launch");
}

int sparse_attn_row_order(const int32_t* kept_cnt, int B, int H, int nqb, int32_t* order, void* stream) {
  if (!kept_cnt || !order) return fail(SA_ERR_INVALID_ARG, "row_order: null pointer");
  if (B <= 0 || H <= 0 || nqb <= 0) return fail(SA_ERR_INVALID_ARG, "row_order: B, H and nqb must be positive");
  if ((long long)B * H * nqb > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "row_order: too many rows");
  return hip_status(sa::launch_row_order(kept_cnt, B * H * nqb, order, static_cast<hipStream_t>(stream)),
                    "row_order: launch");
}

int sparse_attn_fwd_lists_ordered(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                                  const int32_t* kept_cnt, const int32_t* row_order, int B, int H, int N, int d,
                                  int Bq, int Bk, double scale, void* o, float* lse, void* stream) {
  if (!kept_idx || !kept_cnt || !row_order) return fail(SA_ERR_INVALID_ARG, "fwd_lists_ordered: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, o);
  if (rc) return rc;
  return hip_status(sa::launch_attn(q, k, v, dtype, kept_idx, kept_cnt, B * H, N, d, Bq, scale, o, lse,
                                    static_cast<hipStream_t>(stream), row_order),
                    "fwd_lists_ordered: attention launch");
}

int sparse_attn_fwd_lists_window(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                                 const int32_t* kept_cnt, int B, int H, int N, int d, int Bq, int Bk, int window,
                                 double scale, void* o, float* lse, void* stream) {
  if (!kept_idx || !kept_cnt) return fail(SA_ERR_INVALID_ARG, "fwd_lists_window: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, o);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "fwd_lists_window: only SA_BF16 tensors are supported");
  if (Bk != 64) return fail(SA_ERR_UNSUPPORTED, "fwd_lists_window: Bk must be 64");
  if (window <= 0 || N % window != 0) return fail(SA_ERR_INVALID_ARG, "fwd_lists_window: window must divide N");
  if ((long long)N * d * 2 > 0xffffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "fwd_lists_window: one head's rows (N * d * 2 bytes) must stay below 4 GiB");
  if (N / window < 64)
    return fail(SA_ERR_UNSUPPORTED, "fwd_lists_window: N / window = %d runs; at least 64 are needed", N / window);
  return hip_status(sa::launch_attn_window(q, k, v, kept_idx, kept_cnt, B * H, N, d, Bq, scale, window, o, lse,
                                           static_cast<hipStream_t>(stream)),
                    "fwd_lists_window: attention launch");
}

}  // extern "C"

// Scratch of sparse_attn_fwd_noalloc: the kept lists and counts of a group of heads. Every GPU the
// library runs on holds its own copy until the process ends. Host code must not use this name as
// an address (it is a host-side stand-in): the device address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_ERR_UNSUPPORTED, "fwd_noalloc: device %d is beyond the %d devices tracked", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(SA_ERR_HIP, "fwd_noalloc: hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SA_OK;
}

}  // namespace

extern "C" {

int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask, int B, int H,
                            int N, int d, int Bq, int Bk, double scale, void* o, float* lse, void* stream) {
  if (!mask) return fail(SA_ERR_INVALID_ARG, "fwd_noalloc: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, o);
  if (rc) return rc;
  const int nqb = cdiv(N, Bq), nkb = cdiv(N, Bk);
  // one head's lists and counts, each rounded up to the 256-byte alignment of a group's arrays
  const size_t head_bytes = align_up((size_t)nqb * nkb * sizeof(int32_t)) + align_up((size_t)nqb * sizeof(int32_t));
  if (head_bytes > (size_t)SA_NOALLOC_SCRATCH_BYTES)
    return fail(SA_ERR_UNSUPPORTED, "fwd_noalloc: one head's kept lists need %zu bytes; the scratch holds %zu",
                head_bytes, (size_t)SA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  const int BH = B * H;
  const int group = (int)((size_t)SA_NOALLOC_SCRATCH_BYTES / head_bytes < (size_t)BH
                              ? (size_t)SA_NOALLOC_SCRATCH_BYTES / head_bytes
                              : (size_t)BH);
  const size_t es = dtype == SA_BF16 ? 2 : 4;
  const size_t head_elems = (size_t)N * d;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // groups of heads run one after another on the stream, so each reuses the scratch after the
  // previous group's attention has read it
  for (int h0 = 0; h0 < BH; h0 += group) {
    const int g = BH - h0 < group ? BH - h0 : group;
    int32_t* kidx = static_cast<int32_t*>(ws);
    int32_t* kcnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                               align_up((size_t)g * nqb * nkb * sizeof(int32_t)));
    const size_t off = (size_t)h0 * head_elems * es;
    rc = hip_status(sa::launch_compact(mask + (size_t)h0 * nqb * nkb, g * nqb, nkb, kidx, kcnt, s),
                    "fwd_noalloc: compaction launch");
    if (rc) return rc;
    rc = hip_status(sa::launch_attn(static_cast<const char*>(q) + off, static_cast<const char*>(k) + off,
                                    static_cast<const char*>(v) + off, dtype, kidx, kcnt, g, N, d, Bq, scale,
                                    static_cast<char*>(o) + off, lse ? lse + (size_t)h0 * N : nullptr, s),
                    "fwd_noalloc: attention launch");
    if (rc) return rc;
  }
  return ok();
}

int sparse_attn_squad_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d, int Bq,
                          int window, int pass, double scale, void* o, float* lse, void* stream) {
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, 64, scale, o);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "squad_fwd: only SA_BF16 tensors are supported");
  if (pass != SA_SQUAD_LOCAL && pass != SA_SQUAD_GLOBAL)
    return fail(SA_ERR_INVALID_ARG, "squad_fwd: pass must be SA_SQUAD_LOCAL or SA_SQUAD_GLOBAL");
  if (window <= 0 || window > N) return fail(SA_ERR_INVALID_ARG, "squad_fwd: window must be in [1, N]");
  if (pass == SA_SQUAD_GLOBAL) {
    if (N % window != 0) return fail(SA_ERR_INVALID_ARG, "squad_fwd: the global pass needs a window that divides N");
    if ((long long)N * d * 2 > 0xffffffffLL)
      return fail(SA_ERR_UNSUPPORTED, "squad_fwd: one head's rows (N * d * 2 bytes) must stay below 4 GiB");
    if (N / window < 64)
      return fail(SA_ERR_UNSUPPORTED, "squad_fwd: N / window = %d positions per run; at least 64 are needed",
                  N / window);
  }
  return hip_status(sa::launch_attn_squad(q, k, v, B * H, N, d, Bq, scale, window, pass == SA_SQUAD_GLOBAL, o, lse,
                                          static_cast<hipStream_t>(stream)),
                    "squad_fwd: attention launch");
}

int sparse_attn_fwd(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask, int B, int H, int N,
                    int d, int Bq, int Bk, double scale, void* o, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!mask || !workspace) return fail(SA_ERR_INVALID_ARG, "fwd: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, o);
  if (rc) return rc;
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(SA_ERR_INVALID_ARG, "fwd: workspace must be 256-byte aligned");
  const size_t need = sparse_attn_fwd_workspace_size(B, H, N, Bq, Bk);
  if (workspace_bytes < need)
    return fail(SA_ERR_INVALID_ARG, "fwd: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  const int nqb = cdiv(N, Bq), nkb = cdiv(N, Bk);
  const long long rows = (long long)B * H * nqb;
  int32_t* kidx = static_cast<int32_t*>(workspace);
  int32_t* kcnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             align_up((size_t)rows * nkb * sizeof(int32_t)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = hip_status(sa::launch_compact(mask, (int)rows, nkb, kidx, kcnt, s), "fwd: compaction launch");
  if (rc) return rc;
  return hip_status(sa::launch_attn(q, k, v, dtype, kidx, kcnt, B * H, N, d, Bq, scale, o, lse, s),
                    "fwd: attention launch");
}

size_t sparse_attn_bwd_workspace_size(int B, int H, int N, int Bq, int Bk) {
  if (B <= 0 || H <= 0 || N <= 0 || (Bq != 64 && Bq != 128) || Bk != 64) return 0;
  return sa::bwd_workspace_bytes(B * H, N, Bq);
}

int sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    int dtype, const uint8_t* mask, int B, int H, int N, int d, int Bq, int Bk, double scale, void* dq,
                    void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  if (!o || !dout || !lse || !mask || !dq || !dk || !dv || !workspace) return fail(SA_ERR_INVALID_ARG, "bwd: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, Bk, scale, dq);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "bwd: only SA_BF16 tensors are supported");
  if (!aligned16(o) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv))
    return fail(SA_ERR_INVALID_ARG, "bwd: o, dout, dk and dv must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(SA_ERR_INVALID_ARG, "bwd: workspace must be 256-byte aligned");
  const size_t need = sparse_attn_bwd_workspace_size(B, H, N, Bq, Bk);
  if (workspace_bytes < need)
    return fail(SA_ERR_INVALID_ARG, "bwd: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if ((long long)B * H * cdiv(N, Bk) > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "bwd: too many key blocks");
  return hip_status(sa::launch_bwd(q, k, v, o, dout, lse, mask, B * H, N, d, Bq, scale, dq, dk, dv, workspace,
                                   static_cast<hipStream_t>(stream)),
                    "bwd launch");
}

size_t sparse_attn_probe_workspace_size(int B, int H, int N, int d, int Bq, int probes) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128) || (Bq != 64 && Bq != 128) || probes < 1 || probes > 1024)
    return 0;
  if ((long long)B * H > 65535) return 0;
  return sa::probe_workspace_bytes(B * H, N, d, Bq, probes);
}

int sparse_attn_probe_correct(const void* q, const void* k, const void* v, void* o, int dtype, int B, int H, int N,
                              int d, int Bq, double scale, int probes, double ridge, int rank, float* a_out,
                              float* exact_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(SA_ERR_INVALID_ARG, "probe_correct: null workspace");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, 64, scale, o);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "probe_correct: only SA_BF16 tensors are supported");
  if (probes < 1 || probes > 1024) return fail(SA_ERR_INVALID_ARG, "probe_correct: probes=%d not in [1, 1024]", probes);
  if (!(ridge > 0.0) || !isfinite(ridge)) return fail(SA_ERR_INVALID_ARG, "probe_correct: ridge must be finite and > 0");
  if (rank < 1) return fail(SA_ERR_INVALID_ARG, "probe_correct: rank=%d must be at least 1", rank);
  if ((reinterpret_cast<uintptr_t>(a_out) & 15u) || (reinterpret_cast<uintptr_t>(exact_out) & 15u))
    return fail(SA_ERR_INVALID_ARG, "probe_correct: a_out and exact_out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(SA_ERR_INVALID_ARG, "probe_correct: workspace must be 256-byte aligned");
  const size_t need = sparse_attn_probe_workspace_size(B, H, N, d, Bq, probes);
  if (need == 0) return fail(SA_ERR_UNSUPPORTED, "probe_correct: unsupported sizes");
  if (workspace_bytes < need)
    return fail(SA_ERR_INVALID_ARG, "probe_correct: workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  if ((long long)B * H * probes * cdiv(N, 64) > 0x7fffffffLL || (long long)B * H * cdiv(N, 256) > 0x7fffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "probe_correct: too many workgroups");
  return hip_status(sa::launch_probe(q, k, v, o, B * H, N, d, Bq, scale, probes, ridge, rank, a_out, exact_out, workspace,
                                     static_cast<hipStream_t>(stream)),
                    "probe_correct launch");
}

size_t sparse_attn_kmeans_workspace_size(int B, int H, int N, int d, int C) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128) || C <= 0 || C > SA_MAX_CLUSTERS || C > N) return 0;
  return sa::kmeans_workspace_bytes(B * H, N, d, C);
}

int sparse_attn_kmeans(const void* x, int dtype, int B, int H, int N, int d, int C, int iters, const float* init,
                       float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!x || !centroids || !labels || !perm || !offsets || !workspace) return fail(SA_ERR_INVALID_ARG, "kmeans: null pointer");
  int rc = check_shape(B, H, N, d);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "kmeans: only SA_BF16 tensors are supported");
  if (C <= 0 || C > N) return fail(SA_ERR_INVALID_ARG, "kmeans: C=%d must lie in [1, N]", C);
  if (C > SA_MAX_CLUSTERS) return fail(SA_ERR_UNSUPPORTED, "kmeans: C=%d exceeds %d", C, SA_MAX_CLUSTERS);
  if (iters < 1) return fail(SA_ERR_INVALID_ARG, "kmeans: iters must be >= 1");
  if (!aligned16(x)) return fail(SA_ERR_INVALID_ARG, "kmeans: x must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(SA_ERR_INVALID_ARG, "kmeans: workspace must be 256-byte aligned");
  const size_t need = sparse_attn_kmeans_workspace_size(B, H, N, d, C);
  if (workspace_bytes < need)
    return fail(SA_ERR_INVALID_ARG, "kmeans: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if ((long long)cdiv(N, 256) > 65535) return fail(SA_ERR_UNSUPPORTED, "kmeans: N too large");
  return hip_status(sa::launch_kmeans(x, B * H, N, d, C, iters, init, centroids, labels, perm, offsets, workspace,
                                      static_cast<hipStream_t>(stream)),
                    "kmeans launch");
}

int sparse_attn_cluster_select(const float* cq, const float* ck, const int32_t* k_offsets, int B, int H, int Cq, int Ck,
                               int d, double scale, double p, double* probs, uint8_t* mask, void* stream) {
  if (!cq || !ck || !k_offsets || !mask) return fail(SA_ERR_INVALID_ARG, "cluster_select: null pointer");
  if (B <= 0 || H <= 0 || Cq <= 0 || Ck <= 0) return fail(SA_ERR_INVALID_ARG, "cluster_select: sizes must be positive");
  if ((long long)B * H > 65535) return fail(SA_ERR_UNSUPPORTED, "cluster_select: B*H exceeds 65535");
  if (d != 64 && d != 128) return fail(SA_ERR_UNSUPPORTED, "cluster_select: head dim %d not in {64, 128}", d);
  if (Cq > SA_MAX_CLUSTERS || Ck > SA_MAX_CLUSTERS)
    return fail(SA_ERR_UNSUPPORTED, "cluster_select: cluster counts exceed %d", SA_MAX_CLUSTERS);
  if (!(scale > 0.0) || !isfinite(scale)) return fail(SA_ERR_INVALID_ARG, "cluster_select: scale must be finite and > 0");
  if (!(p >= 0.0 && p <= 1.0)) return fail(SA_ERR_INVALID_ARG, "cluster_select: p must lie in [0, 1]");
  return hip_status(sa::launch_cluster_select(cq, ck, k_offsets, B * H, Cq, Ck, d, scale, p, probs, mask,
                                              static_cast<hipStream_t>(stream)),
                    "cluster_select launch");
}

int sparse_attn_permute_rows(const void* x, int dtype, int B, int H, int N, int d, const int32_t* perm, int inverse,
                             void* out, void* stream) {
  if (!x || !perm || !out) return fail(SA_ERR_INVALID_ARG, "permute_rows: null pointer");
  int rc = check_shape(B, H, N, d);
  if (rc) return rc;
  if ((rc = check_dtype(dtype))) return rc;
  if (x == out) return fail(SA_ERR_INVALID_ARG, "permute_rows: out must not alias x");
  if (!aligned16(x) || !aligned16(out)) return fail(SA_ERR_INVALID_ARG, "permute_rows: pointers must be 16-byte aligned");
  const long long pieces = (long long)B * H * N * (d * (dtype == SA_BF16 ? 2 : 4) / 16);
  if ((pieces + 255) / 256 > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "permute_rows: tensor too large");
  return hip_status(sa::launch_permute_rows(x, perm, B * H, N, d * (dtype == SA_BF16 ? 2 : 4), inverse != 0, out,
                                            static_cast<hipStream_t>(stream)),
                    "permute_rows launch");
}

size_t sparse_attn_cluster_fwd_workspace_size(int B, int H, int N, int Cq, int Ck, int Bq) {
  if (B <= 0 || H <= 0 || N <= 0 || Cq <= 0 || Ck <= 0 || Cq > SA_MAX_CLUSTERS || Ck > SA_MAX_CLUSTERS ||
      (Bq != 64 && Bq != 128))
    return 0;
  return sa::cluster_fwd_workspace_bytes(B * H, N, Cq, Ck, Bq);
}

int sparse_attn_cluster_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d,
                            const int32_t* q_offsets, int Cq, const int32_t* k_offsets, int Ck, const uint8_t* mask,
                            const int32_t* q_perm, const int32_t* k_perm, int Bq, double scale, void* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!q_offsets || !k_offsets || !mask || !workspace) return fail(SA_ERR_INVALID_ARG, "cluster_fwd: null pointer");
  int rc = check_fwd_common(q, k, v, dtype, B, H, N, d, Bq, 64, scale, o);
  if (rc) return rc;
  if (dtype != SA_BF16) return fail(SA_ERR_UNSUPPORTED, "cluster_fwd: only SA_BF16 tensors are supported");
  if ((long long)N * d * 2 > 0xffffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "cluster_fwd: one head's rows (N * d * 2 bytes) must stay below 4 GiB");
  if (Cq <= 0 || Ck <= 0 || Cq > N || Ck > N) return fail(SA_ERR_INVALID_ARG, "cluster_fwd: cluster counts must lie in [1, N]");
  if (Cq > SA_MAX_CLUSTERS || Ck > SA_MAX_CLUSTERS)
    return fail(SA_ERR_UNSUPPORTED, "cluster_fwd: cluster counts exceed %d", SA_MAX_CLUSTERS);
  if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
    return fail(SA_ERR_INVALID_ARG, "cluster_fwd: workspace must be 256-byte aligned");
  const size_t need = sparse_attn_cluster_fwd_workspace_size(B, H, N, Cq, Ck, Bq);
  if (workspace_bytes < need)
    return fail(SA_ERR_INVALID_ARG, "cluster_fwd: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                need);
  if ((long long)B * H * sa::cluster_max_tiles(N, Cq, Bq) > 0x7fffffffLL)
    return fail(SA_ERR_UNSUPPORTED, "cluster_fwd: too many query tiles");
  return hip_status(sa::launch_cluster_fwd(q, k, v, B * H, N, d, q_offsets, Cq, k_offsets, Ck, mask, q_perm, k_perm,
                                           Bq, scale, o, lse, workspace, static_cast<hipStream_t>(stream)),
                    "cluster_fwd launch");
}

int sparse_attn_pattern_mask(int patterns, int window, int band, int period, int B, int H, int N, int Bq, int Bk,
                             uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, void* stream) {
  if (!mask) return fail(SA_ERR_INVALID_ARG, "pattern_mask: null mask");
  if ((kept_idx == nullptr) != (kept_cnt == nullptr))
    return fail(SA_ERR_INVALID_ARG, "pattern_mask: kept_idx and kept_cnt must both be given or both be NULL");
  if (B <= 0 || H <= 0 || N <= 0) return fail(SA_ERR_INVALID_ARG, "pattern_mask: B, H and N must be positive");
  if ((long long)B * H > 65535) return fail(SA_ERR_UNSUPPORTED, "pattern_mask: B*H exceeds 65535");
  if ((Bq != 64 && Bq != 128) || (Bk != 64 && Bk != 128))
    return fail(SA_ERR_UNSUPPORTED, "pattern_mask: block sizes Bq=%d Bk=%d not in {64, 128}", Bq, Bk);
  if (patterns <= 0 || (patterns & ~(SA_PAT_LOCAL | SA_PAT_GLOBAL | SA_PAT_DIAG | SA_PAT_MULTIDIAG | SA_PAT_STRIPE)))
    return fail(SA_ERR_INVALID_ARG, "pattern_mask: pattern set 0x%x is empty or has unknown bits", patterns);
  if ((patterns & (SA_PAT_LOCAL | SA_PAT_GLOBAL)) && window <= 0)
    return fail(SA_ERR_INVALID_ARG, "pattern_mask: window must be positive");
  if ((patterns & (SA_PAT_DIAG | SA_PAT_MULTIDIAG)) && band < 0)
    return fail(SA_ERR_INVALID_ARG, "pattern_mask: band must be >= 0");
  if ((patterns & (SA_PAT_MULTIDIAG | SA_PAT_STRIPE)) && period <= 0)
    return fail(SA_ERR_INVALID_ARG, "pattern_mask: period must be positive");
  const int nkb = cdiv(N, Bk);
  if (nkb > SA_MAX_NKB) return fail(SA_ERR_UNSUPPORTED, "pattern_mask: nkb=%d exceeds %d", nkb, SA_MAX_NKB);
  if ((long long)B * H * cdiv(N, Bq) > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "pattern_mask: too many rows");
  return hip_status(sa::launch_pattern_mask(patterns, window > 0 ? window : 1, band, period > 0 ? period : 1, B * H,
                                            N, Bq, Bk, mask, kept_idx, kept_cnt, static_cast<hipStream_t>(stream)),
                    "pattern_mask launch");
}

int sparse_attn_window_transpose(const void* x, int dtype, int B, int H, int N, int d, int window, int inverse,
                                 void* out, void* stream) {
  if (!x || !out) return fail(SA_ERR_INVALID_ARG, "window_transpose: null pointer");
  int rc = check_shape(B, H, N, d);
  if (rc) return rc;
  if ((rc = check_dtype(dtype))) return rc;
  if (window <= 0 || N % window != 0)
    return fail(SA_ERR_INVALID_ARG, "window_transpose: window %d must be positive and divide N = %d", window, N);
  if (x == out) return fail(SA_ERR_INVALID_ARG, "window_transpose: out must not alias x");
  if (!aligned16(x) || !aligned16(out)) return fail(SA_ERR_INVALID_ARG, "window_transpose: pointers must be 16-byte aligned");
  const long long threads = (long long)B * H * N * (d * (dtype == SA_BF16 ? 2 : 4) / 16);
  if ((threads + 255) / 256 > 0x7fffffffLL) return fail(SA_ERR_UNSUPPORTED, "window_transpose: tensor too large");
  return hip_status(sa::launch_window_transpose(x, out, B * H, N, d * (dtype == SA_BF16 ? 2 : 4), window, inverse != 0,
                                                static_cast<hipStream_t>(stream)),
                    "window_transpose launch");
}

}  // extern "C"
