/*
 * sparse_attn.h - C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * Training-free block-sparse softmax attention in the SpargeAttention2 form:
 *   1. sparse_attn_pool_qk      mean-pool Q and K over consecutive token blocks;
 *   2. sparse_attn_select_mask  pooled scores, a softmax per query block, and the hybrid
 *                               Top-k U Top-p block mask;
 *   3. sparse_attn_fwd          flash-style attention of every query block over its kept key
 *                               blocks only.
 *
 * Pages the operations follow:
 *   [SA2]  "SpargeAttention2とは？Top-k+Top-pハイブリッドマスキングでビデオ生成を16.2倍高速化"
 *          (ai-papers.net), sections "Top-kとTop-pの限界を解剖する" and
 *          "ハイブリッドマスキングと蒸留微調整".
 *   [SVG2] "Sparse VideoGen2: Accelerate Video Generation with Sparse Attention via
 *          Semantic-Aware Permutation" (gist.science), sections "1. 問題定義" and "2. 手法" A, B, C.
 *   [SPR]  "Partition the Support, Reconstruct the Residual: Training-Free Sparse Attention for
 *          Video Generation and World Models" (physicalainews.jp), original abstract.
 *   [SQ]   "SQuad: Sub-Quadratic Attention Distillation for Efficient Video Generation"
 *          (gist.science), section "手法".
 *   [SVD]  "Sparse-vDiT: Unleashing the Power of Sparse Attention to Accelerate Video Diffusion
 *          Transformers" (aibr.jp), section "3. 中核となる技術的要素".
 *
 * Conventions for every call:
 *   - Pointers marked "device" are device memory on the current HIP device; all tensors are
 *     dense and contiguous in the stated layout; the caller allocates and owns every buffer.
 *   - The library never allocates, frees or synchronises. Work is enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the null stream) and runs asynchronously.
 *   - Arguments are checked on the host before anything is enqueued. A non-zero return means
 *     nothing was enqueued, except SA_ERR_HIP, which reports a failed launch.
 *     sparse_attn_last_error() then holds a message for the calling thread.
 *   - NaN or Inf inside the tensors is not checked; it propagates.
 *   - Shapes: B batch, H heads, N tokens, d head dim, Bq / Bk query / key block sizes,
 *     nQB = ceil(N / Bq), nKB = ceil(N / Bk). The last block of each may be partial; pooling
 *     averages its valid tokens and padded keys never take part in attention.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define SA_OK 0
#define SA_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, value out of range   */
#define SA_ERR_UNSUPPORTED (-2) /* d, Bq, Bk, dtype or nKB outside the instantiated set    */
#define SA_ERR_HIP (-3)         /* a HIP launch failed; the HIP message is kept          */

/* Element types of Q, K, V and O. SA_BF16 attention runs on bf16 MFMA operands (P rounded to
 * bf16 for the P V product) with fp32 accumulation; SA_F32 attention runs on the fp32 matrix
 * instruction with fp32 P, so no fp32 input is rounded. */
#define SA_BF16 0
#define SA_F32 1

/* Supported values (others return SA_ERR_UNSUPPORTED): d in {64, 128}; Bq in {64, 128};
 * Bk = 64 for sparse_attn_fwd (pooling accepts Bq, Bk in {64, 128}); nKB <= 8192. */
#define SA_MAX_NKB 8192
/* Rows of at most this many key blocks are selected in one kernel that keeps the scores on chip;
 * only there may sparse_attn_select_mask take probs = NULL. */
#define SA_SELECT_FUSED_NKB 1280
#define SA_MAX_CLUSTERS 1024  /* clusters per head for the semantic-aware permutation calls */

/*
 * Block mean pooling of Q and K ([SVG2] "1. 問題定義": consecutive tokens grouped into blocks,
 * each represented by a pooled vector; mean pooling).
 *
 *   q, k      device, [B, H, N, d] of `dtype`.
 *   q_pool    device out, [B, H, nQB, d] float64: q_pool[b,h,i,:] = mean of Q rows
 *             i*Bq .. min(N, (i+1)*Bq) - 1.
 *   k_pool    device out, [B, H, nKB, d] float64, the same over key blocks of Bk.
 * Sums are accumulated in float64, so the means are exact up to the final division.
 */
int sparse_attn_pool_qk(const void* q, const void* k, int dtype, int B, int H, int N, int d,
                        int Bq, int Bk, double* q_pool, double* k_pool, void* stream);

/*
 * Pooled probability pattern and hybrid block mask ([SA2] "Top-kとTop-pの限界を解剖する",
 * "ハイブリッドマスキングと蒸留微調整"; [SVG2] "2. 手法" B).
 *
 *   q_pool, k_pool   device, [B, H, nqb, d] and [B, H, nkb, d] float64 (from pool_qk).
 *   scale            score scale, normally 1/sqrt(d).
 *   k_frac           Top-k fraction in [0, 1]; k = min(nkb, ceil(k_frac * nkb - 1e-9)).
 *   p                Top-p mass in [0, 1]; keeps the shortest prefix of the descending order
 *                    whose running sum is >= p (p = 0 keeps none by Top-p).
 *   probs            device out or NULL, [B, H, nqb, nkb] float64: softmax over j of
 *                    scale * <q_pool[b,h,i], k_pool[b,h,j]>. Given, it also holds the scores
 *                    between the score and selection kernels. NULL (nothing written) is accepted
 *                    for nkb <= SA_SELECT_FUSED_NKB: one kernel then keeps the scores of 16
 *                    query-block rows at a time in LDS (no HBM round trip, but slower than the
 *                    two kernels at the shapes measured); longer rows without probs return
 *                    SA_ERR_INVALID_ARG. Masks and lists are the same either way.
 *   mask             device out, [B, H, nqb, nkb] uint8, 1 = keep. Row i keeps the first
 *                    max(k, m*) blocks of the order "descending probability, lower index first
 *                    on equality", m* being the Top-p prefix length.
 *   kept_idx         device out or NULL, [B, H, nqb, nkb] int32: per row the kept block
 *                    indices in ascending order in the first kept_cnt entries (rest unwritten).
 *   kept_cnt         device out or NULL (both or neither), [B, H, nqb] int32.
 * Scores, softmax and running sums are float64.
 */
int sparse_attn_select_mask(const double* q_pool, const double* k_pool, int B, int H, int nqb,
                            int nkb, int d, double scale, double k_frac, double p, double* probs,
                            uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/* Bytes of device workspace sparse_attn_fwd needs for these shapes (kept-block lists and
 * per-row counts, 256-byte aligned). Returns 0 for invalid shapes. */
size_t sparse_attn_fwd_workspace_size(int B, int H, int N, int Bq, int Bk);

/*
 * Block-sparse attention forward ([SVG2] "2. 手法" C: scattered K/V blocks are loaded, the
 * contiguous query block is computed densely; [SPR] abstract: queries sharing a block route
 * share its key support).
 *
 *   q, k, v     device, [B, H, N, d] of `dtype`.
 *   mask        device, [B, H, nQB, nKB] uint8, any 0/1 pattern (from select_mask, all ones for
 *               dense attention, or a caller's own).
 *   scale       softmax scale, normally 1/sqrt(d).
 *   o           device out, [B, H, N, d] of `dtype`: for every query t of block i,
 *               O[t] = sum_u softmax_u(scale * Q[t].K[u]) V[u] over the keys u < N of the kept
 *               blocks of row i. A row with no kept block gives O = 0.
 *   lse         device out or NULL, [B, H, N] float32: natural-log log-sum-exp of the scaled
 *               scores over the same keys (-inf for an empty row).
 *   workspace   device scratch of at least sparse_attn_fwd_workspace_size() bytes, 256-byte
 *               aligned; overwritten.
 * The mask is compacted into ascending kept-block lists in the workspace, then one workgroup
 * per (b, h, query block) walks its list with bf16 (or, for SA_F32, fp32) MFMA and an fp32
 * online softmax (for SA_BF16 with d = 128 and Bq = 64, one workgroup per two neighbouring query
 * blocks walks the union of their lists, each block scored only for the rows that keep it; same
 * results).
 */
int sparse_attn_fwd(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask,
                    int B, int H, int N, int d, int Bq, int Bk, double scale, void* o, float* lse,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sparse_attn_fwd without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The kept lists go to
 * a scratch array inside the library (SA_NOALLOC_SCRATCH_BYTES per GPU, held until the process
 * ends); heads are processed in groups whose lists fit in it, one group after another on
 * `stream`. The call itself allocates nothing. Arguments, arithmetic and results are those of
 * sparse_attn_fwd (bit-identical outputs).
 * Limit: one head's lists, align256(nQB * nKB * 4) + align256(nQB * 4) bytes, must fit in the
 * scratch (SA_ERR_UNSUPPORTED otherwise; e.g. N = 75600, Bq = 128, Bk = 64 needs 2.8 MB).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (different
 * streams, or threads without ordering) race and give unspecified results.
 */
#define SA_NOALLOC_SCRATCH_BYTES (32u << 20)
int sparse_attn_fwd_noalloc(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask, int B, int H,
                            int N, int d, int Bq, int Bk, double scale, void* o, float* lse, void* stream);

/*
 * The same attention from kept-block lists instead of a mask (the kept_idx / kept_cnt that
 * sparse_attn_select_mask can write), skipping the compaction step.
 *
 *   kept_idx    device, [B, H, nQB, nKB] int32: row r walks kept_idx[r][0 .. kept_cnt[r]-1].
 *   kept_cnt    device, [B, H, nQB] int32.
 * Entries are expected ascending in [0, nKB) and counts in [0, nKB]. The kernel clamps counts
 * and entries to those ranges and never reads K/V outside [0, N); other bad entries give
 * unspecified values.
 * The remaining arguments are those of sparse_attn_fwd.
 */
int sparse_attn_fwd_lists(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                          const int32_t* kept_cnt, int B, int H, int N, int d, int Bq, int Bk, double scale,
                          void* o, float* lse, void* stream);

/*
 * Work order of the attention rows for sparse_attn_fwd_lists_ordered: which row (b, h, query
 * block) each workgroup computes. Scheduling only; it changes no result.
 *   kept_cnt   device, [B, H, nqb] int32 (as sparse_attn_select_mask writes it).
 *   order      device out, [B * H * nqb] int32, a permutation of the rows.
 * Workgroups reach the chip's eight XCDs round-robin. With B * H * nqb >= 8192 (at least 16
 * rounds of the 512 workgroups that run at once) the order is the default one of the kernels,
 * which keeps neighbouring rows of a head in one XCD's L2; below that each XCD takes its rows
 * longest list first (ties in the default order), which shortens the last round.
 * Errors: SA_ERR_INVALID_ARG for null pointers or non-positive sizes.
 */
int sparse_attn_row_order(const int32_t* kept_cnt, int B, int H, int nqb, int32_t* order, void* stream);

/*
 * sparse_attn_fwd_lists with workgroup w computing row row_order[w] (from sparse_attn_row_order;
 * entries are clamped to the row range, and an order that is not a permutation leaves rows
 * uncomputed or computed twice). Results equal those of sparse_attn_fwd_lists bit for bit.
 * With SA_BF16, d = 128 and Bq = 64 (up to 4096 key blocks per head) the rows run in pairs of
 * neighbouring 64-query blocks and row_order is not used.
 */
int sparse_attn_fwd_lists_ordered(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                                  const int32_t* kept_cnt, const int32_t* row_order, int B, int H, int N, int d,
                                  int Bq, int Bk, double scale, void* o, float* lse, void* stream);

/*
 * sparse_attn_fwd_lists over the window-transposed token order without materialising it: the
 * attention's rows (queries and keys alike) are those of sparse_attn_window_transpose's forward
 * order, row s being token (s mod nw) * window + s / nw with nw = N / window, while q, k, v, o
 * and lse stay in the original token order. kept_idx / kept_cnt index blocks of the transposed
 * order. This is the SQuad global pass ([SQ] "手法") as a local pass over runs of nw, with the
 * permutation equivalence of [SVG2] "2. 手法" A; results equal transposing Q, K, V, calling
 * sparse_attn_fwd_lists and transposing O and LSE back.
 *   dtype must be SA_BF16 and Bk 64; window must divide N, and N / window must be at least 64
 *   (a key block then spans at most two runs); one head's rows (N * d * 2 bytes) must stay below
 *   4 GiB. Other arguments as sparse_attn_fwd_lists.
 */
int sparse_attn_fwd_lists_window(const void* q, const void* k, const void* v, int dtype, const int32_t* kept_idx,
                                 const int32_t* kept_cnt, int B, int H, int N, int d, int Bq, int Bk, int window,
                                 double scale, void* o, float* lse, void* stream);

/* Bytes of device workspace sparse_attn_bwd needs (row and column kept lists with counts, the
 * transposed mask, and two floats per query of the nQB * Bq padded rows: D and the LSE in log2
 * units; each part 256-byte aligned). 0 for invalid shapes. */
size_t sparse_attn_bwd_workspace_size(int B, int H, int N, int Bq, int Bk);

/*
 * Gradients of sparse_attn_fwd for the same mask (the sparse student of [SA2]
 * "ハイブリッドマスキングと蒸留微調整" is fine-tuned by distillation). With s = scale * Q K^T over the
 * kept keys, P = exp(s - LSE) and D = rowsum(dO * O):
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
 *   q, k, v, o, dout  device, [B, H, N, d] SA_BF16 (o is the forward's output, dout the
 *                     upstream gradient); `dtype` must be SA_BF16.
 *   lse         device, [B, H, N] float32, the LSE the forward wrote for this mask.
 *   mask        device, [B, H, nQB, nKB] uint8, the forward's mask.
 *   dq, dk, dv  device out, [B, H, N, d] bf16 (fp32 accumulation). Queries of a block with no
 *               kept key get dQ = 0; keys of a block no query block keeps get dK = dV = 0.
 *   workspace   device scratch of at least sparse_attn_bwd_workspace_size() bytes, 256-byte
 *               aligned; overwritten.
 * Each output element is written by one workgroup in a fixed order (no atomics): repeated calls
 * give identical bits. d in {64, 128}, Bq in {64, 128}, Bk = 64.
 */
int sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    int dtype, const uint8_t* mask, int B, int H, int N, int d, int Bq, int Bk, double scale, void* dq,
                    void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fixed block patterns, as masks for sparse_attn_fwd (SQuad page "SQuad: Sub-Quadratic Attention
 * Distillation for Efficient Video Generation" (gist.science), section "手法": local pass inside
 * windows of w tokens, global pass among the tokens at the same position inside their window;
 * Sparse-vDiT page "Sparse-vDiT: Unleashing the Power of Sparse Attention to Accelerate Video
 * Diffusion Transformers" (aibr.jp), section "3. 中核となる技術的要素": diagonal, multi-diagonal
 * and vertical-stripe patterns). Token-level rules, t a query token and u a key token:
 *   SA_PAT_LOCAL      floor(t / window) == floor(u / window)
 *   SA_PAT_GLOBAL     t mod window == u mod window
 *   SA_PAT_DIAG       |t - u| <= band
 *   SA_PAT_MULTIDIAG  |t - u - m * period| <= band for some integer m
 *   SA_PAT_STRIPE     u mod period == 0
 * `patterns` is an OR of these; a block pair is kept when any (query token, key token) pair of
 * the two blocks satisfies any selected rule (the block cover of the token pattern).
 */
#define SA_PAT_LOCAL 1
#define SA_PAT_GLOBAL 2
#define SA_PAT_DIAG 4
#define SA_PAT_MULTIDIAG 8
#define SA_PAT_STRIPE 16

/*
 *   window, band, period   parameters of the selected rules (window > 0 for LOCAL / GLOBAL,
 *                          band >= 0 for DIAG / MULTIDIAG, period > 0 for MULTIDIAG / STRIPE;
 *                          ignored otherwise).
 *   mask        device out, [B, H, nQB, nKB] uint8 (the same pattern for every b, h).
 *   kept_idx    device out or NULL, [B, H, nQB, nKB] int32, ascending kept indices per row.
 *   kept_cnt    device out or NULL (both or neither), [B, H, nQB] int32.
 * Bq, Bk in {64, 128}; nKB <= SA_MAX_NKB.
 */
int sparse_attn_pattern_mask(int patterns, int window, int band, int period, int B, int H, int N, int Bq, int Bk,
                             uint8_t* mask, int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/*
 * Window transpose of the token axis, the permutation that turns the SQuad global pass into a
 * local pass ([SQuad] "手法") and leaves attention unchanged once the output is permuted back
 * ([SVG2] "2. 手法" A: permutation equivalence). With nw = N / window:
 *   forward (inverse = 0):  out[b, h, s, :] = x[b, h, (s mod nw) * window + s / nw, :]
 *   inverse (inverse != 0): out[b, h, t, :] = x[b, h, (t mod window) * nw + t / window, :]
 * so the tokens at one position inside their window form contiguous runs of nw.
 *   x, out   device, [B, H, N, d] of `dtype`, 16-byte aligned, not aliased.
 * window must divide N.
 */
int sparse_attn_window_transpose(const void* x, int dtype, int B, int H, int N, int d, int window, int inverse,
                                 void* out, void* stream);

/*
 * One pass of the SQuad attention operator, token-exact ([SQuad] "手法", "1. SQuad アテンション・
 * オペレーター"): every token attends, with a standard softmax, to exactly the key tokens its
 * rule admits (t a query token, u a key token, w = window):
 *   pass = SA_SQUAD_LOCAL   floor(t / w) == floor(u / w): the window of w consecutive tokens
 *                           (the last window is cut at N when w does not divide N);
 *   pass = SA_SQUAD_GLOBAL  t mod w == u mod w: the tokens at the same position inside their
 *                           windows, across all windows.
 * The operator is the local pass of (Q, K, V) followed by the global pass of (Q, K, O_local):
 * the caller passes the local output as `v` of the global pass. No mask or list is read: a
 * query block walks the key blocks that cover its rows' windows (the global pass in the
 * window-transposed order of sparse_attn_window_transpose, read in place) and masks every key
 * outside a query's own window or position class element by element.
 *   q, k, v     device, [B, H, N, d] SA_BF16, 16-byte aligned.
 *   o           device out, [B, H, N, d] SA_BF16 (must not alias q, k or v).
 *   lse         device out or NULL, [B, H, N] float: natural-log softmax denominators.
 * Arithmetic as sparse_attn_fwd. Bq in {64, 128}, d in {64, 128}, 1 <= window <= N. The global
 * pass needs window | N and N / window >= 64 (SA_ERR_UNSUPPORTED otherwise: transpose with
 * sparse_attn_window_transpose and run the local pass with window N / window instead), and one
 * head's rows (N * d * 2 bytes) below 4 GiB.
 */
#define SA_SQUAD_LOCAL 0
#define SA_SQUAD_GLOBAL 1
int sparse_attn_squad_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d, int Bq,
                          int window, int pass, double scale, void* o, float* lse, void* stream);

/*
 * Bytes of device scratch sparse_attn_probe_correct needs (0 if the sizes are invalid).
 */
size_t sparse_attn_probe_workspace_size(int B, int H, int N, int d, int Bq, int probes);

/*
 * Probe-fitted residual correction of a sparse output, in place ([SPR] original abstract: a few
 * exact query rows calibrate an affine correction from the sparse output, within the output
 * subspace of the probe residuals). Per (b, h):
 *   probes    `probes` query blocks i_p = min(F - 1, floor((p + 1/2) F / probes)), p = 0..probes-1,
 *             F = the number of full query blocks (nQB, or nQB - 1 when N % Bq != 0; at least 1);
 *   exact     dense softmax attention of the probe rows over all N keys (bf16 operands, fp32
 *             accumulation, P rounded to bf16 for the PV product, as in the forward);
 *   fit       X = [O, 1] and R = O_exact - O on the probe rows inside the sequence (duplicated
 *             probes count once per occurrence); A = (X^T X + mu I)^-1 X^T R in float64 by
 *             Cholesky, mu = ridge * trace(X^T X) / (d + 1);
 *   subspace  with rank < d, A <- A V_r V_r^T, V_r the eigenvectors of R^T R for its `rank` largest
 *             eigenvalues (the principal directions of the probe residuals; cyclic Jacobi in
 *             fp32 on R^T R formed in float64), so that every correction row lies in their span;
 *   apply     O <- O + O A[0:d] + A[d] on every row (bf16 MFMA with A rounded to bf16, fp32
 *             accumulation and add, result rounded to bf16).
 *   q, k, v     device, [B, H, N, d] SA_BF16 (`dtype` must be SA_BF16).
 *   o           device in/out, [B, H, N, d] bf16: the sparse output (e.g. of sparse_attn_fwd), replaced
 *               by the corrected output.
 *   probes      1 .. 1024; ridge > 0 (then X^T X + mu I is positive definite); rank >= 1 (rank >= d:
 *               no projection).
 *   a_out       device out or NULL, [B, H, d + 1, d] float32: A.
 *   exact_out   device out or NULL, [B, H, probes * Bq, d] float32: the exact probe rows in probe
 *               order (rows past N, possible only when the sequence has no full block, are
 *               unspecified).
 *   workspace   device scratch of at least sparse_attn_probe_workspace_size() bytes, 256-byte
 *               aligned; overwritten.
 * d in {64, 128}, Bq in {64, 128}; key blocks of 64. Deterministic (no atomics).
 */
int sparse_attn_probe_correct(const void* q, const void* k, const void* v, void* o, int dtype, int B, int H, int N,
                              int d, int Bq, double scale, int probes, double ridge, int rank, float* a_out,
                              float* exact_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Semantic-aware permutation ([SVG2] "2. 手法" A, B, C): tokens are grouped by k-means on Q and on
 * K, permuted so that every cluster is contiguous, clusters of keys are chosen per query cluster
 * by a Top-p over centroid scores, and attention runs over the variable-size blocks that the
 * clusters form. Permuting the output back gives attention in the original order.
 */

/* Bytes of device scratch sparse_attn_kmeans needs (0 if the sizes are invalid). */
size_t sparse_attn_kmeans_workspace_size(int B, int H, int N, int d, int C);

/*
 * Lloyd's k-means of the N token rows of x, per (b, h), into C clusters.
 *   x          device, [B, H, N, d] SA_BF16.
 *   init       device or NULL, [B, H, C, d] float32 starting centroids (a warm start); NULL starts
 *              centroid c at token floor((2c + 1) N / (2C)).
 *   iters      >= 1 iterations of: assign every token to the centroid with the smallest
 *              |mu|^2 - 2 <x, mu> (the order of |x - mu|^2; the lowest index on a tie; the
 *              products use the bf16 token and the centroid split into two bf16 parts, summed
 *              in fp32), then move every centroid to the float64 mean of its tokens (an empty
 *              cluster keeps its centroid).
 *   centroids  device out, [B, H, C, d] float32: after the last update.
 *   labels     device out, [B, H, N] int32: the last assignment.
 *   perm       device out, [B, H, N] int32: the stable sort of tokens by label; perm[t'] is the
 *              token at permuted position t'.
 *   offsets    device out, [B, H, C + 1] int32: cluster c occupies [offsets[c], offsets[c + 1]).
 *   workspace  device scratch of at least sparse_attn_kmeans_workspace_size() bytes, 256-byte
 *              aligned; overwritten.
 * d in {64, 128}, 1 <= C <= min(N, SA_MAX_CLUSTERS). Deterministic.
 */
int sparse_attn_kmeans(const void* x, int dtype, int B, int H, int N, int d, int C, int iters, const float* init,
                       float* centroids, int32_t* labels, int32_t* perm, int32_t* offsets, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Centroid Top-p ([SVG2] "2. 手法" B). For query cluster i the estimated attention mass of key
 * cluster j is n_j exp(S_ij) normalised over j, with S_ij = scale <cq_i, ck_j> (float64) and n_j
 * the cluster's size (empty clusters have none). Clusters are taken in descending mass (the lower
 * index first on equality) until the sequential running sum reaches p; at least one and never an
 * empty cluster is taken.
 *   cq, ck      device, [B, H, Cq, d] and [B, H, Ck, d] float32 centroids.
 *   k_offsets   device, [B, H, Ck + 1] int32: the key clusters' offsets (their sizes).
 *   probs       device out or NULL, [B, H, Cq, Ck] float64 masses.
 *   mask        device out, [B, H, Cq, Ck] uint8, 1 = keep.
 * d in {64, 128}; Cq, Ck <= SA_MAX_CLUSTERS; 0 <= p <= 1.
 */
int sparse_attn_cluster_select(const float* cq, const float* ck, const int32_t* k_offsets, int B, int H, int Cq, int Ck,
                               int d, double scale, double p, double* probs, uint8_t* mask, void* stream);

/*
 * Row permutation: out[b, h, t', :] = x[b, h, perm[t'], :] (inverse = 0), or
 * out[b, h, perm[t'], :] = x[b, h, t', :] (inverse != 0).
 *   x, out   device, [B, H, N, d] of `dtype`, 16-byte aligned, not aliased.
 *   perm     device, [B, H, N] int32, a permutation of 0..N-1 per (b, h) (not checked).
 */
int sparse_attn_permute_rows(const void* x, int dtype, int B, int H, int N, int d, const int32_t* perm, int inverse,
                             void* out, void* stream);

/* Bytes of device scratch sparse_attn_cluster_fwd needs (0 if the sizes are invalid). */
size_t sparse_attn_cluster_fwd_workspace_size(int B, int H, int N, int Cq, int Ck, int Bq);

/*
 * Attention over variable-size blocks ([SVG2] "2. 手法" C), in the permuted order: every query of
 * query cluster i (rows [q_offsets[i], q_offsets[i + 1])) attends to exactly the keys of the key
 * clusters j with mask[i][j] = 1 (rows [k_offsets[j], k_offsets[j + 1])). Arithmetic as in
 * sparse_attn_fwd; a query cluster with no kept key gets O = 0 and LSE = -inf. Queries run in
 * tiles of Bq rows inside each cluster; the kept keys are gathered into 64-row tiles across
 * cluster boundaries, so only the last key tile of a query cluster is partial.
 *   q, k, v     device, [B, H, N, d] SA_BF16: q in the query-permuted order (queries by the query
 *               clusters) and k, v in the key-permuted order (keys by the key clusters), or each
 *               in the original token order when its permutation is given.
 *   q_offsets   device, [B, H, Cq + 1] int32; k_offsets device, [B, H, Ck + 1] int32 (ascending,
 *               from 0 to N; not checked).
 *   mask        device, [B, H, Cq, Ck] uint8.
 *   q_perm      device or NULL, [B, H, N] int32: the query permutation (position t' of the
 *               permuted order holds token q_perm[t'], as sparse_attn_kmeans returns it). When
 *               given, q is read and o / lse are written in the original token order through it,
 *               which replaces permuting Q before the call and O after it. Entries are clamped
 *               to [0, N); a q_perm that is not a permutation leaves rows of o unwritten.
 *   k_perm      device or NULL, [B, H, N] int32: the key permutation. When given, k and v are
 *               in the original token order and each key row of the stream is fetched through it
 *               (replacing permuting K and V before the call). Entries are clamped to [0, N).
 *   o           device out, [B, H, N, d] bf16 in the permuted query order (original order with
 *               q_perm); lse device out or NULL, [B, H, N] float32, same order.
 *   workspace   device scratch of at least sparse_attn_cluster_fwd_workspace_size() bytes,
 *               256-byte aligned; overwritten.
 * d in {64, 128}, Bq in {64, 128}, 1 <= Cq, Ck <= min(N, SA_MAX_CLUSTERS); one head's rows
 * (N * d * 2 bytes) must stay below 4 GiB (SA_ERR_UNSUPPORTED otherwise).
 */
int sparse_attn_cluster_fwd(const void* q, const void* k, const void* v, int dtype, int B, int H, int N, int d,
                            const int32_t* q_offsets, int Cq, const int32_t* k_offsets, int Ck, const uint8_t* mask,
                            const int32_t* q_perm, const int32_t* k_perm, int Bq, double scale, void* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Host helper: the Top-k size for a fraction, as select_mask computes it (-1 if invalid). */
int sparse_attn_topk_count(double k_frac, int nkb);

/* Static text for a return code. */
const char* sparse_attn_error_string(int code);

/* Message of the last failed call on the calling thread ("" if none). */
const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
