/*
 * gns.h - C ABI of the MI355X (gfx950) Gram Newton-Schulz / Dion3 library (libgns.so).
 *
 * What the library computes (sources are the pages on the Dion3 method):
 *   - Muon's orthogonalisation step, computed by Gram Newton-Schulz: normalise X by
 *     its Frobenius norm, form the Gram matrix R = X X^T, run T quintic steps on the
 *     small n x n iterates with a restart, apply the result once as Q X.
 *     ["Dion3: Full-Stack Orthogonal Updates", paper.rainbus.top summary, sections
 *      核心方法 (theorem 2) and 方法步骤详情 (Algorithm 3)]
 *   - standard quintic Newton-Schulz on the same kernels (the baseline).
 *     ["Muon: Orthogonalized Momentum and Why It Trains LLMs 2x Cheaper", section
 *      "Doing an SVD without an SVD"]
 *   - symmetric-output GEMM alpha A B^T + beta C (+ gamma I), lower tiles only,
 *     mirrored.  [paper.rainbus.top, 前置知识 "对称 GEMM 内核" and 方法步骤详情 (2)]
 *   - one Dion3 step: accumulate, row scores, top-k rows, Gram NS on the submatrix,
 *     decoupled weight decay + row update, error feedback.
 *     [paper.rainbus.top, 方法步骤详情 (3), Algorithm 4; 前置知识 error feedback]
 *
 * Conventions (all entry points):
 *   - Pointers named X, O, A, B, C, D, W, M, G, S, score, sumsq, workspace, s_out are
 *     DEVICE pointers; gns_schedule and issued_flops are HOST pointers.
 *   - Matrices are row-major.  "ld" is the row stride in elements, "stride" the batch
 *     stride in elements.  Rows must start 16-byte aligned: ld, stride, and the
 *     matrix dimensions n and m must be multiples of 8 (16-bit types) or 4 (fp32),
 *     and device pointers 16-byte aligned (the Dion3 row count k may be any value); each operand matrix must span less than
 *     2 GiB (the kernels address it with 32-bit offsets); otherwise
 *     GNS_ERR_UNSUPPORTED (GNS_ERR_HIP from symm_gemm / rect_gemm).
 *   - The caller owns every buffer, including the workspace.  The library allocates
 *     nothing and keeps no state between calls (apart from the per-thread text of
 *     gns_last_error); every call is asynchronous on
 *     `stream` (no host synchronisation), so results are ready when the stream is.
 *   - Arguments are checked before any launch; a failed check returns a negative
 *     gns_status and launches nothing.  A launch failure returns GNS_ERR_HIP.
 *   - Outputs must not alias inputs unless stated (dion3 updates W and M in place).
 */
#ifndef GNS_H
#define GNS_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GNS_OK = 0,
  GNS_ERR_INVALID_ARG = -1,   /* null pointer, bad shape (k > N, k < 1, ld < m), bad enum */
  GNS_ERR_UNSUPPORTED = -2,   /* alignment / dtype combination not supported */
  GNS_ERR_WORKSPACE = -3,     /* workspace null or smaller than the *_workspace_size query */
  GNS_ERR_HIP = -4            /* a HIP launch or runtime call failed */
} gns_status;

typedef enum { GNS_BF16 = 0, GNS_F32 = 1, GNS_F16 = 2 } gns_dtype;

#define GNS_MAX_STEPS 16

/* Iteration schedule.  a/b/c: per-step coefficients of p_t(x) = a x + b x^3 + c x^5.
 * restart_after_mask: bit s (1 <= s < steps) set = restart after step s (recompute
 * X <- Q X, R = X X^T, Q = I).  eps: added to the Frobenius norm.
 * square_fallback: when 1 and n == m, gns_orthogonalize_batched runs standard NS
 * (the Gram form saves nothing at aspect ratio 1; the Dion3 page's limitations
 * section says to fall back to kernelized standard NS there).
 * rows_in_place (Dion3 row steps only): 1 = the Gram products read the selected rows
 * straight from M through the row list, so the submatrix M[S, :] is never copied (the
 * error feedback then runs with the weight update); 0 (default) = the rows are first
 * gathered into a contiguous copy.  Both give bitwise the same results.  Measured on
 * MI355X at f = 1/4 on the 8192 x 28672 state, the copy is faster (1.56 against
 * 1.61 ms): written just before the products read it, it sits in the 256 MB Infinity
 * Cache, while the rows in place come from HBM.  The in-place path applies to a bf16
 * state whose submatrix is wide (k <= m, Gram path) with k <= 8192; otherwise the rows
 * are copied.
 * Gram Newton-Schulz: paper.rainbus.top 方法步骤详情 Algorithm 3 (restart at t = 3). */
typedef struct {
  int steps;
  float a[GNS_MAX_STEPS];
  float b[GNS_MAX_STEPS];
  float c[GNS_MAX_STEPS];
  unsigned restart_after_mask;
  float eps;
  int square_fallback;
  int rows_in_place;
} gns_schedule;

/* Fills: 5 steps of (3.4445, -4.7750, 2.0315), restart after step 2, eps 1e-7,
 * square_fallback 1, rows_in_place 0.  [Muon blog, "Doing an SVD without an SVD"; Algorithm 3] */
void gns_default_schedule(gns_schedule* sched);

/* Human-readable name of a gns_status value (static string). */
const char* gns_status_string(int status);

/* Description of the last HIP failure (GNS_ERR_HIP) seen by the calling thread: the
 * failing call and HIP's error name.  Empty if none.  This per-thread text is the
 * library's only state; it never affects results. */
const char* gns_last_error(void);

/* s[b] = 1 / (||X_b||_F + eps) for each of `batch` n x m matrices, fp32 accumulation.
 * X: bf16/f16/f32 [batch][n][ldx] (batch stride stride_x).  s_out: device float[batch].
 * workspace: >= gns_frobenius_workspace_size(batch, n, m) bytes.
 * [Muon blog, "Doing an SVD without an SVD": X / (norm + 1e-7)] */
size_t gns_frobenius_workspace_size(int batch, int n, int m);
int gns_frobenius_scale(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x,
                        int batch, int n, int m, float eps, float* s_out,
                        void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by gns_orthogonalize_batched / gns_newton_schulz_batched. */
size_t gns_workspace_size(int batch, int n, int m, gns_dtype compute);

/* Gram Newton-Schulz on `batch` same-shape matrices in one pass (one launch per step
 * over the whole batch).  X: [batch][n][ldx], n, m >= 1.  The iteration runs on the
 * short side: for n > m the library transposes X into the workspace, runs on X^T and
 * transposes the result back (polar(X^T) = polar(X)^T) [Muon blog, "Doing an SVD
 * without an SVD"].  O: [batch][n][ldo], dtype o_dtype.
 * compute: dtype of the n x n iterates and of the MFMA operands after the first Gram
 * product: GNS_F16 (the pages' half precision, default), GNS_BF16, or GNS_F32.  All
 * products accumulate in fp32.  With GNS_BF16 the Gram chain (R, Z and the R-update
 * product) is stored as a hi/lo pair of bf16 planes, hi = bf16(v), lo = bf16(v - hi),
 * and each of its products runs on bf16 MFMA as hi.hi + hi.lo + lo.hi: one bf16 R
 * squares the condition number of X at 8 significant bits, which loses the small
 * singular values on small and square inputs.  Q and the restarted X are single bf16
 * matrices.  With x_dtype GNS_F32, compute must be GNS_F32.
 * sched: NULL = gns_default_schedule.  issued_flops (nullable, host): receives the
 * MFMA flops the call issues.  X is read-only; O must not alias X or the workspace.
 * A zero matrix gives a zero result.
 * [paper.rainbus.top 方法步骤详情 Algorithm 3; 核心方法 theorem 2] */
int gns_orthogonalize_batched(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x,
                              void* O, gns_dtype o_dtype, long long ldo, long long stride_o,
                              int batch, int n, int m, gns_dtype compute,
                              const gns_schedule* sched, void* workspace, size_t ws_bytes,
                              hipStream_t stream, double* issued_flops);

/* gns_orthogonalize_batched for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels run on a static device array of GNS_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library instead of a caller's workspace; each GPU holds its own copy
 * from the library's load until the process ends.  The call allocates nothing and
 * calls no allocating routine; on its first call on a device it looks up that
 * device's copy (hipGetSymbolAddress).  Arguments, rules and results are those of
 * gns_orthogonalize_batched (bitwise the same output).  Errors: GNS_ERR_WORKSPACE
 * (nothing launched; gns_last_error() says why) when gns_workspace_size(batch, n, m,
 * compute) exceeds GNS_NOALLOC_SCRATCH_BYTES -- the 1024 x 4096 matrix fits with any
 * iterate dtype; GNS_ERR_INVALID_ARG when `stream` belongs to another device than the
 * current one; otherwise as gns_orthogonalize_batched.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined results, so serialise them.  A call reads no part
 * of the array that it did not write first, so nothing needs clearing between calls. */
#define GNS_NOALLOC_SCRATCH_BYTES (64u << 20)
int gns_orthogonalize_batched_noalloc(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x,
                                      void* O, gns_dtype o_dtype, long long ldo, long long stride_o,
                                      int batch, int n, int m, gns_dtype compute,
                                      const gns_schedule* sched, hipStream_t stream,
                                      double* issued_flops);

/* Standard quintic Newton-Schulz (A = X X^T; B = b A + c A A; X <- a X + B X) on the
 * same kernels; same arguments and rules as gns_orthogonalize_batched (the restart
 * mask and square_fallback are ignored).
 * [Muon blog, "Doing an SVD without an SVD"; paper.rainbus.top 前置知识] */
int gns_newton_schulz_batched(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x,
                              void* O, gns_dtype o_dtype, long long ldo, long long stride_o,
                              int batch, int n, int m, gns_dtype compute,
                              const gns_schedule* sched, void* workspace, size_t ws_bytes,
                              hipStream_t stream, double* issued_flops);

/* Symmetric-output GEMM: D = alpha * A * B^T + beta * C + gamma * I, for `batch`
 * problems.  A, B: n x k (row-major, dtype in_dtype); with B symmetric (k == n) this
 * is A * B, with A == B it is the Gram product A A^T.  Only output tiles on or below
 * the diagonal are computed; each is also written transposed above the diagonal, so
 * D is bitwise symmetric.  C: n x n in out_dtype, read from its lower triangle only
 * (may be NULL when beta == 0; may alias D).  D: n x n in out_dtype.
 * in_dtype: GNS_BF16, GNS_F16 or GNS_F32; out_dtype any.
 * [paper.rainbus.top 前置知识 symmetric GEMM kernel; 方法步骤详情 (2): lower-triangle
 *  tile scheduler + transposed-write epilogue; 技术新颖性: alpha A B + beta C] */
int symm_gemm(int batch, int n, int k, float alpha,
              const void* A, long long lda, long long stride_a,
              const void* B, long long ldb, long long stride_b,
              float beta, const void* C, long long ldc, long long stride_c,
              float gamma, void* D, long long ldd, long long stride_d,
              gns_dtype in_dtype, gns_dtype out_dtype, hipStream_t stream);

/* Rectangular GEMM: D = alpha * A * B + beta * C for `batch` problems.  A: n x k
 * (a_dtype, the MFMA operand type); B: k x m (b_dtype; converted to a_dtype on load,
 * after multiplying by b_prescale); C (nullable when beta == 0), D: n x m in
 * out_dtype.  b_prescale must be 1 when b_dtype == a_dtype.  This is the Q X product
 * of Gram NS and the B X product of standard NS.
 * [paper.rainbus.top 核心方法: the two rectangular products X X^T and Q X] */
int rect_gemm(int batch, int n, int k, int m, float alpha,
              const void* A, long long lda, long long stride_a, gns_dtype a_dtype,
              const void* B, long long ldb, long long stride_b, gns_dtype b_dtype,
              float b_prescale, float beta, const void* C, long long ldc, long long stride_c,
              void* D, long long ldd, long long stride_d, gns_dtype out_dtype,
              hipStream_t stream);

/* ---- Dion3 (row-subsampled update with error feedback) -------------------------
 * W, M, G: N x m row-major with row stride ld, all of the state type dt (GNS_BF16,
 * GNS_F16 or GNS_F32; the caller's optimizer state).  m and ld multiples of 8, the
 * pointers 16-byte aligned (else GNS_ERR_UNSUPPORTED).  S: device int32[k], ascending
 * row indices.  Rounding model: each stored value is rounded once to dt (nearest even);
 * element-wise updates are fp32 op by op, no fused multiply-add; the orthogonalised
 * rows O are stored in dt before the update reads them.  The Gram NS reads the
 * submatrix in dt (bf16, f16), or, for an fp32 state, a copy scaled by its Frobenius
 * scale and rounded once to the iterate type (compute), which it normalises again.
 * [paper.rainbus.top 方法步骤详情 (3) Algorithm 4; 前置知识 error feedback] */

/* M <- fl(M + G); score[i] = sum_j |M_ij| (score_norm 1) or sum_j M_ij^2
 * (score_norm 2) of the updated M, float64 accumulation; sumsq[i] = sum_j M_ij^2
 * (float64; nullable).  score, sumsq: device double[N]. */
int dion3_accumulate_score(void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int score_norm,
                           double* score, double* sumsq, hipStream_t stream);

/* S = indices of the k largest scores (ties -> lower index), written ascending.
 * 1 <= k <= N.  One workgroup; no workspace. */
int dion3_select_topk(const double* score, int N, int k, int* S, hipStream_t stream);

/* X[r, :] = M[S[r], :] (type dt, row stride ldx) and then M[S[r], :] <- fl(mu * M[S[r], :])
 * (error feedback: only selected rows decay).  An index S[r] outside [0, N) gives a
 * zero row X[r, :] and touches no row of M. */
int dion3_gather_feedback(void* M, gns_dtype dt, int N, int m, long long ld, const int* S, int k, float mu,
                          void* X, long long ldx, hipStream_t stream);

/* d = fl32(1 - fl32(lr * wd)); W[S[r], :] <- fl(fl32(d * W) - fl32(lr * O[r, :]));
 * when wd != 0 every other row W <- fl(fl32(d * W)).  W: type dt.  O: k x m of any
 * o_dtype, row stride ldo (a multiple of 8).  S must be ascending and hold distinct
 * indices in [0, N). */
int dion3_apply_update(void* W, gns_dtype dt, int N, int m, long long ld, const int* S, int k,
                       const void* O, gns_dtype o_dtype, long long ldo,
                       float lr, float wd, hipStream_t stream);

/* Workspace bytes needed by dion3_step for a state of type dt (it holds the selected
 * submatrix and its orthogonalisation in dt); 0 for invalid arguments. */
size_t dion3_workspace_size(int N, int m, int k, gns_dtype dt, gns_dtype compute);

/* One Dion3 step (in place on W and M of state type dt):
 *   M <- M + G; S = top-k rows by score (score_norm 1 = l1 as on the pages, 2 = l2);
 *   X = M[S, :]; O = GramNS(X) (sched, compute as in gns_orthogonalize_batched, the
 *   Frobenius norm taken from the per-row sums of squares); W <- decay + row update
 *   with lr (the caller passes lr = eta / sqrt(f)); M[S, :] <- mu M[S, :].
 * S_out: device int32[k] (ascending).  O_out: nullable device [k][m] of type dt (row
 * stride m) receiving O; it must not overlap W, M, G or the workspace.  1 <= k <= N, any k
 * (k = ceil(f N) on the pages): the submatrix is held with k rounded up to a multiple
 * of 8 rows, the extra rows zero, which leaves O's k rows unchanged.  With k > m the
 * k x m submatrix is orthogonalized through its transpose, as in
 * gns_orthogonalize_batched.  Every argument, including those of the
 * Gram NS on the submatrix, is checked before the first launch. */
int dion3_step(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k,
               float lr, float weight_decay, float mu, int score_norm, gns_dtype compute,
               const gns_schedule* sched, int* S_out, void* O_out,
               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by dion3_step_batched (state type dt). */
size_t dion3_batched_workspace_size(int batch, int N, int m, int k, gns_dtype dt, gns_dtype compute);

/* dion3_step on `batch` same-shape N x m states at once (W, M, G: [batch][N][ld], entry
 * b at offset b * stride elements, stride >= N * ld): per entry the same scores, top-k,
 * gather, error feedback and update as dion3_step; the batch's k x m submatrices are
 * orthogonalized by one batched Gram NS (one launch per step for all entries, the
 * single-GPU form of the pages' megabatching of same-shape parameters)
 * [paper.rainbus.top 方法步骤详情 (3) and (4); m.montaan.com summary].
 * S_out: device int32 [batch][k] (each row ascending).  O_out: nullable device
 * [batch][k][m] of type dt.  W, M and G must not overlap.  Each entry's result is bitwise the
 * result of dion3_step on that entry alone: every product's summation order depends
 * on the matrix shape only, never on the batch size (a long-K Gram product that splits
 * K splits the same way in any batch).  Errors as dion3_step. */
int dion3_step_batched(void* W, void* M, const void* G, gns_dtype dt, int batch, int N, int m, long long ld,
                       long long stride, int k, float lr, float weight_decay, float mu,
                       int score_norm, gns_dtype compute, const gns_schedule* sched, int* S_out,
                       void* O_out, void* workspace, size_t ws_bytes, hipStream_t stream);

/* dion3_step on a row set S chosen by the caller instead of the top-k rows: the pages
 * report that rows drawn at random train about as well as the rows of largest norm,
 * and that a set chosen without reading M lets a data-parallel step exchange only
 * M[S, :] [paper.rainbus.top, 局限与改进 and the future-work paragraph after it].  The
 * draw is the caller's.  Otherwise as dion3_step: M <- M + G; X = M[S, :]; O =
 * GramNS(X) (its Frobenius norm from the rows' sums of squares); W <- decay + row
 * update with lr; M[S, :] <- mu M[S, :].
 * S: device int32[k], distinct indices in [0, N), ascending; the library cannot check
 * this without a host synchronisation.  An index outside [0, N) reads as a zero row of
 * X and updates nothing; repeated or unordered indices give unspecified W and M (no
 * out-of-bounds access).  O_out: nullable device [k][m] of type dt.  Workspace:
 * dion3_workspace_size(N, m, k, dt, compute).  1 <= k <= N (any k, as dion3_step); other
 * errors as dion3_step. */
int dion3_step_rows(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, const int* S, int k,
                    float lr, float weight_decay, float mu, gns_dtype compute,
                    const gns_schedule* sched, void* O_out, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/* Workspace bytes needed by dion3_step_cols (state type dt). */
size_t dion3_cols_workspace_size(int N, int m, int k, gns_dtype dt, gns_dtype compute);

/* One Dion3 step that subsamples columns instead of rows (in place on W and M): the
 * pages let f select rows or columns [paper.rainbus.top 核心方法 and 方法步骤详情 (3);
 * m.montaan.com summary].  M <- M + G; S = the k columns of largest score (score_norm
 * as in dion3_step); X = M[:, S] (N x k); O = GramNS(X); W <- decay + update of the
 * columns S; M[:, S] <- mu M[:, S].  For a tall state (N > m) this keeps the
 * orthogonalised submatrix wide: 28672 x 8192 at f = 1/4 gives a 28672 x 2048
 * submatrix, where row selection would give 7168 x 8192.
 * The columns are scored, gathered (into the k x N transpose of the submatrix, with
 * the error feedback applied in place) and updated in the state's own row-major
 * layout.  S_out: device int32[k], ascending column indices.
 * O_out: nullable device [k][N] of type dt: row j is the update of column S[j] (the
 * transpose of the orthogonalised N x k submatrix).  1 <= k <= m (any k, padded as in
 * dion3_step), N a multiple of 8; W, M, G must not overlap; other errors as
 * dion3_step. */
int dion3_step_cols(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k,
                    float lr, float weight_decay, float mu, int score_norm, gns_dtype compute,
                    const gns_schedule* sched, int* S_out, void* O_out,
                    void* workspace, size_t ws_bytes, hipStream_t stream);

/* dion3_step with lr, weight decay and mu read from device memory when the step runs:
 * lr_wd_mu is a device float[3] = {lr, weight_decay, mu}.  A step captured once in a
 * HIP graph then follows a schedule that the caller writes into that buffer between
 * replays, with no new capture [paper.rainbus.top 方法步骤详情 (4): the optimizer step
 * captured in a CUDA graph].  Results are bitwise those of dion3_step with the same
 * values.  The values are not checked (non-finite ones give non-finite W and M).  The
 * update launch covers all N rows, since the host cannot see whether the weight decay
 * is zero; without decay each unselected row returns at once.  lr_wd_mu must be 4-byte
 * aligned (else GNS_ERR_UNSUPPORTED); other arguments and errors as dion3_step. */
int dion3_step_dev_scalars(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k,
                           const float* lr_wd_mu, int score_norm, gns_dtype compute,
                           const gns_schedule* sched, int* S_out, void* O_out,
                           void* workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by muon_step_batched on a state of type dt (0 for invalid
 * arguments). */
size_t muon_workspace_size(int batch, int n, int m, gns_dtype dt, gns_dtype compute, int nesterov);

/* One Muon step on `batch` same-shape n x m matrices ("Muon: Orthogonalized Momentum
 * and Why It Trains LLMs 2x Cheaper", the step listed after "Doing an SVD without an
 * SVD" and the notes on decoupled weight decay and update-scale matching):
 *   M <- mu M + G                     (heavy-ball momentum, in place)
 *   U  = G + mu M  with nesterov = 1  (lookahead on the updated M); U = M with 0
 *   O  = GramNS(U)                    (the schedule and iterate dtype of
 *                                      gns_orthogonalize_batched; a tall U runs on U^T;
 *                                      ||U||_F from row sums of squares formed in
 *                                      the momentum pass: fp64, rounded to fp32
 *                                      partial sums of the Gram product for a
 *                                      16-bit state with n <= 1024)
 *   W <- (1 - lr weight_decay) W - lr scale O   (decoupled decay first, in place)
 * scale == 0 selects 0.2 sqrt(max(n, m)) (fp32), which matches the update's RMS to
 * AdamW's; a negative scale is GNS_ERR_INVALID_ARG.  Dion3 with every row selected is
 * this step without the lookahead.
 * W, M, G: device [batch][n][ld] of the state type dt (GNS_BF16, GNS_F16 or GNS_F32,
 * one type for the three), entry b at offset b * stride elements (stride >= n * ld
 * when batch > 1); they must not overlap.  Each stored value (M, U, O, W) is rounded
 * once to dt from fp32 arithmetic done op by op; an fp32 U reaches the 16-bit iterates
 * through a copy scaled by its Frobenius scale and rounded once to the iterate type.
 * O_out: nullable device [batch][n][m] of type dt (contiguous) that receives O; it must
 * not overlap W, M, G or the workspace.  Workspace: muon_workspace_size(batch, n, m,
 * dt, compute, nesterov) bytes, 16-byte aligned, owned by the caller.  Asynchronous on
 * `stream`; no host synchronisation.
 * Errors (nothing is launched): GNS_ERR_INVALID_ARG for a null matrix, n or m < 1,
 * ld < m, a short stride, overlapping buffers, nesterov not 0 or 1, a negative
 * scale, or a non-finite scalar; GNS_ERR_UNSUPPORTED for n, m, ld or stride not a
 * multiple of 8, a pointer not 16-byte aligned, or compute = GNS_F32; GNS_ERR_WORKSPACE
 * for a short or null workspace; GNS_ERR_HIP for a launch failure (gns_last_error()
 * describes it). */
int muon_step_batched(void* W, void* M, const void* G, gns_dtype dt, int batch, int n, int m, long long ld,
                      long long stride, float lr, float weight_decay, float mu, int nesterov,
                      float scale, gns_dtype compute, const gns_schedule* sched, void* O_out,
                      void* workspace, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GNS_H */
