// Internal (C++) interface between the C-ABI / orchestration layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gns.h"

namespace gns {

// Parameters of one batched GEMM launch (see gemm_kernel.h).
//   symmetric (NT, lower tiles):  D = alpha' A B^T + beta C + gamma I, A,B: M x K
//   rectangular (NN):             D = alpha' A B + beta C,            A: M x K, B: K x N
// alpha' = alpha * scale[b]^alpha_pow.  NN with B of another 16-bit type converts
// B on load after multiplying by b_mul * scale[b]^b_pow.
struct GemmParams {
  int M = 0, N = 0, K = 0;
  const void* A = nullptr; long long lda = 0, sA = 0;
  const void* B = nullptr; long long ldb = 0, sB = 0;
  const void* C = nullptr; long long ldc = 0, sC = 0;
  void* D = nullptr; long long ldd = 0, sD = 0;
  float alpha = 1.f, beta = 0.f, gamma = 0.f;
  const float* scale = nullptr; int alpha_pow = 0;
  float b_mul = 1.f; int b_pow = 0;
  // pair (symmetric only): one launch also computes D' = alpha' A' B^T + beta C' for
  // the same B, shapes and coefficients; workgroups of batch index >= batch take
  // (A2, C2, Dp) at the same strides.
  int pair = 0;
  const void* A2 = nullptr; const void* C2 = nullptr; void* Dp = nullptr;
  // partials (symmetric only, instead of scale): scale[b] = 1 / (sqrt(sum of the
  // n_partials sums of squares of batch entry b) + eps), formed in every workgroup
  // in one fixed order; tile 0 of entry b also stores it to s_out[b].
  const float* partials = nullptr; int n_partials = 0; float eps = 0.f; float* s_out = nullptr;
  // K split (symmetric, 16-bit operands): with ksplit > 1 and reduce == 0 each output
  // tile is computed as ksplit partial products over K ranges of kchunk values whose
  // raw fp32 accumulators go to part; reduce == 1 then sums them in range order and
  // runs the epilogue.
  int ksplit = 1, kchunk = 0, reduce = 0;
  float* part = nullptr;
  // hi/lo planes (16-bit kernel only): a matrix held in 2 planes stores hi = round(v)
  // at its address and lo = round(v - hi) `plane` elements further, so hi + lo keeps
  // about twice the significant bits of one 16-bit value.  A product of two such
  // matrices is hi.hi + hi.lo + lo.hi (lo.lo is below the rounding of the others),
  // run as one K loop over the plane pairs in that order; a 2-plane C is read as
  // hi + lo, and a 2-plane output writes both planes.  a2/c2/dp: the second product
  // of a pair.
  int a_planes = 1, a2_planes = 1, b_planes = 1, c_planes = 1, c2_planes = 1, d_planes = 1, dp_planes = 1;
  long long plane = 0;
  // indexed rows (16-bit kernel only): the X operand is read straight from a larger
  // source matrix -- the A and B operands of a symmetric product (the Gram product
  // X X^T, A == B), the B operand of a rectangular one.  Row r of batch entry b is
  // source row rows[b * rows_stride + r]; rows r >= rows_valid, and indices outside
  // [0, src_rows), read as zeros.  The source is addressed through A (B) with lda
  // (ldb) and the batch stride sA (sB) as usual.
  const int* rows = nullptr; int rows_valid = 0; long long rows_stride = 0; int src_rows = 0;
  int tiles_m = 0, tiles_n = 0;   // set by the launcher
  int batch = 0, tiles = 0;       // set by the launcher: grid = batch * tiles workgroups
};

// flops (nullable): incremented by the MFMA flops the launch issues.
hipError_t launch_symm(gns_dtype in, gns_dtype out, const GemmParams& p, int batch,
                       hipStream_t stream, double* flops);
hipError_t launch_rect(gns_dtype a, gns_dtype b, gns_dtype out, const GemmParams& p, int batch,
                       hipStream_t stream, double* flops);
// The symmetric product with K split over several workgroups per output tile when the
// problem is one long-K matrix with too few tiles to fill the GPU (two launches: the
// partial products, then their ordered sum and the epilogue), else launch_symm.
// part: fp32 scratch of at least symm_split_bytes(batch, n, K) bytes (nullable: no split).
hipError_t launch_symm_ws(gns_dtype in, gns_dtype out, const GemmParams& p, int batch, float* part,
                          size_t part_bytes, hipStream_t stream, double* flops);
size_t symm_split_bytes(int batch, int n, int K, gns_dtype in);
bool rect_pair_supported(gns_dtype a, gns_dtype b);

// Frobenius scale: partial sums of squares, then s[b] = 1 / (sqrt(sum) + eps).
int frob_partials_per_batch(int n, int m);
// at most this many partial sums per batch entry feed a Gram product's Frobenius scale
constexpr int kMaxPartials = 1024;
// s_out[b] = 1 / (sqrt(sum of the P partials of entry b) + eps)
hipError_t launch_frob_finish(const float* partials, int P, int batch, float eps, float* s_out, hipStream_t stream);
hipError_t launch_frob(const void* X, gns_dtype dt, long long ldx, long long stride_x, int batch,
                       int n, int m, float eps, float* s_out, float* partials, hipStream_t stream);
// ... only the partial sums (frob_partials_per_batch of them per batch entry), for a
// GEMM that forms the scale itself (GemmParams::partials).
hipError_t launch_frob_partials(const void* X, gns_dtype dt, long long ldx, long long stride_x, int batch,
                                int n, int m, float* partials, hipStream_t stream);
// Y = cast(mul * scale[b]^pow * X) elementwise, for batch x n x m matrices.
hipError_t launch_cast_scale(const void* X, gns_dtype xdt, long long ldx, long long sx, void* Y,
                             gns_dtype ydt, long long ldy, long long sy, int batch, int n, int m,
                             float mul, const float* scale, int pow, hipStream_t stream);

// part[t][0][:] = sum over r = 0 .. ranges-1 of part[t][r][:] (in that order) for each
// of `tiles` tiles of `ranges` blocks of `block_floats` floats (a multiple of 4).
hipError_t launch_sum_ranges(float* part, long long tiles, int ranges, long long block_floats, hipStream_t stream);

// Y[b] = X[b]^T for batch x rows x cols matrices (rows, cols, ldx, ldy multiples of 8
// for 16-bit types, of 4 for fp32).
hipError_t launch_transpose(const void* X, gns_dtype dt, long long ldx, long long sx, int batch, int rows, int cols,
                            void* Y, long long ldy, long long sy, hipStream_t stream);

// Dion3 element-wise kernels (dion3.hip), over `batch` same-shape N x m matrices whose
// entries are `stride` elements apart; per-entry vectors (score, sumsq: N; S: k;
// X, O: k rows; s: 1) are packed back to back.  The state (W, M, G, and X, which
// holds rows of M) has the element type dt: bf16, f16 or fp32.
hipError_t launch_accumulate_score(void* M, const void* G, gns_dtype dt, int batch, int N, int m, long long ld,
                                   long long stride, int score_norm, double* score, double* sumsq, hipStream_t s);
hipError_t launch_topk(const double* score, int batch, int N, int k, int* S, hipStream_t s);
// dev_scalars (nullable): device float[3] = {lr, wd, mu} read when the kernel runs,
// replacing the host values.
// X holds kx >= k rows per batch entry (rows k .. kx-1 are written as zeros).  Xh
// (bf16 state only, nullable): also written, the fp16 copy fl16(fl32(hP hs[b]) x) of
// the same rows with X's row stride.
hipError_t launch_gather_feedback(void* M, gns_dtype dt, int batch, int N, int m, long long ld, long long stride,
                                  const int* S, int k, int kx, float mu, const float* dev_scalars, void* X,
                                  long long ldx, hipStream_t s, void* Xh = nullptr, const float* hs = nullptr,
                                  float hP = 1.0f);
// O: k rows (row stride ldo, element type o_dtype) per batch entry, entries so
// elements apart.  Mfb (nullable): also apply the error feedback M[S] <- fl(mu M[S]) to
// the same rows (M with W's row stride, batch stride and element type).
hipError_t launch_apply_update(void* W, gns_dtype dt, int batch, int N, int m, long long ld, long long stride,
                               const int* S, int k, const void* O, gns_dtype o_dtype, long long ldo, long long so,
                               float lr, float wd, const float* dev_scalars, hipStream_t s, void* Mfb = nullptr,
                               float mu = 0.0f);
// Largest row count of an indexed rectangular product (its row table sits in LDS).
constexpr int kMaxIndexedRows = 8192;
// s[b] = 1 / (sqrt(sum_i sumsq[b][S[b][i]]) + eps): the Frobenius scale of the rows S.
hipError_t launch_selected_sumsq(const double* sumsq, const int* S, int batch, int k, int N, float eps,
                                 float* s_out, hipStream_t s);

// Column selection (dion3.hip): the state is N x m row-major; S holds column indices.
// Partial column sums: dion3_cols_partials(N) blocks of m doubles each, for the score
// and for the sum of squares.
size_t dion3_cols_partials(int N);
hipError_t launch_accumulate_colscore(void* M, const void* G, gns_dtype dt, int N, int m, long long ld,
                                      int score_norm, double* part_s, double* part_q, double* score, double* sumsq,
                                      hipStream_t s);
// Xt (kx x N, row stride ldx, type dt): row j < k = column S[j] of M, rows k .. kx-1
// zero; then M[:, S] <- fl(mu M[:, S])
hipError_t launch_gather_cols_feedback(void* M, gns_dtype dt, int N, int m, long long ld, const int* S, int k, int kx,
                                       float mu, void* Xt, long long ldx, hipStream_t s);
// W[:, S[j]] <- fl(d W - lr O[j, :]^T) (O: type dt); with wd != 0 every other column
// decays (mark: m bytes of scratch)
hipError_t launch_update_cols(void* W, gns_dtype dt, int N, int m, long long ld, const int* S, int k, const void* O,
                              long long ldo, float lr, float wd, uint8_t* mark, hipStream_t s);

}  // namespace gns
