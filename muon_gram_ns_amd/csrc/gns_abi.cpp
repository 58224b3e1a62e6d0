// C ABI of libgns: argument checks, workspace carving and the launch schedules of
// Gram Newton-Schulz, standard Newton-Schulz and the Dion3 step.
//
// Gram Newton-Schulz ("Dion3: Full-Stack Orthogonal Updates", paper.rainbus.top,
// 核心方法 theorem 2 and 方法步骤详情 Algorithm 3), per matrix, s = 1/(||X||_F + eps):
//   R = s^2 X X^T, Q = I
//   step t:  Z = c_t R R + b_t R
//            Q <- Q Z + a_t Q            (Q = Z + a_t I while Q is the identity)
//            R <- (Z + a_t I) R (Z + a_t I), as Y = R Z + a_t R, R = Z Y + a_t Y
//                                        (skipped when no later step reads R)
//   restart after step s: X <- Q X, R = X X^T, Q = I
//   output Q X
// Every launch covers the whole batch.  The normalised X is never stored: s stays on
// the device and enters the epilogues (R = s^2 X X^T, X2 = s Q X, O = s Q X).
// With fp16 iterates, matrices shaped like X are stored times a power of two
// P ~ sqrt(n m) so their entries sit near 1, well inside fp16's normal range; the
// factor is divided out exactly in the epilogues.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "internal.h"
#include "muon_kernels.h"

using namespace gns;

namespace {

size_t esize(gns_dtype d) { return d == GNS_F32 ? 4 : 2; }
bool valid_dtype(int d) { return d == GNS_BF16 || d == GNS_F16 || d == GNS_F32; }
size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Carver {
  uint8_t* base;
  size_t off;
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

// With bf16 iterates, the Gram chain R, Z, Y is kept as hi/lo pairs of bf16 planes
// (about 16 significant bits) and its products run on bf16 MFMA as hi.hi + hi.lo +
// lo.hi; Q and the restarted X stay single bf16 planes.  A single bf16 R squares the
// condition number of X at 8 significant bits and misses the 2e-2 output bar on
// small and square inputs; fp16 iterates (11 bits) keep one plane.  Every n x n
// buffer of the call then has room for two planes ([batch][2][n][n]), so one batch
// stride serves all of them.
int gram_planes(gns_dtype cdt) { return cdt == GNS_BF16 ? 2 : 1; }

struct NsLayout {
  float* s;
  float* partials;
  float* part;            // fp32 partial products of a K-split Gram product (may be empty)
  size_t part_bytes;
  void *R, *Z, *Y, *Q0, *Q1, *Xa, *Xb;   // Gram NS
  void *A, *Bm, *Sa, *Sb;                // standard NS (overlaps the Gram region)
  size_t bytes;
};

NsLayout ns_layout(void* base, int batch, int n, int m, gns_dtype cdt) {
  Carver c{reinterpret_cast<uint8_t*>(base), 0};
  NsLayout L{};
  const size_t e = esize(cdt);
  const size_t nn = (size_t)n * n * e * batch, nm = (size_t)n * m * e * batch;
  const size_t nn_gram = nn * gram_planes(cdt);      // every n x n Gram NS buffer, all planes
  L.s = (float*)c.take(sizeof(float) * (size_t)batch);
  L.partials = (float*)c.take(sizeof(float) * (size_t)batch * frob_partials_per_batch(n, m));
  // both Gram products of a call (and standard NS's) have K = m
  L.part_bytes = symm_split_bytes(batch, n, m, cdt);
  L.part = L.part_bytes ? (float*)c.take(L.part_bytes) : nullptr;
  const size_t common = c.off;
  L.R = c.take(nn_gram); L.Z = c.take(nn_gram); L.Y = c.take(nn_gram);
  L.Q0 = c.take(nn_gram); L.Q1 = c.take(nn_gram);
  L.Xa = c.take(nm); L.Xb = c.take(nm);
  const size_t gram_end = c.off;
  c.off = common;
  L.A = c.take(nn); L.Bm = c.take(nn); L.Sa = c.take(nm); L.Sb = c.take(nm);
  L.bytes = std::max(gram_end, c.off);
  return L;
}

// A tall call (n > m) runs on the transposes: Xt = X^T and Ot (both [batch][m][n]),
// then the wide call's workspace.  Element sizes: X's is 4 bytes iff the iterates are
// fp32; O may be any dtype, so Ot is sized for 4 bytes.
struct TallLayout {
  void *Xt, *Ot, *inner;
  size_t inner_bytes, bytes;
};

TallLayout tall_layout(void* base, int batch, int n, int m, gns_dtype cdt) {
  Carver c{reinterpret_cast<uint8_t*>(base), 0};
  TallLayout L{};
  const size_t elems = (size_t)batch * n * m;
  L.Xt = c.take(elems * (cdt == GNS_F32 ? 4 : 2));
  L.Ot = c.take(elems * 4);
  L.inner_bytes = ns_layout(nullptr, batch, m, n, cdt).bytes;
  L.inner = c.take(L.inner_bytes);
  L.bytes = c.off;
  return L;
}

size_t ns_workspace_bytes(int batch, int n, int m, gns_dtype cdt) {
  return n > m ? tall_layout(nullptr, batch, n, m, cdt).bytes : ns_layout(nullptr, batch, n, m, cdt).bytes;
}

float pow2_scale(gns_dtype cdt, int n, int m) {
  if (cdt != GNS_F16) return 1.0f;
  const int e = (int)std::lround(0.5 * std::log2((double)n * (double)m));
  return std::ldexp(1.0f, e);
}

struct NsCall {
  const void* X; gns_dtype xdt; long long ldx, sx;
  void* O; gns_dtype odt; long long ldo, so;
  int batch, n, m; gns_dtype cdt;
  gns_schedule sch;
  void* ws; size_t ws_bytes;
  hipStream_t stream;
  double* flops;
  const float* s_given;   // precomputed device scale (Dion3), or null
  // partial sums of squares of each entry already formed on the device (the Muon
  // momentum pass's row sums), [batch][n_partials_given], n_partials_given <=
  // kMaxPartials: they replace the Frobenius pass over X; null when absent
  const float* partials_given; int n_partials_given;
  // X read through a row table (Dion3's selected rows, straight from the state): row r
  // of entry b is source row rows[b * rows_stride + r] of the state at X (rows r >=
  // rows_valid are zero rows); only the Gram path of a wide call reads X this way
  const int* rows;
  int rows_valid, src_rows;
  long long rows_stride;
  // fp16 copy of X already multiplied by P s (Dion3's gather writes it), read by the
  // products that take X as their B operand instead of converting X on load; null
  // when absent
  const void* Xh; long long ldxh, sxh;
};

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int check_schedule(const gns_schedule& s) {
  if (s.steps < 1 || s.steps > GNS_MAX_STEPS) return GNS_ERR_INVALID_ARG;
  const unsigned allowed = ((1u << s.steps) - 1u) & ~1u;    // bits 1..steps-1
  if (s.restart_after_mask & ~allowed) return GNS_ERR_INVALID_ARG;
  if (!(s.eps >= 0.0f) || !std::isfinite(s.eps)) return GNS_ERR_INVALID_ARG;
  if (s.square_fallback != 0 && s.square_fallback != 1) return GNS_ERR_INVALID_ARG;
  if (s.rows_in_place != 0 && s.rows_in_place != 1) return GNS_ERR_INVALID_ARG;
  for (int t = 0; t < s.steps; ++t)
    if (!std::isfinite(s.a[t]) || !std::isfinite(s.b[t]) || !std::isfinite(s.c[t])) return GNS_ERR_INVALID_ARG;
  return GNS_OK;
}

int check_ns(const NsCall& c) {
  if (!valid_dtype(c.xdt) || !valid_dtype(c.odt) || !valid_dtype(c.cdt)) return GNS_ERR_INVALID_ARG;
  if (c.batch < 0 || c.n < 1 || c.m < 1) return GNS_ERR_INVALID_ARG;
  if (!c.X || !c.O) return GNS_ERR_INVALID_ARG;
  if (c.ldx < c.m || c.ldo < c.m) return GNS_ERR_INVALID_ARG;
  if (c.batch > 1 && (c.sx < (long long)c.n * c.ldx || c.so < (long long)c.n * c.ldo)) return GNS_ERR_INVALID_ARG;
  int st = check_schedule(c.sch);
  if (st) return st;
  if ((c.xdt == GNS_F32) != (c.cdt == GNS_F32)) return GNS_ERR_UNSUPPORTED;
  if (c.n % 8 || c.m % 8 || c.ldx % 8 || c.ldo % 8) return GNS_ERR_UNSUPPORTED;
  if (c.batch > 1 && (c.sx % 8 || c.so % 8)) return GNS_ERR_UNSUPPORTED;
  if (!aligned16(c.X) || !aligned16(c.O) || !aligned16(c.ws)) return GNS_ERR_UNSUPPORTED;
  const size_t xb = ((size_t)(c.batch > 0 ? c.batch - 1 : 0) * c.sx + (size_t)(c.n - 1) * c.ldx + c.m) * esize(c.xdt);
  const size_t ob = ((size_t)(c.batch > 0 ? c.batch - 1 : 0) * c.so + (size_t)(c.n - 1) * c.ldo + c.m) * esize(c.odt);
  if (overlaps(c.X, xb, c.O, ob)) return GNS_ERR_INVALID_ARG;
  // every operand matrix is addressed with 32-bit offsets inside the kernels
  if (((size_t)(c.n - 1) * c.ldx + c.m) * esize(c.xdt) >= (size_t(1) << 31) ||
      (size_t)c.n * c.m * 4 >= (size_t(1) << 31))
    return GNS_ERR_UNSUPPORTED;
  const size_t need = ns_workspace_bytes(c.batch, c.n, c.m, c.cdt);
  if (c.batch > 0 && (!c.ws || c.ws_bytes < need)) return GNS_ERR_WORKSPACE;
  if (c.ws && c.batch > 0 && (overlaps(c.ws, need, c.O, ob) || overlaps(c.ws, need, c.X, xb))) return GNS_ERR_INVALID_ARG;
  return GNS_OK;
}

// The only library state: a per-thread description of the last HIP failure, for
// gns_last_error().  It never influences a computation.
thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return GNS_ERR_HIP;
}

#define HIP_OK(expr)                                   \
  do {                                                 \
    const hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, #expr);  \
  } while (0)

// Symmetric product on n x n (or the Gram product with K = m) for the whole batch.
GemmParams symm_params(int n, int K, const void* A, long long lda, long long sA, const void* B, long long ldb,
                       long long sB, void* D, long long ldd, long long sD) {
  GemmParams g;
  g.M = g.N = n;
  g.K = K;
  g.A = A; g.lda = lda; g.sA = sA;
  g.B = B; g.ldb = ldb; g.sB = sB;
  g.D = D; g.ldd = ldd; g.sD = sD;
  return g;
}

int run_standard(const NsCall& c);

int run_gram(const NsCall& c) {
  const NsLayout L = ns_layout(c.ws, c.batch, c.n, c.m, c.cdt);
  const int n = c.n, m = c.m, B = c.batch;
  const long long nn = (long long)n * n, nm = (long long)n * m;
  const int pl = gram_planes(c.cdt);        // planes of R, Z, Y (Q: always one)
  const long long sn = nn * pl;             // batch stride of every n x n buffer
  const float P = pow2_scale(c.cdt, n, m);
  const gns_dtype cdt = c.cdt;
  const float* s = c.s_given ? c.s_given : L.s;
  if (!c.s_given && !c.partials_given)
    HIP_OK(launch_frob_partials(c.X, c.xdt, c.ldx, c.sx, B, n, m, L.partials, c.stream));
  // planes of one symmetric product: A, B, C, D of the chain (R, Z, Y) carry pl planes
  auto chain = [&](GemmParams& g, int a, int b, int cpl, int d) {
    g.plane = nn;
    g.a_planes = a; g.b_planes = b; g.c_planes = cpl; g.d_planes = d;
  };

  // R0 = s^2 X X^T: operands in X's dtype, result in the iterate dtype.  Without a
  // given scale, the product forms s from the partial sums and stores it to L.s.
  // the X operand's row table, when X is read from the Dion3 state directly
  auto x_rows = [&](GemmParams& g) {
    g.rows = c.rows; g.rows_valid = c.rows_valid; g.rows_stride = c.rows_stride; g.src_rows = c.src_rows;
  };
  {
    GemmParams g = symm_params(n, m, c.X, c.ldx, c.sx, c.X, c.ldx, c.sx, L.R, n, sn);
    chain(g, 1, 1, 1, pl);
    if (c.rows) x_rows(g);
    g.alpha_pow = 2;
    if (c.s_given) {
      g.scale = s;
    } else {
      g.partials = c.partials_given ? c.partials_given : L.partials;
      g.n_partials = c.partials_given ? c.n_partials_given : frob_partials_per_batch(n, m);
      g.eps = c.sch.eps; g.s_out = L.s;
    }
    HIP_OK(launch_symm_ws(c.xdt, cdt, g, B, L.part, L.part_bytes, c.stream, c.flops));
  }
  const void* cx = c.X; gns_dtype cxdt = c.xdt; long long cld = c.ldx, csx = c.sx; bool cx_orig = true;
  bool q_identity = true;
  void* Q = L.Q0; void* Qn = L.Q1;
  const unsigned mask = c.sch.restart_after_mask;
  auto restart_before = [&](int t) { return t >= 2 && (mask >> (t - 1)) & 1u; };

  // rect product  out = (alpha) Q cx, with the scaling rules for cx described above
  auto apply_q = [&](void* out, gns_dtype odt, long long ldo, long long so, bool final_out) -> int {
    GemmParams g;
    g.M = n; g.N = m; g.K = n;
    g.A = Q; g.lda = n; g.sA = sn;
    g.B = cx; g.ldb = cld; g.sB = csx;
    g.D = out; g.ldd = ldo; g.sD = so;
    const float out_mul = final_out ? 1.0f : P;      // stored X-like iterates carry P
    if (cx_orig && c.Xh) {
      // the fp16 copy P s X: the same operand values the conversion below would form
      g.B = c.Xh; g.ldb = c.ldxh; g.sB = c.sxh;
      g.alpha = out_mul / P;
      HIP_OK(launch_rect(cdt, cdt, odt, g, B, c.stream, c.flops));
      return GNS_OK;
    }
    if (cx_orig && c.rows) x_rows(g);
    if (cx_orig) {
      if (cxdt == cdt) {
        g.alpha = out_mul; g.scale = s; g.alpha_pow = 1;
      } else {
        g.b_mul = P; g.scale = s; g.b_pow = 1; g.alpha = out_mul / P;
      }
    } else {
      g.alpha = out_mul / P;
    }
    HIP_OK(launch_rect(cdt, cxdt, odt, g, B, c.stream, c.flops));
    return GNS_OK;
  };

  for (int t = 1; t <= c.sch.steps; ++t) {
    const float a = c.sch.a[t - 1], b = c.sch.b[t - 1], cc = c.sch.c[t - 1];
    if (restart_before(t) && !q_identity) {
      void* xn = (cx == L.Xa) ? L.Xb : L.Xa;
      int st = apply_q(xn, cdt, m, nm, false);
      if (st) return st;
      cx = xn; cxdt = cdt; cld = m; csx = nm; cx_orig = false;
      GemmParams g = symm_params(n, m, cx, m, nm, cx, m, nm, L.R, n, sn);
      chain(g, 1, 1, 1, pl);
      g.alpha = 1.0f / (P * P);
      HIP_OK(launch_symm_ws(cdt, cdt, g, B, L.part, L.part_bytes, c.stream, c.flops));
      q_identity = true;
    }
    // Za = Z + a I = a I + b R + c R R, stored once (its diagonal rounded with the
    // rest): every later use of Z in the step is through Z + a I -- Q Za, R Za and
    // Za Y -- so those products need no beta C term.  While Q is the identity Za is
    // also the new Q, so it goes straight to Q's buffer.
    void* za = q_identity ? Q : L.Z;
    {
      GemmParams g = symm_params(n, n, L.R, n, sn, L.R, n, sn, za, n, sn);
      chain(g, pl, pl, pl, pl);
      g.alpha = cc; g.beta = b; g.C = L.R; g.ldc = n; g.sC = sn; g.gamma = a;
      HIP_OK(launch_symm(cdt, cdt, g, B, c.stream, c.flops));
    }
    const bool need_r = t < c.sch.steps && !restart_before(t + 1);
    // Q <- Q Za and Y = R Za read the same Za: with both needed, one launch computes
    // the pair
    const bool q_update = !q_identity;
    if (q_update) {
      GemmParams g = symm_params(n, n, Q, n, sn, za, n, sn, Qn, n, sn);
      chain(g, 1, pl, 1, 1);
      if (need_r) {
        g.pair = 1; g.A2 = L.R; g.Dp = L.Y;
        g.a2_planes = pl; g.dp_planes = pl;
      }
      HIP_OK(launch_symm(cdt, cdt, g, B, c.stream, c.flops));
      std::swap(Q, Qn);
    }
    q_identity = false;
    if (need_r) {
      if (!q_update) {
        GemmParams g1 = symm_params(n, n, L.R, n, sn, za, n, sn, L.Y, n, sn);     // Y = R Za
        chain(g1, pl, pl, pl, pl);
        HIP_OK(launch_symm(cdt, cdt, g1, B, c.stream, c.flops));
      }
      GemmParams g2 = symm_params(n, n, za, n, sn, L.Y, n, sn, L.R, n, sn);       // R = Za Y
      chain(g2, pl, pl, pl, pl);
      HIP_OK(launch_symm(cdt, cdt, g2, B, c.stream, c.flops));
    }
  }
  return apply_q(c.O, c.odt, c.ldo, c.so, true);
}

// Standard quintic NS on the same kernels: X0 = P s X (iterate dtype), then per step
// A = X X^T / P^2, Ba = a I + b A + c A A, X <- Ba X (= a X + (b A + c A A) X);
// finally O = X / P.
int run_standard(const NsCall& c) {
  const NsLayout L = ns_layout(c.ws, c.batch, c.n, c.m, c.cdt);
  const int n = c.n, m = c.m, B = c.batch;
  const long long nn = (long long)n * n, nm = (long long)n * m;
  const float P = pow2_scale(c.cdt, n, m);
  const float* s = c.s_given ? c.s_given : L.s;
  if (!c.s_given && c.partials_given)
    HIP_OK(launch_frob_finish(c.partials_given, c.n_partials_given, B, c.sch.eps, L.s, c.stream));
  else if (!c.s_given)
    HIP_OK(launch_frob(c.X, c.xdt, c.ldx, c.sx, B, n, m, c.sch.eps, L.s, L.partials, c.stream));
  HIP_OK(launch_cast_scale(c.X, c.xdt, c.ldx, c.sx, L.Sa, c.cdt, m, nm, B, n, m, P, s, 1, c.stream));
  void* cur = L.Sa; void* nxt = L.Sb;
  for (int t = 1; t <= c.sch.steps; ++t) {
    const float a = c.sch.a[t - 1], b = c.sch.b[t - 1], cc = c.sch.c[t - 1];
    GemmParams g1 = symm_params(n, m, cur, m, nm, cur, m, nm, L.A, n, nn);
    g1.alpha = 1.0f / (P * P);
    HIP_OK(launch_symm_ws(c.cdt, c.cdt, g1, B, L.part, L.part_bytes, c.stream, c.flops));
    // Ba stored once (its diagonal rounded with the rest), so the X update reads no C
    GemmParams g2 = symm_params(n, n, L.A, n, nn, L.A, n, nn, L.Bm, n, nn);
    g2.alpha = cc; g2.beta = b; g2.C = L.A; g2.ldc = n; g2.sC = nn; g2.gamma = a;
    HIP_OK(launch_symm(c.cdt, c.cdt, g2, B, c.stream, c.flops));
    GemmParams g3;
    g3.M = n; g3.N = m; g3.K = n;
    g3.A = L.Bm; g3.lda = n; g3.sA = nn;
    g3.B = cur; g3.ldb = m; g3.sB = nm;
    g3.D = nxt; g3.ldd = m; g3.sD = nm;
    HIP_OK(launch_rect(c.cdt, c.cdt, c.cdt, g3, B, c.stream, c.flops));
    std::swap(cur, nxt);
  }
  HIP_OK(launch_cast_scale(cur, c.cdt, m, nm, c.O, c.odt, c.ldo, c.so, B, n, m, 1.0f / P, nullptr, 0, c.stream));
  return GNS_OK;
}

// Gram NS (gram) or standard NS for any orientation.  n > m: Newton-Schulz iterates
// on the short side, so the call runs on X^T and transposes the result back ("Muon:
// Orthogonalized Momentum ...", section "Doing an SVD without an SVD"); polar(X^T) =
// polar(X)^T, and so does every step of the iteration.
int run_ns(const NsCall& c, bool gram) {
  if (c.n <= c.m) return (gram && !(c.sch.square_fallback && c.n == c.m)) ? run_gram(c) : run_standard(c);
  const TallLayout L = tall_layout(c.ws, c.batch, c.n, c.m, c.cdt);
  const long long tn = (long long)c.m * c.n;     // batch stride of the transposes
  HIP_OK(launch_transpose(c.X, c.xdt, c.ldx, c.sx, c.batch, c.n, c.m, L.Xt, c.n, tn, c.stream));
  NsCall w = c;
  w.X = L.Xt; w.ldx = c.n; w.sx = tn;
  w.O = L.Ot; w.ldo = c.n; w.so = tn;
  w.n = c.m; w.m = c.n;
  w.ws = L.inner; w.ws_bytes = L.inner_bytes;
  const int st = (gram && !(w.sch.square_fallback && w.n == w.m)) ? run_gram(w) : run_standard(w);
  if (st) return st;
  HIP_OK(launch_transpose(L.Ot, c.odt, c.n, tn, c.batch, c.m, c.n, c.O, c.ldo, c.so, c.stream));
  return GNS_OK;
}

NsCall make_call(const void* X, gns_dtype xdt, long long ldx, long long sx, void* O, gns_dtype odt, long long ldo,
                 long long so, int batch, int n, int m, gns_dtype cdt, const gns_schedule* sched, void* ws,
                 size_t ws_bytes, hipStream_t stream, double* flops) {
  NsCall c{};
  c.X = X; c.xdt = xdt; c.ldx = ldx; c.sx = sx;
  c.O = O; c.odt = odt; c.ldo = ldo; c.so = so;
  c.batch = batch; c.n = n; c.m = m; c.cdt = cdt;
  if (sched) c.sch = *sched; else gns_default_schedule(&c.sch);
  c.ws = ws; c.ws_bytes = ws_bytes; c.stream = stream; c.flops = flops; c.s_given = nullptr;
  c.partials_given = nullptr; c.n_partials_given = 0;
  c.rows = nullptr; c.rows_valid = 0; c.src_rows = 0; c.rows_stride = 0;
  c.Xh = nullptr; c.ldxh = 0; c.sxh = 0;
  return c;
}

// ---- the no-allocation entry point's scratch ------------------------------------
// gns_orthogonalize_batched_noalloc runs the workspace variant's kernels on this
// file-scope device array instead of a caller's workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code the array's name is
// only a stand-in: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept in g_scratch.
constexpr size_t kScratchBytes = GNS_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (which must be the stream's).
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  HIP_OK(hipGetDevice(&dev));
  if (stream) {
    hipDevice_t sdev = 0;
    HIP_OK(hipStreamGetDevice(stream, &sdev));
    if ((int)sdev != dev) {
      std::snprintf(g_last_error, sizeof(g_last_error), "the stream belongs to device %d, the current device is %d",
                    (int)sdev, dev);
      return GNS_ERR_INVALID_ARG;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) return GNS_ERR_UNSUPPORTED;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // this device is current
    slot.ptr = p;
  });
  if (slot.err != hipSuccess) return hip_fail(slot.err, "hipGetSymbolAddress(scratch)");
  *out = slot.ptr;
  return GNS_OK;
}

}  // namespace

extern "C" {

void gns_default_schedule(gns_schedule* s) {
  if (!s) return;
  std::memset(s, 0, sizeof(*s));
  s->steps = 5;
  for (int t = 0; t < 5; ++t) { s->a[t] = 3.4445f; s->b[t] = -4.7750f; s->c[t] = 2.0315f; }
  s->restart_after_mask = 1u << 2;    // restart after step 2 (before step 3)
  s->eps = 1e-7f;
  s->square_fallback = 1;
  s->rows_in_place = 0;
}

const char* gns_last_error(void) { return g_last_error; }

const char* gns_status_string(int status) {
  switch (status) {
    case GNS_OK: return "GNS_OK";
    case GNS_ERR_INVALID_ARG: return "GNS_ERR_INVALID_ARG";
    case GNS_ERR_UNSUPPORTED: return "GNS_ERR_UNSUPPORTED";
    case GNS_ERR_WORKSPACE: return "GNS_ERR_WORKSPACE";
    case GNS_ERR_HIP: return "GNS_ERR_HIP";
  }
  return "GNS_UNKNOWN_STATUS";
}

size_t gns_frobenius_workspace_size(int batch, int n, int m) {
  if (batch < 0 || n < 1 || m < 1) return 0;
  return align_up(sizeof(float) * (size_t)batch * frob_partials_per_batch(n, m));
}

int gns_frobenius_scale(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x, int batch, int n,
                        int m, float eps, float* s_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(x_dtype) || batch < 0 || n < 1 || m < 1 || ldx < m) return GNS_ERR_INVALID_ARG;
  if (batch == 0) return GNS_OK;
  if (!X || !s_out) return GNS_ERR_INVALID_ARG;
  if (batch > 1 && stride_x < (long long)n * ldx) return GNS_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return GNS_ERR_INVALID_ARG;
  const int q = x_dtype == GNS_F32 ? 4 : 8;
  if (m % q || ldx % q || (batch > 1 && stride_x % q) || !aligned16(X)) return GNS_ERR_UNSUPPORTED;
  if (!workspace || ws_bytes < gns_frobenius_workspace_size(batch, n, m)) return GNS_ERR_WORKSPACE;
  HIP_OK(launch_frob(X, x_dtype, ldx, stride_x, batch, n, m, eps, s_out, (float*)workspace, stream));
  return GNS_OK;
}

size_t gns_workspace_size(int batch, int n, int m, gns_dtype compute) {
  if (batch < 0 || n < 1 || m < 1 || !valid_dtype(compute)) return 0;
  return ns_workspace_bytes(batch, n, m, compute);
}

int gns_orthogonalize_batched(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x, void* O,
                              gns_dtype o_dtype, long long ldo, long long stride_o, int batch, int n, int m,
                              gns_dtype compute, const gns_schedule* sched, void* workspace, size_t ws_bytes,
                              hipStream_t stream, double* issued_flops) {
  NsCall c = make_call(X, x_dtype, ldx, stride_x, O, o_dtype, ldo, stride_o, batch, n, m, compute, sched, workspace,
                       ws_bytes, stream, issued_flops);
  if (issued_flops) *issued_flops = 0.0;
  const int st = check_ns(c);
  if (st) return st;
  if (batch == 0) return GNS_OK;
  return run_ns(c, true);
}

int gns_newton_schulz_batched(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x, void* O,
                              gns_dtype o_dtype, long long ldo, long long stride_o, int batch, int n, int m,
                              gns_dtype compute, const gns_schedule* sched, void* workspace, size_t ws_bytes,
                              hipStream_t stream, double* issued_flops) {
  NsCall c = make_call(X, x_dtype, ldx, stride_x, O, o_dtype, ldo, stride_o, batch, n, m, compute, sched, workspace,
                       ws_bytes, stream, issued_flops);
  c.sch.restart_after_mask = 0;
  if (issued_flops) *issued_flops = 0.0;
  const int st = check_ns(c);
  if (st) return st;
  if (batch == 0) return GNS_OK;
  return run_ns(c, false);
}

int gns_orthogonalize_batched_noalloc(const void* X, gns_dtype x_dtype, long long ldx, long long stride_x, void* O,
                                      gns_dtype o_dtype, long long ldo, long long stride_o, int batch, int n, int m,
                                      gns_dtype compute, const gns_schedule* sched, hipStream_t stream,
                                      double* issued_flops) {
  if (issued_flops) *issued_flops = 0.0;
  if (batch < 0 || n < 1 || m < 1 || !valid_dtype(compute)) return GNS_ERR_INVALID_ARG;
  const size_t need = ns_workspace_bytes(batch, n, m, compute);
  if (need > kScratchBytes) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "the call needs %zu bytes of scratch, more than the %zu bytes of the static scratch", need,
                  kScratchBytes);
    return GNS_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  int st = scratch_address(stream, &ws);
  if (st) return st;
  NsCall c = make_call(X, x_dtype, ldx, stride_x, O, o_dtype, ldo, stride_o, batch, n, m, compute, sched, ws,
                       kScratchBytes, stream, issued_flops);
  if ((st = check_ns(c))) return st;
  if (batch == 0) return GNS_OK;
  return run_ns(c, true);
}

static int check_gemm_common(int batch, gns_dtype in, gns_dtype out, const void* A, long long lda, long long sA,
                             const void* D, long long ldd, long long sD) {
  (void)sA; (void)sD;
  if (!valid_dtype(in) || !valid_dtype(out) || batch < 0) return GNS_ERR_INVALID_ARG;
  if (batch > 0 && (!A || !D)) return GNS_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(D)) return GNS_ERR_UNSUPPORTED;
  (void)lda; (void)ldd;
  return GNS_OK;
}

int symm_gemm(int batch, int n, int k, float alpha, const void* A, long long lda, long long stride_a, const void* B,
              long long ldb, long long stride_b, float beta, const void* C, long long ldc, long long stride_c,
              float gamma, void* D, long long ldd, long long stride_d, gns_dtype in_dtype, gns_dtype out_dtype,
              hipStream_t stream) {
  int st = check_gemm_common(batch, in_dtype, out_dtype, A, lda, stride_a, D, ldd, stride_d);
  if (st) return st;
  if (n < 0 || k < 0) return GNS_ERR_INVALID_ARG;
  if (batch == 0 || n == 0) return GNS_OK;
  if (!B || (beta != 0.0f && !C)) return GNS_ERR_INVALID_ARG;
  if (lda < k || ldb < k || ldd < n || (C && ldc < n)) return GNS_ERR_INVALID_ARG;
  if (batch > 1 && (stride_a < (long long)n * lda || stride_b < (long long)n * ldb || stride_d < (long long)n * ldd ||
                    (C && stride_c < (long long)n * ldc)))
    return GNS_ERR_INVALID_ARG;
  const int q = in_dtype == GNS_F32 ? 4 : 8, qo = out_dtype == GNS_F32 ? 4 : 8;
  if (n % 8 || k % q || lda % q || ldb % q || ldd % qo || (C && ldc % qo)) return GNS_ERR_UNSUPPORTED;
  if (batch > 1 && (stride_a % q || stride_b % q || stride_d % qo || (C && stride_c % qo))) return GNS_ERR_UNSUPPORTED;
  if (!aligned16(B) || (C && !aligned16(C))) return GNS_ERR_UNSUPPORTED;
  GemmParams g = symm_params(n, k, A, lda, stride_a, B, ldb, stride_b, D, ldd, stride_d);
  g.alpha = alpha; g.beta = beta; g.gamma = gamma;
  if (C && beta != 0.0f) { g.C = C; g.ldc = ldc; g.sC = stride_c; }
  HIP_OK(launch_symm(in_dtype, out_dtype, g, batch, stream, nullptr));
  return GNS_OK;
}

int rect_gemm(int batch, int n, int k, int m, float alpha, const void* A, long long lda, long long stride_a,
              gns_dtype a_dtype, const void* B, long long ldb, long long stride_b, gns_dtype b_dtype,
              float b_prescale, float beta, const void* C, long long ldc, long long stride_c, void* D, long long ldd,
              long long stride_d, gns_dtype out_dtype, hipStream_t stream) {
  int st = check_gemm_common(batch, a_dtype, out_dtype, A, lda, stride_a, D, ldd, stride_d);
  if (st) return st;
  if (!valid_dtype(b_dtype) || n < 0 || k < 0 || m < 0) return GNS_ERR_INVALID_ARG;
  if (batch == 0 || n == 0 || m == 0) return GNS_OK;
  if (!rect_pair_supported(a_dtype, b_dtype)) return GNS_ERR_UNSUPPORTED;
  if (a_dtype == b_dtype && b_prescale != 1.0f) return GNS_ERR_INVALID_ARG;
  if (!B || (beta != 0.0f && !C)) return GNS_ERR_INVALID_ARG;
  if (lda < k || ldb < m || ldd < m || (C && ldc < m)) return GNS_ERR_INVALID_ARG;
  if (batch > 1 && (stride_a < (long long)n * lda || stride_b < (long long)k * ldb || stride_d < (long long)n * ldd ||
                    (C && stride_c < (long long)n * ldc)))
    return GNS_ERR_INVALID_ARG;
  const int q = a_dtype == GNS_F32 ? 4 : 8, qo = out_dtype == GNS_F32 ? 4 : 8;
  if (k % q || m % 8 || lda % q || ldb % q || ldd % qo || (C && ldc % qo)) return GNS_ERR_UNSUPPORTED;
  if (batch > 1 && (stride_a % q || stride_b % q || stride_d % qo || (C && stride_c % qo))) return GNS_ERR_UNSUPPORTED;
  if (!aligned16(B) || (C && !aligned16(C))) return GNS_ERR_UNSUPPORTED;
  GemmParams g;
  g.M = n; g.N = m; g.K = k;
  g.A = A; g.lda = lda; g.sA = stride_a;
  g.B = B; g.ldb = ldb; g.sB = stride_b;
  g.D = D; g.ldd = ldd; g.sD = stride_d;
  g.alpha = alpha; g.beta = beta; g.b_mul = b_prescale;
  if (C && beta != 0.0f) { g.C = C; g.ldc = ldc; g.sC = stride_c; }
  HIP_OK(launch_rect(a_dtype, b_dtype, out_dtype, g, batch, stream, nullptr));
  return GNS_OK;
}

// ---- Dion3 ------------------------------------------------------------------------

static int check_dion3_matrix(const void* P, gns_dtype dt, int N, int m, long long ld) {
  if (!P || !valid_dtype(dt) || N < 1 || m < 1 || ld < m) return GNS_ERR_INVALID_ARG;
  if (m % 8 || ld % 8 || !aligned16(P)) return GNS_ERR_UNSUPPORTED;
  return GNS_OK;
}

int dion3_accumulate_score(void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int score_norm,
                           double* score, double* sumsq, hipStream_t stream) {
  int st = check_dion3_matrix(M, dt, N, m, ld);
  if (st) return st;
  st = check_dion3_matrix(G, dt, N, m, ld);
  if (st) return st;
  if (!score || (score_norm != 1 && score_norm != 2)) return GNS_ERR_INVALID_ARG;
  HIP_OK(launch_accumulate_score(M, G, dt, 1, N, m, ld, 0, score_norm, score, sumsq, stream));
  return GNS_OK;
}

int dion3_select_topk(const double* score, int N, int k, int* S, hipStream_t stream) {
  if (!score || !S || N < 1 || k < 1 || k > N) return GNS_ERR_INVALID_ARG;
  HIP_OK(launch_topk(score, 1, N, k, S, stream));
  return GNS_OK;
}

int dion3_gather_feedback(void* M, gns_dtype dt, int N, int m, long long ld, const int* S, int k, float mu, void* X,
                          long long ldx, hipStream_t stream) {
  int st = check_dion3_matrix(M, dt, N, m, ld);
  if (st) return st;
  if (!S || !X || k < 1 || k > N || ldx < m || !std::isfinite(mu)) return GNS_ERR_INVALID_ARG;
  if (ldx % 8 || !aligned16(X)) return GNS_ERR_UNSUPPORTED;
  HIP_OK(launch_gather_feedback(M, dt, 1, N, m, ld, 0, S, k, k, mu, nullptr, X, ldx, stream));
  return GNS_OK;
}

int dion3_apply_update(void* W, gns_dtype dt, int N, int m, long long ld, const int* S, int k, const void* O,
                       gns_dtype o_dtype, long long ldo, float lr, float wd, hipStream_t stream) {
  int st = check_dion3_matrix(W, dt, N, m, ld);
  if (st) return st;
  if (!S || !O || k < 1 || k > N || ldo < m || !std::isfinite(lr) || !std::isfinite(wd)) return GNS_ERR_INVALID_ARG;
  if (!valid_dtype(o_dtype)) return GNS_ERR_INVALID_ARG;
  if (ldo % 8 || !aligned16(O)) return GNS_ERR_UNSUPPORTED;
  HIP_OK(launch_apply_update(W, dt, 1, N, m, ld, 0, S, k, O, o_dtype, ldo, (long long)k * ldo, lr, wd, nullptr,
                             stream));
  return GNS_OK;
}

struct Dion3Layout {
  double* score; double* sumsq; float* s; void* X; void* Xc; void* Xh; void* O; void* gns_ws; size_t gns_bytes;
  size_t bytes;
};

// An fp32 state meets the 16-bit iterates through a copy of the submatrix scaled by
// its Frobenius scale and rounded once to the iterate type (the iteration reads a
// 16-bit X with 16-bit iterates); the iteration then normalises that copy itself,
// whose norm is 1 up to the rounding.
static bool state_casts_x(gns_dtype dt) { return dt == GNS_F32; }

// A bf16 state with fp16 iterates and at least 2048 selected rows: the gather also
// writes the selected rows as the fp16 copy P s X that the restart and final products
// read instead of converting the bf16 rows on every load (each 256 x 256 tile row of
// the product converts them once; the Gram products keep the bf16 rows, so the step
// stays bitwise the step that reads the rows in place).  Measured on MI355X: the
// 8192 x 28672 state at k = 2048 1.476 against 1.490 ms per step; at k = 1024 no
// change; 16 states of 2048 x 8192 at k = 512 0.963 against 0.928 ms, so fewer rows
// keep the conversion.
constexpr int kHalfCopyMinRows = 2048;
static bool state_half_copy(gns_dtype dt, gns_dtype cdt, int kp) {
  return dt == GNS_BF16 && cdt == GNS_F16 && kp >= kHalfCopyMinRows;
}

// The selected submatrix is held with kp = k rounded up to a multiple of 8 rows; the
// extra rows are zero.  Zero rows leave the iteration's result on the other rows
// unchanged (they add zero rows and columns to R and every polynomial in it), and
// every kernel then works on whole 8-row groups.
int padded_rows(int k) { return (k + 7) / 8 * 8; }

static Dion3Layout dion3_layout(void* base, int batch, int N, int m, int k, gns_dtype dt, gns_dtype cdt) {
  Carver c{reinterpret_cast<uint8_t*>(base), 0};
  Dion3Layout L{};
  const size_t B = (size_t)batch;
  const int kp = padded_rows(k);
  L.score = (double*)c.take(sizeof(double) * B * N);
  L.sumsq = (double*)c.take(sizeof(double) * B * N);
  L.s = (float*)c.take(sizeof(float) * B);
  L.X = c.take(B * kp * m * esize(dt));
  L.Xc = state_casts_x(dt) ? c.take(B * kp * m * esize(cdt)) : nullptr;
  L.Xh = state_half_copy(dt, cdt, kp) ? c.take(B * kp * m * 2) : nullptr;
  L.O = c.take(B * kp * m * esize(dt));
  L.gns_bytes = ns_workspace_bytes(batch, kp, m, cdt);
  L.gns_ws = c.take(L.gns_bytes);
  L.bytes = c.off;
  return L;
}

size_t dion3_batched_workspace_size(int batch, int N, int m, int k, gns_dtype dt, gns_dtype compute) {
  if (batch < 1 || N < 1 || m < 1 || k < 1 || !valid_dtype(dt) || !valid_dtype(compute)) return 0;
  return dion3_layout(nullptr, batch, N, m, k, dt, compute).bytes;
}

size_t dion3_workspace_size(int N, int m, int k, gns_dtype dt, gns_dtype compute) {
  return dion3_batched_workspace_size(1, N, m, k, dt, compute);
}

// One Dion3 step over `batch` states: the rows are the top-k by score (S_in null; S
// receives them) or the caller's set S_in.
static int dion3_run(void* W, void* M, const void* G, gns_dtype dt, int batch, int N, int m, long long ld,
                     long long stride, int k,
                     float lr, float weight_decay, float mu, int score_norm, gns_dtype compute,
                     const gns_schedule* sched, const int* S_in, int* S_out, void* O_out, void* workspace,
                     size_t ws_bytes, hipStream_t stream, const float* dev_scalars = nullptr) {
  if (batch < 0) return GNS_ERR_INVALID_ARG;
  if (batch == 0) return GNS_OK;
  int st = check_dion3_matrix(W, dt, N, m, ld);
  if (st) return st;
  if ((st = check_dion3_matrix(M, dt, N, m, ld))) return st;
  if ((st = check_dion3_matrix(G, dt, N, m, ld))) return st;
  if (batch > 1 && stride < (long long)N * ld) return GNS_ERR_INVALID_ARG;
  if (batch > 1 && stride % 8) return GNS_ERR_UNSUPPORTED;
  if ((!S_in && !S_out) || k < 1 || k > N) return GNS_ERR_INVALID_ARG;
  if (score_norm != 1 && score_norm != 2) return GNS_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(mu)) return GNS_ERR_INVALID_ARG;
  if (!valid_dtype(compute)) return GNS_ERR_INVALID_ARG;
  if (compute == GNS_F32) return GNS_ERR_UNSUPPORTED;
  if (O_out && !aligned16(O_out)) return GNS_ERR_UNSUPPORTED;
  // W, M and G must be distinct (each is read and written by different passes)
  const size_t es = esize(dt);
  const size_t span = ((size_t)(batch - 1) * (size_t)(batch > 1 ? stride : 0) + (size_t)(N - 1) * ld + m) * es;
  if (overlaps(W, span, M, span) || overlaps(W, span, G, span) || overlaps(M, span, G, span))
    return GNS_ERR_INVALID_ARG;
  gns_schedule sch;
  if (sched) sch = *sched; else gns_default_schedule(&sch);
  if ((st = check_schedule(sch))) return st;
  const Dion3Layout L = dion3_layout(workspace, batch, N, m, k, dt, compute);
  if (!workspace || ws_bytes < L.bytes) return GNS_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GNS_ERR_UNSUPPORTED;

  // the submatrices are padded to kp rows (zeros); with kp == k the caller's O_out
  // receives O directly, else O goes to the workspace and its k rows are copied out
  const int kp = padded_rows(k);
  void* O = (O_out && kp == k) ? O_out : L.O;
  const long long km = (long long)k * m, kpm = (long long)kp * m;
  if (overlaps(workspace, L.bytes, W, span) || overlaps(workspace, L.bytes, M, span) ||
      overlaps(workspace, L.bytes, G, span))
    return GNS_ERR_INVALID_ARG;
  // With rows_in_place, the selected rows are read straight from M by the Gram path's
  // products (the submatrix X is never written; Algorithm 4 orthogonalises M[S, :]
  // itself), and the error feedback on M[S, :] runs with the weight update, after the
  // last read.  That needs the Gram path on a wide submatrix (a square one may fall
  // back to standard NS, a tall one runs on a transpose), a bf16 state (the indexed
  // products read bf16 rows), a row table that fits in LDS and a state addressable with
  // 32-bit offsets; otherwise the rows are gathered into X first (the default: faster
  // on MI355X, where the fresh copy sits in the Infinity Cache for the products that
  // re-read it).
  const bool gram_path = kp < m || (kp == m && !sch.square_fallback);
  const bool direct = sch.rows_in_place && dt == GNS_BF16 && gram_path && kp <= kMaxIndexedRows &&
                      ((size_t)(N - 1) * ld + m) * es < (size_t(1) << 31);
  // one batched Gram NS over the selected kp x m submatrices of every entry (input and
  // output in the state type); its arguments are checked before anything is launched
  const bool cast_x = state_casts_x(dt);
  NsCall c = direct ? make_call(M, dt, ld, stride, O, dt, m, kpm, batch, kp, m, compute, &sch, L.gns_ws,
                                L.gns_bytes, stream, nullptr)
                    : make_call(cast_x ? L.Xc : L.X, cast_x ? compute : dt, m, kpm, O, dt, m, kpm, batch, kp, m,
                                compute, &sch, L.gns_ws, L.gns_bytes, stream, nullptr);
  c.s_given = cast_x ? nullptr : L.s;
  if ((st = check_ns(c))) return st;
  const size_t o_bytes = (size_t)batch * km * es;
  if (O_out && (overlaps(O_out, o_bytes, workspace, L.bytes) || overlaps(O_out, o_bytes, W, span) ||
                overlaps(O_out, o_bytes, M, span) || overlaps(O_out, o_bytes, G, span)))
    return GNS_ERR_INVALID_ARG;

  HIP_OK(launch_accumulate_score(M, G, dt, batch, N, m, ld, stride, score_norm, L.score, L.sumsq, stream));
  const int* S = S_in;
  if (!S_in) {
    HIP_OK(launch_topk(L.score, batch, N, k, S_out, stream));
    S = S_out;
  }
  // the Frobenius scale of the selected rows comes from the accumulate pass's row sums,
  // so it is known before the gather (which scales the fp16 copy with it)
  HIP_OK(launch_selected_sumsq(L.sumsq, S, batch, k, N, sch.eps, L.s, stream));
  if (direct) {
    c.rows = S; c.rows_valid = k; c.rows_stride = k; c.src_rows = N;
  } else if (L.Xh && gram_path) {
    HIP_OK(launch_gather_feedback(M, dt, batch, N, m, ld, stride, S, k, kp, mu, dev_scalars, L.X, m, stream, L.Xh,
                                  L.s, pow2_scale(compute, kp, m)));
    c.Xh = L.Xh; c.ldxh = m; c.sxh = kpm;
  } else {
    HIP_OK(launch_gather_feedback(M, dt, batch, N, m, ld, stride, S, k, kp, mu, dev_scalars, L.X, m, stream));
  }
  if (cast_x)
    HIP_OK(launch_cast_scale(L.X, dt, m, kpm, L.Xc, compute, m, kpm, batch, kp, m, 1.0f, L.s, 1, stream));
  if ((st = run_ns(c, true))) return st;
  if (O_out && O != O_out)
    HIP_OK(launch_cast_scale(O, dt, m, kpm, O_out, dt, m, km, batch, k, m, 1.0f, nullptr, 0, stream));
  HIP_OK(launch_apply_update(W, dt, batch, N, m, ld, stride, S, k, O, dt, m, kpm, lr, weight_decay, dev_scalars,
                             stream, direct ? M : nullptr, mu));
  return GNS_OK;
}

int dion3_step_batched(void* W, void* M, const void* G, gns_dtype dt, int batch, int N, int m, long long ld,
                       long long stride, int k, float lr, float weight_decay, float mu, int score_norm,
                       gns_dtype compute, const gns_schedule* sched, int* S_out, void* O_out, void* workspace,
                       size_t ws_bytes, hipStream_t stream) {
  if (!S_out) return GNS_ERR_INVALID_ARG;
  return dion3_run(W, M, G, dt, batch, N, m, ld, stride, k, lr, weight_decay, mu, score_norm, compute, sched,
                   nullptr, S_out, O_out, workspace, ws_bytes, stream);
}

int dion3_step(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k, float lr,
               float weight_decay, float mu, int score_norm, gns_dtype compute, const gns_schedule* sched, int* S_out,
               void* O_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return dion3_step_batched(W, M, G, dt, 1, N, m, ld, (long long)N * ld, k, lr, weight_decay, mu, score_norm,
                            compute, sched, S_out, O_out, workspace, ws_bytes, stream);
}

int dion3_step_dev_scalars(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k,
                           const float* lr_wd_mu, int score_norm, gns_dtype compute, const gns_schedule* sched,
                           int* S_out, void* O_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!S_out || !lr_wd_mu) return GNS_ERR_INVALID_ARG;
  if ((uintptr_t)lr_wd_mu & 3u) return GNS_ERR_UNSUPPORTED;
  // the host scalars are placeholders (finite, as checked); the kernels read the device values
  return dion3_run(W, M, G, dt, 1, N, m, ld, (long long)N * ld, k, 0.0f, 0.0f, 0.0f, score_norm, compute, sched,
                   nullptr, S_out, O_out, workspace, ws_bytes, stream, lr_wd_mu);
}

// Column selection workspace: partial column sums, the column scores and sums of
// squares, the column marks (for the decay), the scale, X^T and O (k x N), then the
// Gram NS workspace for the k x N submatrix.
struct Dion3ColsLayout {
  double *part_s, *part_q, *score, *sumsq;
  uint8_t* mark;
  float* s;
  void *Xt, *Xtc, *O, *gns_ws;
  size_t gns_bytes, bytes;
};

static Dion3ColsLayout dion3_cols_layout(void* base, int N, int m, int k, gns_dtype dt, gns_dtype cdt) {
  Carver c{reinterpret_cast<uint8_t*>(base), 0};
  Dion3ColsLayout L{};
  const size_t parts = dion3_cols_partials(N) * (size_t)m;
  L.part_s = (double*)c.take(sizeof(double) * parts);
  L.part_q = (double*)c.take(sizeof(double) * parts);
  L.score = (double*)c.take(sizeof(double) * (size_t)m);
  L.sumsq = (double*)c.take(sizeof(double) * (size_t)m);
  L.mark = (uint8_t*)c.take((size_t)m);
  L.s = (float*)c.take(sizeof(float));
  const int kp = padded_rows(k);
  L.Xt = c.take((size_t)kp * N * esize(dt));
  L.Xtc = state_casts_x(dt) ? c.take((size_t)kp * N * esize(cdt)) : nullptr;
  L.O = c.take((size_t)kp * N * esize(dt));
  L.gns_bytes = ns_workspace_bytes(1, kp, N, cdt);
  L.gns_ws = c.take(L.gns_bytes);
  L.bytes = c.off;
  return L;
}

size_t dion3_cols_workspace_size(int N, int m, int k, gns_dtype dt, gns_dtype compute) {
  if (N < 1 || m < 1 || k < 1 || !valid_dtype(dt) || !valid_dtype(compute)) return 0;
  return dion3_cols_layout(nullptr, N, m, k, dt, compute).bytes;
}

int dion3_step_cols(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, int k, float lr,
                    float weight_decay, float mu, int score_norm, gns_dtype compute, const gns_schedule* sched,
                    int* S_out, void* O_out, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_dion3_matrix(W, dt, N, m, ld);
  if (st) return st;
  if ((st = check_dion3_matrix(M, dt, N, m, ld))) return st;
  if ((st = check_dion3_matrix(G, dt, N, m, ld))) return st;
  if (!S_out || k < 1 || k > m) return GNS_ERR_INVALID_ARG;
  if (score_norm != 1 && score_norm != 2) return GNS_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(mu)) return GNS_ERR_INVALID_ARG;
  if (!valid_dtype(compute)) return GNS_ERR_INVALID_ARG;
  if (compute == GNS_F32) return GNS_ERR_UNSUPPORTED;
  if (N % 8) return GNS_ERR_UNSUPPORTED;   // N is the row length of X^T and O
  if (O_out && !aligned16(O_out)) return GNS_ERR_UNSUPPORTED;
  const size_t es = esize(dt);
  const size_t span = ((size_t)(N - 1) * ld + m) * es;
  if (overlaps(W, span, M, span) || overlaps(W, span, G, span) || overlaps(M, span, G, span))
    return GNS_ERR_INVALID_ARG;
  gns_schedule sch;
  if (sched) sch = *sched; else gns_default_schedule(&sch);
  if ((st = check_schedule(sch))) return st;
  const Dion3ColsLayout L = dion3_cols_layout(workspace, N, m, k, dt, compute);
  if (!workspace || ws_bytes < L.bytes) return GNS_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GNS_ERR_UNSUPPORTED;

  // X^T is padded to kp rows (zeros), as in the row step
  const int kp = padded_rows(k);
  void* O = (O_out && kp == k) ? O_out : L.O;
  const long long kN = (long long)k * N, kpN = (long long)kp * N;
  // the kp x N transpose of the selected columns: Gram NS iterates on its short side;
  // its arguments are checked before anything is launched
  const bool cast_x = state_casts_x(dt);
  NsCall c = make_call(cast_x ? L.Xtc : L.Xt, cast_x ? compute : dt, N, kpN, O, dt, N, kpN, 1, kp, N, compute, &sch,
                       L.gns_ws, L.gns_bytes, stream, nullptr);
  c.s_given = cast_x ? nullptr : L.s;
  if ((st = check_ns(c))) return st;
  const size_t o_bytes = (size_t)kN * es;
  if (O_out && (overlaps(O_out, o_bytes, workspace, L.bytes) || overlaps(O_out, o_bytes, W, span) ||
                overlaps(O_out, o_bytes, M, span) || overlaps(O_out, o_bytes, G, span)))
    return GNS_ERR_INVALID_ARG;

  HIP_OK(launch_accumulate_colscore(M, G, dt, N, m, ld, score_norm, L.part_s, L.part_q, L.score, L.sumsq, stream));
  HIP_OK(launch_topk(L.score, 1, m, k, S_out, stream));
  HIP_OK(launch_gather_cols_feedback(M, dt, N, m, ld, S_out, k, kp, mu, L.Xt, N, stream));
  HIP_OK(launch_selected_sumsq(L.sumsq, S_out, 1, k, m, sch.eps, L.s, stream));
  if (cast_x) HIP_OK(launch_cast_scale(L.Xt, dt, N, kpN, L.Xtc, compute, N, kpN, 1, kp, N, 1.0f, L.s, 1, stream));
  if ((st = run_ns(c, true))) return st;
  if (O_out && O != O_out)
    HIP_OK(launch_cast_scale(O, dt, N, kpN, O_out, dt, N, kN, 1, k, N, 1.0f, nullptr, 0, stream));
  HIP_OK(launch_update_cols(W, dt, N, m, ld, S_out, k, O, N, lr, weight_decay, L.mark, stream));
  return GNS_OK;
}

int dion3_step_rows(void* W, void* M, const void* G, gns_dtype dt, int N, int m, long long ld, const int* S, int k,
                    float lr, float weight_decay, float mu, gns_dtype compute, const gns_schedule* sched, void* O_out,
                    void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!S) return GNS_ERR_INVALID_ARG;
  // the sums of squares of the rows (score_norm 2) give the submatrix's Frobenius norm
  return dion3_run(W, M, G, dt, 1, N, m, ld, (long long)N * ld, k, lr, weight_decay, mu, 2, compute, sched, S,
                   nullptr, O_out, workspace, ws_bytes, stream);
}

// Muon step workspace: the row sums of squares and the scale of each matrix, U (the
// lookahead, only with nesterov), O, then the Gram NS workspace of the batch.
// Muon step workspace: the row sums of squares and the scale of each matrix, U (the
// lookahead, only with nesterov) and O in the state type, the scaled 16-bit copy of
// the matrix the iteration reads (fp32 states only, as for Dion3), then the Gram NS
// workspace of the batch.
struct MuonLayout {
  double* rowsq;
  float* rowsq32;        // the row sums rounded to fp32: the Gram products' partial sums
  float* s;
  void *U, *Xc, *O, *gns_ws;
  size_t gns_bytes, bytes;
};

static MuonLayout muon_layout(void* base, int batch, int n, int m, gns_dtype dt, gns_dtype cdt, int nesterov) {
  Carver c{reinterpret_cast<uint8_t*>(base), 0};
  MuonLayout L{};
  const size_t elems = (size_t)batch * n * m;
  L.rowsq = (double*)c.take(sizeof(double) * (size_t)batch * n);
  L.rowsq32 = (float*)c.take(sizeof(float) * (size_t)batch * n);
  L.s = (float*)c.take(sizeof(float) * (size_t)batch);
  L.U = nesterov ? c.take(elems * esize(dt)) : nullptr;
  L.Xc = state_casts_x(dt) ? c.take(elems * esize(cdt)) : nullptr;
  L.O = c.take(elems * esize(dt));
  L.gns_bytes = ns_workspace_bytes(batch, n, m, cdt);
  L.gns_ws = c.take(L.gns_bytes);
  L.bytes = c.off;
  return L;
}

size_t muon_workspace_size(int batch, int n, int m, gns_dtype dt, gns_dtype compute, int nesterov) {
  if (batch < 1 || n < 1 || m < 1 || !valid_dtype(dt) || !valid_dtype(compute) || (nesterov != 0 && nesterov != 1))
    return 0;
  return muon_layout(nullptr, batch, n, m, dt, compute, nesterov).bytes;
}

int muon_step_batched(void* W, void* M, const void* G, gns_dtype dt, int batch, int n, int m, long long ld,
                      long long stride, float lr, float weight_decay, float mu, int nesterov, float scale,
                      gns_dtype compute, const gns_schedule* sched, void* O_out, void* workspace, size_t ws_bytes,
                      hipStream_t stream) {
  if (batch < 0) return GNS_ERR_INVALID_ARG;
  if (batch == 0) return GNS_OK;
  int st = check_dion3_matrix(W, dt, n, m, ld);
  if (st) return st;
  if ((st = check_dion3_matrix(M, dt, n, m, ld))) return st;
  if ((st = check_dion3_matrix(G, dt, n, m, ld))) return st;
  if (batch > 1 && stride < (long long)n * ld) return GNS_ERR_INVALID_ARG;
  if (batch > 1 && stride % 8) return GNS_ERR_UNSUPPORTED;
  if (nesterov != 0 && nesterov != 1) return GNS_ERR_INVALID_ARG;
  if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(mu) || !std::isfinite(scale) ||
      scale < 0.0f)
    return GNS_ERR_INVALID_ARG;
  if (!valid_dtype(compute)) return GNS_ERR_INVALID_ARG;
  if (compute == GNS_F32) return GNS_ERR_UNSUPPORTED;
  if (O_out && !aligned16(O_out)) return GNS_ERR_UNSUPPORTED;
  // W, M and G must be distinct (each is read and written by different passes)
  const size_t es = esize(dt);
  const size_t span = ((size_t)(batch - 1) * (size_t)(batch > 1 ? stride : 0) + (size_t)(n - 1) * ld + m) * es;
  if (overlaps(W, span, M, span) || overlaps(W, span, G, span) || overlaps(M, span, G, span))
    return GNS_ERR_INVALID_ARG;
  gns_schedule sch;
  if (sched) sch = *sched; else gns_default_schedule(&sch);
  if ((st = check_schedule(sch))) return st;
  const MuonLayout L = muon_layout(workspace, batch, n, m, dt, compute, nesterov);
  if (!workspace || ws_bytes < L.bytes) return GNS_ERR_WORKSPACE;
  if (!aligned16(workspace)) return GNS_ERR_UNSUPPORTED;
  // the update's RMS matched to AdamW's: 0.2 sqrt(max(n, m)) unless the caller gives one
  // (scale == 0 asks for that default; a negative scale was rejected above)
  const float sc = scale != 0.0f ? scale : 0.2f * std::sqrt((float)std::max(n, m));

  void* O = O_out ? O_out : L.O;
  const long long nm = (long long)n * m;
  // the batched Gram NS of U (or of M itself without the lookahead), or of their
  // scaled 16-bit copy for an fp32 state; its arguments are checked before anything is
  // launched
  const void* src = nesterov ? L.U : M;
  const long long lds = nesterov ? m : ld, ss = nesterov ? nm : stride;
  const bool cast_x = state_casts_x(dt);
  NsCall c = cast_x ? make_call(L.Xc, compute, m, nm, O, dt, m, nm, batch, n, m, compute, &sch, L.gns_ws,
                                L.gns_bytes, stream, nullptr)
                    : make_call(src, dt, lds, ss, O, dt, m, nm, batch, n, m, compute, &sch, L.gns_ws, L.gns_bytes,
                                stream, nullptr);
  // The momentum pass also forms what the Frobenius scale needs: for a 16-bit state
  // its row sums (at most kMaxPartials rows) are the Gram products' partial sums, so
  // no pass over U and no scale launch precede Gram NS; otherwise it forms the scale
  // itself (an fp32 state's 16-bit copy is scaled by it).
  const bool rows_as_partials = !cast_x && n <= kMaxPartials;
  c.s_given = (cast_x || rows_as_partials) ? nullptr : L.s;
  if (rows_as_partials) {
    c.partials_given = L.rowsq32;
    c.n_partials_given = n;
  }
  if ((st = check_ns(c))) return st;
  const size_t o_bytes = (size_t)batch * nm * es;
  if (O_out && (overlaps(O_out, o_bytes, workspace, L.bytes) || overlaps(O_out, o_bytes, W, span) ||
                overlaps(O_out, o_bytes, M, span) || overlaps(O_out, o_bytes, G, span)))
    return GNS_ERR_INVALID_ARG;

  HIP_OK(launch_muon_momentum(M, G, dt, batch, n, m, ld, stride, mu, L.U, m, nm, L.rowsq,
                              rows_as_partials ? L.rowsq32 : nullptr, sch.eps, rows_as_partials ? nullptr : L.s,
                              stream));
  if (cast_x) HIP_OK(launch_cast_scale(src, dt, lds, ss, L.Xc, compute, m, nm, batch, n, m, 1.0f, L.s, 1, stream));
  if ((st = run_ns(c, true))) return st;
  HIP_OK(launch_muon_update(W, dt, batch, n, m, ld, stride, O, m, nm, lr, weight_decay, sc, stream));
  return GNS_OK;
}

}  // extern "C"

