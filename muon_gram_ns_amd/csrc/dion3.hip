// Dion3 element-wise and selection kernels (all HBM- or latency-bound).
//
// The update rule ("Dion3: Full-Stack Orthogonal Updates", paper.rainbus.top,
// 方法步骤详情 (3), Algorithm 4): M <- M + G; pick the k rows of largest norm;
// orthogonalise that submatrix; decay all weights by (1 - lr wd) and subtract
// lr O from the selected weight rows; decay only the selected momentum rows by mu
// (error feedback, same page, 前置知识).
//
// Rounding model (the pages do not fix it; this is the reading the oracle emulates):
// W, M, G are stored in one state type T (bf16, f16 or fp32); each stored value is
// rounded once, to nearest even, from fp32 results computed op by op.  This file is
// compiled with -ffp-contract=off and uses explicit __fmul_rn/__fsub_rn so no
// multiply-add is fused.  Row scores accumulate in fp64 (the per-element terms are
// exact in fp64).  Every kernel moves the state in 16-byte chunks: 8 elements of a
// 16-bit type or 4 fp32 elements.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "state_types.h"

namespace gns {

// 512 threads per row: measured on MI355X on the 8192 x 28672 bf16 state, the row
// gather reaches 6.0 TB/s against 5.4 TB/s with 256 threads, and the row update 6.5
// against 6.2 TB/s (more bytes in flight per row)
constexpr int kRowThreads = 512;

__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;
}

// ---- M <- fl(M + G); per-row score and sum of squares -------------------------------
// One workgroup per row.  Each thread takes chunks c, c+512, c+1024, ...; four chunks'
// loads are issued before any is used (more bytes in flight per wave), and the chunks
// are then summed in that same order, so each thread's fp64 sums do not depend on the
// unrolling.
// Streaming accesses of the state (each element read and written once per pass):
// non-temporal loads and stores.  Measured on MI355X on the 8192 x 28672 bf16 state,
// the accumulate pass goes from 5.2 to 5.8 TB/s with them (torch's in-place add on
// the same tensors: 5.8 TB/s).
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(const uint4& v, uint4* p) {
  const u32x4_nt x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(p));
}

constexpr int kAccUnroll = 4;

template <class T>
__device__ __forceinline__ uint4 accumulate_chunk(const uint4& mv, const uint4& gv, int score_norm, double& acc_s,
                                                  double& acc_q) {
  constexpr int E = T::kPerChunk;
  float a[E], g[E];
  unpack<T>(mv, a);
  unpack<T>(gv, g);
#pragma unroll
  for (int i = 0; i < E; ++i) a[i] = __fadd_rn(a[i], g[i]);
  const uint4 out = pack<T>(a);
  float st[E];
  unpack<T>(out, st);                 // the stored (rounded) values
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const double v = (double)st[i];
    acc_s += (score_norm == 1) ? fabs(v) : v * v;
    acc_q += v * v;
  }
  return out;
}

template <class T>
__global__ void __launch_bounds__(kRowThreads)
accumulate_score_kernel(void* M, const void* G, int N, int m, long long ld, long long stride, int score_norm,
                        double* score, double* sumsq) {
  __shared__ double sh[kRowThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  uint4* mr = row_chunks<T>(M, (long long)b * stride + (long long)r * ld);
  const uint4* gr = row_chunks<T>(G, (long long)b * stride + (long long)r * ld);
  score += (size_t)b * N;
  if (sumsq) sumsq += (size_t)b * N;
  const int nch = m / T::kPerChunk;
  double acc_s = 0.0, acc_q = 0.0;
  for (int c0 = threadIdx.x; c0 < nch; c0 += kAccUnroll * kRowThreads) {
    uint4 mv[kAccUnroll], gv[kAccUnroll];
#pragma unroll
    for (int u = 0; u < kAccUnroll; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c < nch) {
        mv[u] = load_nt(&mr[c]);
        gv[u] = load_nt(&gr[c]);
      }
    }
#pragma unroll
    for (int u = 0; u < kAccUnroll; ++u) {
      const int c = c0 + u * kRowThreads;
      if (c < nch) store_nt(accumulate_chunk<T>(mv[u], gv[u], score_norm, acc_s, acc_q), &mr[c]);
    }
  }
  const double ts = block_sum_f64(acc_s, sh);
  const double tq = block_sum_f64(acc_q, sh);
  if (threadIdx.x == 0) {
    score[r] = ts;
    if (sumsq) sumsq[r] = tq;
  }
}

hipError_t launch_accumulate_score(void* M, const void* G, gns_dtype dt, int batch, int N, int m, long long ld,
                                   long long stride, int score_norm, double* score, double* sumsq, hipStream_t s) {
  if (N <= 0 || batch <= 0) return hipSuccess;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    hipLaunchKernelGGL(accumulate_score_kernel<T>, dim3(N, batch), dim3(kRowThreads), 0, s, M, G, N, m, ld, stride,
                       score_norm, score, sumsq);
    return hipGetLastError();
  });
}

// ---- top-k rows: radix select on the fp64 bit patterns, then ordered compaction ----
// Scores are >= +0 (sums of |x| or x^2), so their IEEE bit patterns order like the
// values; a NaN score orders above +inf.  Ties at the threshold go to lower indices.
constexpr int kTopkThreads = 1024;

__device__ __forceinline__ unsigned block_excl_scan(unsigned v, unsigned* sh, unsigned& total) {
  // inclusive scan within each wave, then across the 16 wave totals
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  unsigned x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  __syncthreads();
  if (lane == 63) sh[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned run = 0;
    for (int i = 0; i < kTopkThreads / 64; ++i) { const unsigned t = sh[i]; sh[i] = run; run += t; }
    sh[kTopkThreads / 64] = run;
  }
  __syncthreads();
  total = sh[kTopkThreads / 64];
  return sh[w] + x - v;
}

// Keys are staged in LDS when they fit (N <= kTopkLdsKeys), else read from memory.
// The leading bits that every key shares (found from the OR and the AND of all keys)
// are settled at once: scores of one magnitude share their sign, exponent and first
// mantissa bits, and counting them digit by digit would send every key's atomic add
// to one histogram bin.  The remaining bits are resolved 8 at a time from the top;
// the bin holding the k-th largest key is found by one wave: each lane holds 4 bins
// (from the top), a prefix sum over lanes finds the crossing lane.  The search stops
// early once every candidate left is selected.
constexpr int kTopkLdsKeys = 12288;

__device__ __forceinline__ unsigned long long wave_or(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v |= __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ unsigned long long wave_and(unsigned long long v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v &= __shfl_xor(v, off, 64);
  return v;
}

__global__ void __launch_bounds__(kTopkThreads)
topk_kernel(const double* score, int N, int k, int* S) {
  score += (size_t)blockIdx.x * N;     // one workgroup per batch entry
  S += (size_t)blockIdx.x * k;
  constexpr int kWaves = kTopkThreads / 64;
  __shared__ unsigned hist[256];
  __shared__ unsigned scan_sh[kWaves + 1];
  __shared__ unsigned long long red_or[kWaves], red_and[kWaves];
  __shared__ unsigned long long sh_prefix;
  __shared__ unsigned sh_krem, sh_done;
  __shared__ unsigned long long keys_lds[kTopkLdsKeys];
  const unsigned long long* gkey = reinterpret_cast<const unsigned long long*>(score);
  const bool in_lds = N <= kTopkLdsKeys;
  unsigned long long vor = 0, vand = ~0ull;
  if (in_lds) {
    // all of a thread's loads are issued before the first is used, so the staging
    // costs one memory latency instead of one per key
    constexpr int kPer = kTopkLdsKeys / kTopkThreads;
    static_assert(kTopkLdsKeys % kTopkThreads == 0, "whole rounds of keys per thread");
    unsigned long long v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = threadIdx.x + j * kTopkThreads;
      v[j] = i < N ? gkey[i] : 0ull;
    }
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = threadIdx.x + j * kTopkThreads;
      if (i < N) {
        keys_lds[i] = v[j];
        vor |= v[j];
        vand &= v[j];
      }
    }
  } else {
    for (int i = threadIdx.x; i < N; i += kTopkThreads) {
      const unsigned long long kv = gkey[i];
      vor |= kv;
      vand &= kv;
    }
  }
  vor = wave_or(vor);
  vand = wave_and(vand);
  if ((threadIdx.x & 63) == 0) {
    red_or[threadIdx.x >> 6] = vor;
    red_and[threadIdx.x >> 6] = vand;
  }
  __syncthreads();
  vor = 0;
  vand = ~0ull;
  for (int w = 0; w < kWaves; ++w) {
    vor |= red_or[w];
    vand &= red_and[w];
  }
  const unsigned long long* key = in_lds ? keys_lds : gkey;
  // bits 63 .. nbits are the same in every key; they form the starting prefix
  const unsigned long long differ = vor ^ vand;
  const int nbits = differ ? 64 - __clzll((long long)differ) : 0;
  unsigned long long mask = nbits == 64 ? 0ull : ~((1ull << nbits) - 1ull);
  unsigned long long prefix = vand & mask;
  unsigned krem = (unsigned)k;
  for (int top = nbits; top > 0;) {
    const int width = top < 8 ? top : 8;
    const int shift = top - width;
    const unsigned dmask = (1u << width) - 1u;
    for (int i = threadIdx.x; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += kTopkThreads) {
      const unsigned long long kv = key[i];
      if ((kv & mask) == prefix) atomicAdd(&hist[(unsigned)(kv >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 255-4l .. 252-4l; counts above a lane's bins by prefix sum
      // (bins at or above 2^width stay empty)
      const int lane = threadIdx.x;
      unsigned c[4], local = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hist[255 - 4 * lane - q];
        local += c[q];
      }
      unsigned incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const unsigned excl = incl - local;
      // the crossing lane: the k-th largest candidate lies in one of its bins
      // (the last lane always crosses: krem never exceeds the candidate count)
      if (excl < krem && (krem <= incl || lane == 63)) {
        unsigned above = excl, cnt = c[3];
        int bin = 255 - 4 * lane - 3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int b = 255 - 4 * lane - q;
          if (above + c[q] >= krem || b == 0) {
            bin = b;
            cnt = c[q];
            break;
          }
          above += c[q];
        }
        sh_prefix = prefix | ((unsigned long long)bin << shift);
        sh_krem = krem - above;
        sh_done = (cnt == krem - above) ? 1u : 0u;   // every key of the bin is taken
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    krem = sh_krem;
    mask |= (unsigned long long)dmask << shift;
    top = sh_done ? 0 : shift;
    __syncthreads();
  }
  // Keys whose masked bits exceed the prefix are above every candidate and are all
  // taken; of the candidates (masked bits equal to the prefix) the first krem by index
  // are taken.  With all 64 bits resolved that is: every key above the k-th largest
  // and the lowest-index keys equal to it.  Each thread owns one contiguous range of
  // indices, so a block-wide scan of the counts gives ascending output positions.
  const int per = (N + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(N, (int)threadIdx.x * per), hi = min(N, lo + per);
  unsigned n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi; ++i) {
    const unsigned long long kv = key[i] & mask;
    n_gt += kv > prefix ? 1u : 0u;
    n_eq += kv == prefix ? 1u : 0u;
  }
  unsigned eq_total;
  const unsigned eq_before = block_excl_scan(n_eq, scan_sh, eq_total);
  const unsigned eq_take = eq_before >= krem ? 0u : min(n_eq, krem - eq_before);
  unsigned sel_total;
  unsigned pos = block_excl_scan(n_gt + eq_take, scan_sh, sel_total);
  unsigned eq_seen = 0;
  for (int i = lo; i < hi; ++i) {
    const unsigned long long kv = key[i] & mask;
    bool take = kv > prefix;
    if (kv == prefix) take = eq_seen++ < eq_take;
    if (take) {
      if (pos < (unsigned)k) S[pos] = i;
      ++pos;
    }
  }
}

hipError_t launch_topk(const double* score, int batch, int N, int k, int* S, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kTopkThreads), 0, s, score, N, k, S);
  return hipGetLastError();
}

// ---- X[r] = M[S[r]]; M[S[r]] <- fl(mu * M[S[r]]) -------------------------------------
// X (state type) holds kx >= k rows per batch entry: rows k .. kx-1 (the padding of the
// submatrix to a whole number of 8-row groups) are written as zeros.
// Xh (bf16 state only, nullable): also the fp16 copy fl16(fl32(fl32(hP s[b]) x)) of the
// same rows, with X's row stride -- the restart product's operand, so that product
// reads fp16 instead of converting bf16 on every load (the same two roundings as that
// conversion, so the values are bitwise those it would form).
template <class T>
__global__ void __launch_bounds__(kRowThreads)
gather_feedback_kernel(void* M, int N, int m, long long ld, long long stride, const int* S, int k, int kx,
                       float mu_host, const float* dev_scalars, void* X, long long ldx, void* Xh,
                       const float* hs, float hP) {
  constexpr int E = T::kPerChunk;
  constexpr bool kHalfCopy = T::kId == GNS_BF16;
  const int r = blockIdx.x, b = blockIdx.y;
  const float mu = dev_scalars ? dev_scalars[2] : mu_host;
  const int src = r < k ? S[(size_t)b * k + r] : -1;
  uint4* xr = row_chunks<T>(X, ((long long)b * kx + r) * ldx);
  uint4* hr = (kHalfCopy && Xh) ? row_chunks<TF16>(Xh, ((long long)b * kx + r) * ldx) : nullptr;
  const int nch = m / E;
  if (src < 0 || src >= N) {           // padding row, or an index out of range: a zero row of X, M untouched
    for (int c = threadIdx.x; c < nch; c += kRowThreads) {
      xr[c] = make_uint4(0u, 0u, 0u, 0u);
      if (hr) hr[c] = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  const float hmul = hr ? __fmul_rn(hP, hs[b]) : 0.0f;
  uint4* mr = row_chunks<T>(M, (long long)b * stride + (long long)src * ld);
  for (int c = threadIdx.x; c < nch; c += kRowThreads) {
    const uint4 v = load_nt(&mr[c]);
    xr[c] = v;
    float x[E];
    unpack<T>(v, x);
    if constexpr (kHalfCopy) {
      if (hr) {
        float h[E];
#pragma unroll
        for (int i = 0; i < E; ++i) h[i] = __fmul_rn(x[i], hmul);
        hr[c] = pack<TF16>(h);
      }
    }
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = __fmul_rn(mu, x[i]);
    store_nt(pack<T>(x), &mr[c]);
  }
}

hipError_t launch_gather_feedback(void* M, gns_dtype dt, int batch, int N, int m, long long ld, long long stride,
                                  const int* S, int k, int kx, float mu, const float* dev_scalars, void* X,
                                  long long ldx, hipStream_t s, void* Xh, const float* hs, float hP) {
  if (k <= 0 || batch <= 0) return hipSuccess;
  if (kx < k) return hipErrorInvalidValue;
  if (Xh && (dt != GNS_BF16 || !hs)) return hipErrorInvalidValue;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    hipLaunchKernelGGL(gather_feedback_kernel<T>, dim3(kx, batch), dim3(kRowThreads), 0, s, M, N, m, ld, stride, S,
                       k, kx, mu, dev_scalars, X, ldx, Xh, hs, hP);
    return hipGetLastError();
  });
}

// E elements of O (type TO) from p, widened to fp32: whole 16-byte chunks, or half of
// one (4 fp32 state elements against a 16-bit O).
template <class TO, int E>
__device__ __forceinline__ void load_o(const uint8_t* p, float (&o)[E]) {
  constexpr int PER = TO::kPerChunk;
  if constexpr (E >= PER) {
#pragma unroll
    for (int q = 0; q < E / PER; ++q) {
      const uint4 c = reinterpret_cast<const uint4*>(p)[q];
#pragma unroll
      for (int i = 0; i < PER; ++i) o[q * PER + i] = TO::to_f32(elem_bits<TO>(c, i));
    }
  } else {
    const uint2 h = *reinterpret_cast<const uint2*>(p);
    const uint4 c = make_uint4(h.x, h.y, 0u, 0u);
#pragma unroll
    for (int i = 0; i < E; ++i) o[i] = TO::to_f32(elem_bits<TO>(c, i));
  }
}

// ---- weight decay + selected-row update, one rounding per element --------------------
template <class T, class TO>
__global__ void __launch_bounds__(kRowThreads)
apply_update_kernel(void* W, int N, int m, long long ld, long long stride, const int* S, int k, const void* O,
                    long long ldo, long long so, float lr_host, float wd_host, const float* dev_scalars, int all_rows,
                    void* Mfb, float mu_host) {
  constexpr int E = T::kPerChunk;
  const float lr = dev_scalars ? dev_scalars[0] : lr_host;
  const float wd = dev_scalars ? dev_scalars[1] : wd_host;
  const float mu = dev_scalars ? dev_scalars[2] : mu_host;
  const int d_over = blockIdx.x, b = blockIdx.y;
  S += (size_t)b * k;
  const uint8_t* Ob = static_cast<const uint8_t*>(O) + (size_t)b * so * TO::kBytes;
  int row, oi;
  if (all_rows) {
    row = d_over;
    // binary search for row in the ascending list S
    int lo = 0, hi = k - 1;
    oi = -1;
    while (lo <= hi) {
      const int mid = (lo + hi) >> 1;
      const int v = S[mid];
      if (v == row) { oi = mid; break; }
      if (v < row) lo = mid + 1; else hi = mid - 1;
    }
  } else {
    oi = d_over;
    row = S[oi];
    if (row < 0 || row >= N) return;
  }
  // an unselected row without weight decay keeps its bits (d = 1 would not change it)
  if (oi < 0 && wd == 0.0f) return;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  uint4* wr = row_chunks<T>(W, (long long)b * stride + (long long)row * ld);
  // error feedback on the same selected row, in the same pass: M[S[oi]] <- fl(mu
  // M[S[oi]]), the arithmetic of gather_feedback_kernel (the Gram products have read
  // these rows already); W and M chunks are loaded together for more bytes in flight
  uint4* mr = (Mfb && oi >= 0) ? row_chunks<T>(Mfb, (long long)b * stride + (long long)row * ld) : nullptr;
  for (int c = threadIdx.x; c < m / E; c += kRowThreads) {
    const uint4 v = load_nt(&wr[c]);
    const uint4 mv = mr ? load_nt(&mr[c]) : make_uint4(0u, 0u, 0u, 0u);
    float o[E];
    if (oi >= 0) load_o<TO, E>(Ob + ((size_t)oi * ldo + (size_t)c * E) * TO::kBytes, o);
    float x[E];
    unpack<T>(v, x);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      float y = __fmul_rn(d, x[i]);
      if (oi >= 0) y = __fsub_rn(y, __fmul_rn(lr, o[i]));
      x[i] = y;
    }
    store_nt(pack<T>(x), &wr[c]);
    if (mr) {
      float mm[E];
      unpack<T>(mv, mm);
#pragma unroll
      for (int i = 0; i < E; ++i) mm[i] = __fmul_rn(mu, mm[i]);
      store_nt(pack<T>(mm), &mr[c]);
    }
  }
}

hipError_t launch_apply_update(void* W, gns_dtype dt, int batch, int N, int m, long long ld, long long stride,
                               const int* S, int k, const void* O, gns_dtype o_dtype, long long ldo, long long so,
                               float lr, float wd, const float* dev_scalars, hipStream_t s, void* Mfb, float mu) {
  // with the weight decay on the device the host cannot tell whether unselected rows
  // decay: cover all rows (each unselected row returns at once when wd == 0)
  const int all_rows = (dev_scalars || wd != 0.0f) ? 1 : 0;
  const int blocks = all_rows ? N : k;
  if (blocks <= 0 || batch <= 0) return hipSuccess;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    return with_state_type(o_dtype, [&](auto otag) {
      using TO = decltype(otag);
      clear_stale_error();
      hipLaunchKernelGGL((apply_update_kernel<T, TO>), dim3(blocks, batch), dim3(kRowThreads), 0, s, W, N, m, ld,
                         stride, S, k, O, ldo, so, lr, wd, dev_scalars, all_rows, Mfb, mu);
      return hipGetLastError();
    });
  });
}

// ---- s = 1 / (sqrt(sum_i sumsq[S[i]]) + eps) ------------------------------------------
__global__ void __launch_bounds__(kRowThreads)
selected_sumsq_kernel(const double* sumsq, const int* S, int k, int N, float eps, float* s_out) {
  __shared__ double sh[kRowThreads / 64];
  sumsq += (size_t)blockIdx.x * N;     // one workgroup per batch entry
  S += (size_t)blockIdx.x * k;
  s_out += blockIdx.x;
  const int per = (k + kRowThreads - 1) / kRowThreads;
  const int lo = min(k, (int)threadIdx.x * per), hi = min(k, lo + per);
  // each thread sums its range in index order; the loads of 8 terms are issued
  // before the first is added
  constexpr int kUnroll = 8;
  double acc = 0.0;
  for (int i0 = lo; i0 < hi; i0 += kUnroll) {
    int r[kUnroll];
    double v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = i0 + u < hi ? S[i0 + u] : -1;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = (r[u] >= 0 && r[u] < N) ? sumsq[r[u]] : 0.0;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (r[u] >= 0 && r[u] < N) acc += v[u];
  }
  const double t = block_sum_f64(acc, sh);
  if (threadIdx.x == 0) s_out[0] = (float)(1.0 / (sqrt(t) + (double)eps));
}

hipError_t launch_selected_sumsq(const double* sumsq, const int* S, int batch, int k, int N, float eps, float* s_out,
                                 hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(selected_sumsq_kernel, dim3(batch), dim3(kRowThreads), 0, s, sumsq, S, k, N, eps, s_out);
  return hipGetLastError();
}

// ---- column selection: scores, gather + error feedback, update, decay -------------
// The same rule as the row kernels with the roles of rows and columns swapped: the
// step subsamples columns of the row-major N x m state.  Tiles of 64 selected columns
// x 64 rows go through LDS so that X^T (row j = column S[j]) and O (k x N) are read
// and written in 16-byte row vectors, while a wave's 64 lanes touch the 64 selected
// columns of one state row (ascending, so a few cache lines per access).
constexpr int kColThreads = 256;
constexpr int kColRowsPerPart = 128;   // rows summed into one partial column score
constexpr int kColTile = 64;

// Element storage of T in LDS tiles: its raw bits, rows padded by 4 bytes so a wave's
// 64 lanes reading one tile column hit distinct banks.
template <class T>
struct ColTile {
  using Bits = typename std::conditional<T::kBytes == 4, uint32_t, uint16_t>::type;
  static constexpr int kPad = 4 / T::kBytes;
  Bits v[kColTile][kColTile + kPad];
};

// M <- fl(M + G) and, per column, fp64 sums over a block of kColRowsPerPart rows:
// part_s[rb][col] (|x| or x^2 by score_norm) and part_q[rb][col] (x^2).  Thread =
// one 16-byte chunk of columns; rows in ascending order, four loaded at a time.
template <class T>
__global__ void __launch_bounds__(kColThreads)
accumulate_colscore_kernel(void* M, const void* G, int N, int m, long long ld, int score_norm, double* part_s,
                           double* part_q) {
  constexpr int E = T::kPerChunk;
  const int c = blockIdx.x * kColThreads + threadIdx.x;
  const int nch = m / E;
  if (c >= nch) return;
  const int rb = blockIdx.y;
  const int i0 = rb * kColRowsPerPart, i1 = min(N, i0 + kColRowsPerPart);
  double s[E], q[E];
#pragma unroll
  for (int e = 0; e < E; ++e) s[e] = q[e] = 0.0;
  constexpr int U = 4;
  for (int ib = i0; ib < i1; ib += U) {
    uint4 mv[U], gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = ib + u;
      if (i < i1) {
        mv[u] = load_nt(row_chunks<T>(M, (long long)i * ld) + c);
        gv[u] = load_nt(row_chunks<T>(G, (long long)i * ld) + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = ib + u;
      if (i >= i1) continue;
      float a[E], g[E];
      unpack<T>(mv[u], a);
      unpack<T>(gv[u], g);
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] = __fadd_rn(a[e], g[e]);
      const uint4 out = pack<T>(a);
      float st[E];
      unpack<T>(out, st);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double v = (double)st[e];
        s[e] += (score_norm == 1) ? fabs(v) : v * v;
        q[e] += v * v;
      }
      store_nt(out, row_chunks<T>(M, (long long)i * ld) + c);
    }
  }
  double* ps = part_s + (size_t)rb * m + (size_t)E * c;
  double* pq = part_q + (size_t)rb * m + (size_t)E * c;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    ps[e] = s[e];
    pq[e] = q[e];
  }
}

// score[col], sumsq[col]: the partials of the row blocks added in block order
__global__ void __launch_bounds__(kColThreads)
reduce_colscore_kernel(const double* part_s, const double* part_q, int nparts, int m, double* score, double* sumsq) {
  const int col = blockIdx.x * kColThreads + threadIdx.x;
  if (col >= m) return;
  double s = 0.0, q = 0.0;
  for (int rb = 0; rb < nparts; ++rb) {
    s += part_s[(size_t)rb * m + col];
    q += part_q[(size_t)rb * m + col];
  }
  score[col] = s;
  sumsq[col] = q;
}

// Xt[j, i] = M[i, S[j]] (Xt: k x N, row stride ldx) and M[i, S[j]] <- fl(mu M[i, S[j]]).
// An index S[j] outside [0, m) gives a zero row of Xt and touches M nowhere.
template <class T>
__global__ void __launch_bounds__(kColThreads)
gather_cols_feedback_kernel(void* M, int N, int m, long long ld, const int* S, int k, int kx, float mu, void* Xt,
                            long long ldx) {
  using Bits = typename ColTile<T>::Bits;
  __shared__ __align__(16) ColTile<T> tile;    // [j][i]
  const int j0 = blockIdx.x * kColTile, i0 = blockIdx.y * kColTile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = j0 + lane;
  const int col = (j < k) ? S[j] : -1;
  const bool ok = col >= 0 && col < m;
  for (int r = w; r < kColTile; r += kColThreads / 64) {
    const int i = i0 + r;
    Bits x = 0;
    if (ok && i < N) {
      Bits* p = static_cast<Bits*>(M) + (size_t)i * ld + col;
      x = *p;
      *p = (Bits)round_to<T>(__fmul_rn(mu, T::to_f32(x)));
    }
    tile.v[lane][r] = x;
  }
  __syncthreads();
  // row jr of the tile, 16 values from column 16 q, in 16-byte stores; rows k .. kx-1
  // (padding to a whole number of 8-row groups) are written as zeros
  const int jr = threadIdx.x >> 2, qd = threadIdx.x & 3;
  if (j0 + jr >= kx) return;
  const uint32_t* t32 = reinterpret_cast<const uint32_t*>(&tile.v[jr][0]);
  constexpr int E = T::kPerChunk;
#pragma unroll
  for (int h = 0; h < 16 / E; ++h) {
    const int a = 16 * qd + E * h;                   // tile column of the chunk's first element
    if (i0 + a >= N) continue;                       // N % 8 == 0: a chunk is all in or all out
    const int w0 = a * T::kBytes / 4;
    const uint4 v = make_uint4(t32[w0], t32[w0 + 1], t32[w0 + 2], t32[w0 + 3]);
    *row_chunks<T>(Xt, (long long)(j0 + jr) * ldx + i0 + a) = v;
  }
}

// W[i, S[j]] <- fl(fl32(d W) - fl32(lr O[j, i])), d = fl32(1 - fl32(lr wd)); O: k x N
// (row stride ldo, state type).  An index S[j] outside [0, m) updates nothing.
template <class T>
__global__ void __launch_bounds__(kColThreads)
update_cols_kernel(void* W, int N, int m, long long ld, const int* S, int k, const void* O, long long ldo, float lr,
                   float wd) {
  using Bits = typename ColTile<T>::Bits;
  __shared__ __align__(16) ColTile<T> tile;    // [j][i]
  constexpr int E = T::kPerChunk;
  const int j0 = blockIdx.x * kColTile, i0 = blockIdx.y * kColTile;
  {
    const int jr = threadIdx.x >> 2, qd = threadIdx.x & 3;
    uint32_t* t32 = reinterpret_cast<uint32_t*>(&tile.v[jr][0]);
#pragma unroll
    for (int h = 0; h < 16 / E; ++h) {
      const int a = 16 * qd + E * h;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j0 + jr < k && i0 + a < N) v = *row_chunks<T>(O, (long long)(j0 + jr) * ldo + i0 + a);
      const int w0 = a * T::kBytes / 4;
      t32[w0] = v.x; t32[w0 + 1] = v.y; t32[w0 + 2] = v.z; t32[w0 + 3] = v.w;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = j0 + lane;
  const int col = (j < k) ? S[j] : -1;
  if (col < 0 || col >= m) return;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  for (int r = w; r < kColTile; r += kColThreads / 64) {
    const int i = i0 + r;
    if (i >= N) break;
    Bits* p = static_cast<Bits*>(W) + (size_t)i * ld + col;
    const float x = T::to_f32(*p);
    const float o = T::to_f32(tile.v[lane][r]);
    *p = (Bits)round_to<T>(__fsub_rn(__fmul_rn(d, x), __fmul_rn(lr, o)));
  }
}

// mark[col] = 1 for the selected columns (after clear_marks): the decay pass skips them
__global__ void __launch_bounds__(kColThreads) clear_marks_kernel(uint8_t* mark, int m) {
  const int c = blockIdx.x * kColThreads + threadIdx.x;
  if (c < m) mark[c] = 0;
}
__global__ void __launch_bounds__(kColThreads) set_marks_kernel(uint8_t* mark, int m, const int* S, int k) {
  const int j = blockIdx.x * kColThreads + threadIdx.x;
  if (j >= k) return;
  const int col = S[j];
  if (col >= 0 && col < m) mark[col] = 1;
}

// W[i, c] <- fl(fl32(d W[i, c])) for every column c not marked (decoupled weight decay);
// marked columns keep their bits
template <class T>
__global__ void __launch_bounds__(kColThreads)
decay_unmarked_kernel(void* W, int N, int m, long long ld, const uint8_t* mark, float lr, float wd) {
  constexpr int E = T::kPerChunk;
  const int c = blockIdx.x * kColThreads + threadIdx.x;   // 16-byte chunk
  if (c >= m / E) return;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  for (int i = blockIdx.y; i < N; i += gridDim.y) {
    uint4* p = row_chunks<T>(W, (long long)i * ld) + c;
    const uint4 v = load_nt(p);
    uint32_t nb[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t bits = elem_bits<T>(v, e);
      nb[e] = mark[E * c + e] ? bits : round_to<T>(__fmul_rn(d, T::to_f32(bits)));
    }
    store_nt(pack_bits<T>(nb), p);
  }
}

size_t dion3_cols_partials(int N) { return (size_t)((N + kColRowsPerPart - 1) / kColRowsPerPart); }

hipError_t launch_accumulate_colscore(void* M, const void* G, gns_dtype dt, int N, int m, long long ld,
                                      int score_norm, double* part_s, double* part_q, double* score, double* sumsq,
                                      hipStream_t s) {
  if (N <= 0 || m <= 0) return hipSuccess;
  const int nparts = (int)dion3_cols_partials(N);
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    const int nch = m / T::kPerChunk;
    hipLaunchKernelGGL(accumulate_colscore_kernel<T>, dim3((nch + kColThreads - 1) / kColThreads, nparts),
                       dim3(kColThreads), 0, s, M, G, N, m, ld, score_norm, part_s, part_q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(reduce_colscore_kernel, dim3((m + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s,
                       part_s, part_q, nparts, m, score, sumsq);
    return hipGetLastError();
  });
}

hipError_t launch_gather_cols_feedback(void* M, gns_dtype dt, int N, int m, long long ld, const int* S, int k, int kx,
                                       float mu, void* Xt, long long ldx, hipStream_t s) {
  if (k <= 0 || N <= 0) return hipSuccess;
  if (kx < k) return hipErrorInvalidValue;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    hipLaunchKernelGGL(gather_cols_feedback_kernel<T>,
                       dim3((kx + kColTile - 1) / kColTile, (N + kColTile - 1) / kColTile), dim3(kColThreads), 0, s, M,
                       N, m, ld, S, k, kx, mu, Xt, ldx);
    return hipGetLastError();
  });
}

hipError_t launch_update_cols(void* W, gns_dtype dt, int N, int m, long long ld, const int* S, int k, const void* O,
                              long long ldo, float lr, float wd, uint8_t* mark, hipStream_t s) {
  if (k <= 0 || N <= 0) return hipSuccess;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    if (wd != 0.0f) {
      const int nch = m / T::kPerChunk;
      hipLaunchKernelGGL(clear_marks_kernel, dim3((m + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s, mark,
                         m);
      hipLaunchKernelGGL(set_marks_kernel, dim3((k + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s, mark, m,
                         S, k);
      hipLaunchKernelGGL(decay_unmarked_kernel<T>, dim3((nch + kColThreads - 1) / kColThreads, std::min(N, 4096)),
                         dim3(kColThreads), 0, s, W, N, m, ld, mark, lr, wd);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(update_cols_kernel<T>, dim3((k + kColTile - 1) / kColTile, (N + kColTile - 1) / kColTile),
                       dim3(kColThreads), 0, s, W, N, m, ld, S, k, O, ldo, lr, wd);
    return hipGetLastError();
  });
}

}  // namespace gns
