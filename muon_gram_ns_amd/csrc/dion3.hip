// Dion3 element-wise and selection kernels (all HBM- or latency-bound).
//
// The update rule ("Dion3: Full-Stack Orthogonal Updates", paper.rainbus.top,
// 方法步骤详情 (3), Algorithm 4): M <- M + G; pick the k rows of largest norm;
// orthogonalise that submatrix; decay all weights by (1 - lr wd) and subtract
// lr O from the selected weight rows; decay only the selected momentum rows by mu
// (error feedback, same page, 前置知识).
//
// Rounding model (the pages do not fix it; this is the reading the oracle emulates):
// W, M, G are bf16; each stored value is rounded once, to nearest even, from fp32
// results computed op by op.  This file is compiled with -ffp-contract=off and uses
// explicit __fmul_rn/__fsub_rn so no multiply-add is fused.  Row scores accumulate
// in fp64 (the per-element terms are exact in fp64).
#include "common.h"
#include "internal.h"

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

// ---- M <- bf16(M + G); per-row score and sum of squares ---------------------------
// One workgroup per row.  Each thread takes chunks c, c+256, c+512, ... of 8 values;
// four chunks' loads are issued before any is used (more bytes in flight per wave),
// and the chunks are then summed in that same order, so each thread's fp64 sums do
// not depend on the unrolling.
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

__device__ __forceinline__ uint4 accumulate_chunk(uint4 mv, const uint4& gv, int score_norm, double& acc_s,
                                                  double& acc_q) {
  uint32_t* mw = reinterpret_cast<uint32_t*>(&mv);
  const uint32_t* gw = reinterpret_cast<const uint32_t*>(&gv);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t out = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float a = bf16_bits_to_f32((mw[i] >> (16 * h)) & 0xffffu);
      const float g = bf16_bits_to_f32((gw[i] >> (16 * h)) & 0xffffu);
      const uint32_t nb = f32_to_bf16_bits(__fadd_rn(a, g));
      out |= nb << (16 * h);
      const double v = (double)bf16_bits_to_f32(nb);
      acc_s += (score_norm == 1) ? fabs(v) : v * v;
      acc_q += v * v;
    }
    mw[i] = out;
  }
  return mv;
}

__global__ void __launch_bounds__(kRowThreads)
accumulate_score_kernel(uint16_t* M, const uint16_t* G, int N, int m, long long ld, long long stride, int score_norm,
                        double* score, double* sumsq) {
  __shared__ double sh[kRowThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  uint4* mr = reinterpret_cast<uint4*>(M + (size_t)b * stride + (size_t)r * ld);
  const uint4* gr = reinterpret_cast<const uint4*>(G + (size_t)b * stride + (size_t)r * ld);
  score += (size_t)b * N;
  if (sumsq) sumsq += (size_t)b * N;
  const int nch = m / 8;
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
      if (c < nch) store_nt(accumulate_chunk(mv[u], gv[u], score_norm, acc_s, acc_q), &mr[c]);
    }
  }
  const double ts = block_sum_f64(acc_s, sh);
  const double tq = block_sum_f64(acc_q, sh);
  if (threadIdx.x == 0) {
    score[r] = ts;
    if (sumsq) sumsq[r] = tq;
  }
}

hipError_t launch_accumulate_score(uint16_t* M, const uint16_t* G, int batch, int N, int m, long long ld,
                                   long long stride, int score_norm, double* score, double* sumsq, hipStream_t s) {
  if (N <= 0 || batch <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(accumulate_score_kernel, dim3(N, batch), dim3(kRowThreads), 0, s, M, G, N, m, ld, stride,
                     score_norm, score, sumsq);
  return hipGetLastError();
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

// ---- X[r] = M[S[r]]; M[S[r]] <- bf16(mu * M[S[r]]) ----------------------------------
// X holds kx >= k rows per batch entry: rows k .. kx-1 (the padding of the submatrix
// to a whole number of 8-row groups) are written as zeros.
__global__ void __launch_bounds__(kRowThreads)
gather_feedback_kernel(uint16_t* M, int N, int m, long long ld, long long stride, const int* S, int k, int kx,
                       float mu_host, const float* dev_scalars, uint16_t* X, long long ldx) {
  const int r = blockIdx.x, b = blockIdx.y;
  const float mu = dev_scalars ? dev_scalars[2] : mu_host;
  const int src = r < k ? S[(size_t)b * k + r] : -1;
  uint4* xr = reinterpret_cast<uint4*>(X + ((size_t)b * kx + r) * ldx);
  if (src < 0 || src >= N) {           // padding row, or an index out of range: a zero row of X, M untouched
    for (int c = threadIdx.x; c < m / 8; c += kRowThreads) xr[c] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  uint4* mr = reinterpret_cast<uint4*>(M + (size_t)b * stride + (size_t)src * ld);
  for (int c = threadIdx.x; c < m / 8; c += kRowThreads) {
    uint4 v = load_nt(&mr[c]);
    xr[c] = v;
    uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = f32_to_bf16_bits(__fmul_rn(mu, bf16_bits_to_f32(w[i] & 0xffffu)));
      const uint32_t hi = f32_to_bf16_bits(__fmul_rn(mu, bf16_bits_to_f32(w[i] >> 16)));
      w[i] = lo | (hi << 16);
    }
    store_nt(v, &mr[c]);
  }
}

hipError_t launch_gather_feedback(uint16_t* M, int batch, int N, int m, long long ld, long long stride, const int* S,
                                  int k, int kx, float mu, const float* dev_scalars, uint16_t* X, long long ldx,
                                  hipStream_t s) {
  if (k <= 0 || batch <= 0 || kx < k) return k <= 0 || batch <= 0 ? hipSuccess : hipErrorInvalidValue;
  clear_stale_error();
  hipLaunchKernelGGL(gather_feedback_kernel, dim3(kx, batch), dim3(kRowThreads), 0, s, M, N, m, ld, stride, S, k, kx,
                     mu, dev_scalars, X, ldx);
  return hipGetLastError();
}

// ---- weight decay + selected-row update, one rounding per element --------------------
template <bool O_F32>
__global__ void __launch_bounds__(kRowThreads)
apply_update_kernel(uint16_t* W, int N, int m, long long ld, long long stride, const int* S, int k, const void* O,
                    long long ldo, long long so, float lr_host, float wd_host, const float* dev_scalars, int all_rows,
                    uint16_t* Mfb, float mu_host) {
  const float lr = dev_scalars ? dev_scalars[0] : lr_host;
  const float wd = dev_scalars ? dev_scalars[1] : wd_host;
  const float mu = dev_scalars ? dev_scalars[2] : mu_host;
  const int d_over = blockIdx.x, b = blockIdx.y;
  W += (size_t)b * stride;
  if (Mfb) Mfb += (size_t)b * stride;
  S += (size_t)b * k;
  O = reinterpret_cast<const uint8_t*>(O) + (size_t)b * so * (O_F32 ? 4 : 2);
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
  uint4* wr = reinterpret_cast<uint4*>(W + (size_t)row * ld);
  // error feedback on the same selected row, in the same pass: M[S[oi]] <- bf16(mu
  // M[S[oi]]), the arithmetic of gather_feedback_kernel (the Gram products have read
  // these rows already); W and M chunks are loaded together for more bytes in flight
  uint4* mr = (Mfb && oi >= 0) ? reinterpret_cast<uint4*>(Mfb + (size_t)row * ld) : nullptr;
  for (int c = threadIdx.x; c < m / 8; c += kRowThreads) {
    uint4 v = load_nt(&wr[c]);
    uint4 mv = mr ? load_nt(&mr[c]) : make_uint4(0u, 0u, 0u, 0u);
    uint32_t* w = reinterpret_cast<uint32_t*>(&v);
    float o[8];
    if (oi >= 0) {
      if constexpr (O_F32) {
        const float4* op = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(O) + (size_t)oi * ldo + (size_t)c * 8);
        const float4 a = op[0], b = op[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
      } else {
        const uint4 q = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(O) + (size_t)oi * ldo)[c];
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(&q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = bf16_bits_to_f32(qw[i] & 0xffffu);
          o[2 * i + 1] = bf16_bits_to_f32(qw[i] >> 16);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t out = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float x = bf16_bits_to_f32((w[i] >> (16 * h)) & 0xffffu);
        float y = __fmul_rn(d, x);
        if (oi >= 0) y = __fsub_rn(y, __fmul_rn(lr, o[2 * i + h]));
        out |= f32_to_bf16_bits(y) << (16 * h);
      }
      w[i] = out;
    }
    store_nt(v, &wr[c]);
    if (mr) {
      uint32_t* mw = reinterpret_cast<uint32_t*>(&mv);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = f32_to_bf16_bits(__fmul_rn(mu, bf16_bits_to_f32(mw[i] & 0xffffu)));
        const uint32_t hi = f32_to_bf16_bits(__fmul_rn(mu, bf16_bits_to_f32(mw[i] >> 16)));
        mw[i] = lo | (hi << 16);
      }
      store_nt(mv, &mr[c]);
    }
  }
}

hipError_t launch_apply_update(uint16_t* W, int batch, int N, int m, long long ld, long long stride, const int* S, int k,
                               const void* O, gns_dtype o_dtype, long long ldo, long long so, float lr, float wd,
                               const float* dev_scalars, hipStream_t s, uint16_t* Mfb, float mu) {
  // with the weight decay on the device the host cannot tell whether unselected rows
  // decay: cover all rows (each unselected row returns at once when wd == 0)
  const int all_rows = (dev_scalars || wd != 0.0f) ? 1 : 0;
  const int blocks = all_rows ? N : k;
  if (blocks <= 0 || batch <= 0) return hipSuccess;
  clear_stale_error();
  if (o_dtype == GNS_F32)
    hipLaunchKernelGGL(apply_update_kernel<true>, dim3(blocks, batch), dim3(kRowThreads), 0, s, W, N, m, ld, stride, S,
                       k, O, ldo, so, lr, wd, dev_scalars, all_rows, Mfb, mu);
  else
    hipLaunchKernelGGL(apply_update_kernel<false>, dim3(blocks, batch), dim3(kRowThreads), 0, s, W, N, m, ld, stride,
                       S, k, O, ldo, so, lr, wd, dev_scalars, all_rows, Mfb, mu);
  return hipGetLastError();
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

// M <- bf16(M + G) and, per column, fp64 sums over a block of kColRowsPerPart rows:
// part_s[rb][col] (|x| or x^2 by score_norm) and part_q[rb][col] (x^2).  Thread =
// one 16-byte chunk (8 columns); rows in ascending order, four loaded at a time.
__global__ void __launch_bounds__(kColThreads)
accumulate_colscore_kernel(uint16_t* M, const uint16_t* G, int N, int m, long long ld, int score_norm,
                           double* part_s, double* part_q) {
  const int c = blockIdx.x * kColThreads + threadIdx.x;
  const int nch = m / 8;
  if (c >= nch) return;
  const int rb = blockIdx.y;
  const int i0 = rb * kColRowsPerPart, i1 = min(N, i0 + kColRowsPerPart);
  double s[8], q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = q[e] = 0.0;
  constexpr int U = 4;
  for (int ib = i0; ib < i1; ib += U) {
    uint4 mv[U], gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = ib + u;
      if (i < i1) {
        mv[u] = load_nt(reinterpret_cast<const uint4*>(M + (size_t)i * ld) + c);
        gv[u] = load_nt(reinterpret_cast<const uint4*>(G + (size_t)i * ld) + c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = ib + u;
      if (i >= i1) continue;
      uint32_t* mw = reinterpret_cast<uint32_t*>(&mv[u]);
      const uint32_t* gw = reinterpret_cast<const uint32_t*>(&gv[u]);
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t out = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float a = bf16_bits_to_f32((mw[e2] >> (16 * h)) & 0xffffu);
          const float g = bf16_bits_to_f32((gw[e2] >> (16 * h)) & 0xffffu);
          const uint32_t nb = f32_to_bf16_bits(__fadd_rn(a, g));
          out |= nb << (16 * h);
          const double v = (double)bf16_bits_to_f32(nb);
          const int e = 2 * e2 + h;
          s[e] += (score_norm == 1) ? fabs(v) : v * v;
          q[e] += v * v;
        }
        mw[e2] = out;
      }
      store_nt(mv[u], reinterpret_cast<uint4*>(M + (size_t)i * ld) + c);
    }
  }
  double* ps = part_s + (size_t)rb * m + 8 * (size_t)c;
  double* pq = part_q + (size_t)rb * m + 8 * (size_t)c;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
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

// Xt[j, i] = M[i, S[j]] (Xt: k x N, row stride ldx) and M[i, S[j]] <- bf16(mu M[i, S[j]]).
// An index S[j] outside [0, m) gives a zero row of Xt and touches M nowhere.
__global__ void __launch_bounds__(kColThreads)
gather_cols_feedback_kernel(uint16_t* M, int N, int m, long long ld, const int* S, int k, int kx, float mu,
                            uint16_t* Xt, long long ldx) {
  __shared__ __align__(16) uint16_t tile[kColTile][kColTile + 2];   // [j][i]; rows of 132 bytes
  const int j0 = blockIdx.x * kColTile, i0 = blockIdx.y * kColTile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = j0 + lane;
  const int col = (j < k) ? S[j] : -1;
  const bool ok = col >= 0 && col < m;
  for (int r = w; r < kColTile; r += kColThreads / 64) {
    const int i = i0 + r;
    uint16_t x = 0;
    if (ok && i < N) {
      uint16_t* p = M + (size_t)i * ld + col;
      x = *p;
      *p = (uint16_t)f32_to_bf16_bits(__fmul_rn(mu, bf16_bits_to_f32(x)));
    }
    tile[lane][r] = x;
  }
  __syncthreads();
  // row jr of the tile, 16 values from column 16 q: two 16-byte stores; rows k .. kx-1
  // (padding to a whole number of 8-row groups) are written as zeros
  const int jr = threadIdx.x >> 2, qd = threadIdx.x & 3;
  if (j0 + jr >= kx) return;
  const uint32_t* t32 = reinterpret_cast<const uint32_t*>(&tile[jr][0]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int a = 16 * qd + 8 * h;                   // tile column (even: 4-byte aligned)
    if (i0 + a >= N) continue;                       // N % 8 == 0: 8 values all in or all out
    const uint4 v = make_uint4(t32[a / 2], t32[a / 2 + 1], t32[a / 2 + 2], t32[a / 2 + 3]);
    *reinterpret_cast<uint4*>(Xt + (size_t)(j0 + jr) * ldx + i0 + a) = v;
  }
}

// W[i, S[j]] <- bf16(fl32(d W) - fl32(lr O[j, i])), d = fl32(1 - fl32(lr wd)); O: k x N
// (row stride ldo).  An index S[j] outside [0, m) updates nothing.
__global__ void __launch_bounds__(kColThreads)
update_cols_kernel(uint16_t* W, int N, int m, long long ld, const int* S, int k, const uint16_t* O, long long ldo,
                   float lr, float wd) {
  __shared__ __align__(16) uint16_t tile[kColTile][kColTile + 2];   // [j][i]
  const int j0 = blockIdx.x * kColTile, i0 = blockIdx.y * kColTile;
  {
    const int jr = threadIdx.x >> 2, qd = threadIdx.x & 3;
    uint32_t* t32 = reinterpret_cast<uint32_t*>(&tile[jr][0]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int a = 16 * qd + 8 * h;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (j0 + jr < k && i0 + a < N) v = *reinterpret_cast<const uint4*>(O + (size_t)(j0 + jr) * ldo + i0 + a);
      t32[a / 2] = v.x; t32[a / 2 + 1] = v.y; t32[a / 2 + 2] = v.z; t32[a / 2 + 3] = v.w;
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
    uint16_t* p = W + (size_t)i * ld + col;
    const float x = bf16_bits_to_f32(*p);
    const float o = bf16_bits_to_f32(tile[lane][r]);
    *p = (uint16_t)f32_to_bf16_bits(__fsub_rn(__fmul_rn(d, x), __fmul_rn(lr, o)));
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

// W[i, c] <- bf16(fl32(d W[i, c])) for every column c not marked (decoupled weight decay)
__global__ void __launch_bounds__(kColThreads)
decay_unmarked_kernel(uint16_t* W, int N, int m, long long ld, const uint8_t* mark, float lr, float wd) {
  const int c = blockIdx.x * kColThreads + threadIdx.x;   // 16-byte chunk
  if (c >= m / 8) return;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  for (int i = blockIdx.y; i < N; i += gridDim.y) {
    uint4* p = reinterpret_cast<uint4*>(W + (size_t)i * ld) + c;
    uint4 v = load_nt(p);
    uint32_t* vw = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      uint32_t out = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t bits = (vw[e2] >> (16 * h)) & 0xffffu;
        const int col = 8 * c + 2 * e2 + h;
        const uint32_t nb = mark[col] ? bits : f32_to_bf16_bits(__fmul_rn(d, bf16_bits_to_f32(bits)));
        out |= nb << (16 * h);
      }
      vw[e2] = out;
    }
    store_nt(v, p);
  }
}

size_t dion3_cols_partials(int N) { return (size_t)((N + kColRowsPerPart - 1) / kColRowsPerPart); }

hipError_t launch_accumulate_colscore(uint16_t* M, const uint16_t* G, int N, int m, long long ld, int score_norm,
                                      double* part_s, double* part_q, double* score, double* sumsq, hipStream_t s) {
  if (N <= 0 || m <= 0) return hipSuccess;
  const int nparts = (int)dion3_cols_partials(N);
  clear_stale_error();
  hipLaunchKernelGGL(accumulate_colscore_kernel, dim3((m / 8 + kColThreads - 1) / kColThreads, nparts),
                     dim3(kColThreads), 0, s, M, G, N, m, ld, score_norm, part_s, part_q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_colscore_kernel, dim3((m + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s,
                     part_s, part_q, nparts, m, score, sumsq);
  return hipGetLastError();
}

hipError_t launch_gather_cols_feedback(uint16_t* M, int N, int m, long long ld, const int* S, int k, int kx,
                                       float mu, uint16_t* Xt, long long ldx, hipStream_t s) {
  if (k <= 0 || N <= 0) return hipSuccess;
  if (kx < k) return hipErrorInvalidValue;
  clear_stale_error();
  hipLaunchKernelGGL(gather_cols_feedback_kernel, dim3((kx + kColTile - 1) / kColTile, (N + kColTile - 1) / kColTile),
                     dim3(kColThreads), 0, s, M, N, m, ld, S, k, kx, mu, Xt, ldx);
  return hipGetLastError();
}

hipError_t launch_update_cols(uint16_t* W, int N, int m, long long ld, const int* S, int k, const uint16_t* O,
                              long long ldo, float lr, float wd, uint8_t* mark, hipStream_t s) {
  if (k <= 0 || N <= 0) return hipSuccess;
  clear_stale_error();
  if (wd != 0.0f) {
    hipLaunchKernelGGL(clear_marks_kernel, dim3((m + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s, mark, m);
    hipLaunchKernelGGL(set_marks_kernel, dim3((k + kColThreads - 1) / kColThreads), dim3(kColThreads), 0, s, mark, m,
                       S, k);
    hipLaunchKernelGGL(decay_unmarked_kernel, dim3((m / 8 + kColThreads - 1) / kColThreads, std::min(N, 4096)),
                       dim3(kColThreads), 0, s, W, N, m, ld, mark, lr, wd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(update_cols_kernel, dim3((k + kColTile - 1) / kColTile, (N + kColTile - 1) / kColTile),
                     dim3(kColThreads), 0, s, W, N, m, ld, S, k, O, ldo, lr, wd);
  return hipGetLastError();
}

}  // namespace gns
