// Muon step element-wise passes (HBM-bound): momentum with the lookahead, and the
// decoupled decay with the scaled update.
//
// The step ("Muon: Orthogonalized Momentum and Why It Trains LLMs 2x Cheaper", the
// step listed after "Doing an SVD without an SVD" and the notes on decoupled weight
// decay and update-scale matching):
//   M <- mu M + G                    heavy-ball momentum
//   U  = G + mu M  (lookahead)  or  U = M
//   O  = NS(U)                       (the Gram NS of this library)
//   W <- (1 - lr wd) W - lr scale O,  scale = 0.2 sqrt(max(n, m)) by default
//
// Rounding model (the page leaves it open; the same reading as the Dion3 step): W, M,
// G, U and O share the state type T (bf16, f16 or fp32); each stored value is rounded
// once, to nearest even, from fp32 results computed op by op.  This file is compiled
// with -ffp-contract=off and uses explicit __fmul_rn/__fadd_rn/__fsub_rn so no
// multiply-add is fused.
#include "common.h"
#include "muon_kernels.h"
#include "state_types.h"

namespace gns {

// one workgroup per matrix row, 512 threads, one 16-byte chunk per access
constexpr int kMuonThreads = 512;

// Streaming accesses (each element read or written once per pass) bypass the caches.
typedef unsigned int u32x4_stream __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4_stream v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_stream*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(const uint4& v, uint4* p) {
  const u32x4_stream x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_stream*>(p));
}

// fp64 sum over the workgroup; the total is valid in thread 0
__device__ __forceinline__ double muon_block_sum(double v, double* sh) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int i = 0; i < kMuonThreads / 64; ++i) t += sh[i];
  return t;
}

// M' = fl(fl32(mu M) + G);  U = fl(G + fl32(mu M')) when U is given.  M and G share
// the row stride ld and matrix stride; U is [batch][n][ldu].  rowsq[b][r] receives the
// fp64 sum of squares of row r of the matrix the orthogonalisation reads (U, or M'
// without the lookahead), so its Frobenius norm needs no further pass over it; rowsq32
// (when non-null) the same sums rounded to fp32.
template <class T>
__global__ void __launch_bounds__(kMuonThreads)
muon_momentum_kernel(void* M, const void* G, int n, int m, long long ld, long long stride, float mu, void* U,
                     long long ldu, long long su, double* rowsq, float* rowsq32) {
  constexpr int E = T::kPerChunk;
  __shared__ double sh[kMuonThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  double acc = 0.0;
  uint4* mr = row_chunks<T>(M, (long long)b * stride + (long long)r * ld);
  const uint4* gr = row_chunks<T>(G, (long long)b * stride + (long long)r * ld);
  uint4* ur = U ? row_chunks<T>(U, (long long)b * su + (long long)r * ldu) : nullptr;
  for (int c = threadIdx.x; c < m / E; c += kMuonThreads) {
    const uint4 mv = load_stream(&mr[c]);
    const uint4 gv = load_stream(&gr[c]);
    float x[E], g[E];
    unpack<T>(mv, x);
    unpack<T>(gv, g);
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = __fadd_rn(__fmul_rn(mu, x[i]), g[i]);
    const uint4 mn = pack<T>(x);
    unpack<T>(mn, x);                              // the stored M'
    store_stream(mn, &mr[c]);
    if (ur) {
#pragma unroll
      for (int i = 0; i < E; ++i) x[i] = __fadd_rn(g[i], __fmul_rn(mu, x[i]));
      const uint4 uv = pack<T>(x);
      unpack<T>(uv, x);                            // the stored U
      ur[c] = uv;      // read next by the Gram product: an ordinary store
    }
#pragma unroll
    for (int i = 0; i < E; ++i) {                  // what the orthogonalisation reads
      const double v = (double)x[i];
      acc += v * v;
    }
  }
  const double t = muon_block_sum(acc, sh);
  if (threadIdx.x == 0) {
    rowsq[(size_t)b * n + r] = t;
    if (rowsq32) rowsq32[(size_t)b * n + r] = (float)t;
  }
}

// s[b] = 1 / (sqrt(sum_r rowsq[b][r]) + eps), one workgroup per matrix; each thread
// adds a contiguous range of rows in order, so the result does not depend on the batch.
__global__ void __launch_bounds__(kMuonThreads)
muon_scale_kernel(const double* rowsq, int n, float eps, float* s) {
  __shared__ double sh[kMuonThreads / 64];
  const int b = blockIdx.x;
  rowsq += (size_t)b * n;
  const int per = (n + kMuonThreads - 1) / kMuonThreads;
  const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
  double acc = 0.0;
  for (int i = lo; i < hi; ++i) acc += rowsq[i];
  const double t = muon_block_sum(acc, sh);
  if (threadIdx.x == 0) s[b] = (float)(1.0 / (sqrt(t) + (double)eps));
}

hipError_t launch_muon_momentum(void* M, const void* G, gns_dtype dt, int batch, int n, int m, long long ld,
                                long long stride, float mu, void* U, long long ldu, long long su, double* rowsq,
                                float* rowsq32, float eps, float* s_out, hipStream_t s) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    hipLaunchKernelGGL(muon_momentum_kernel<T>, dim3(n, batch), dim3(kMuonThreads), 0, s, M, G, n, m, ld, stride,
                       mu, U, ldu, su, rowsq, rowsq32);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !s_out) return e;
    hipLaunchKernelGGL(muon_scale_kernel, dim3(batch), dim3(kMuonThreads), 0, s, rowsq, n, eps, s_out);
    return hipGetLastError();
  });
}

// W' = fl( fl32( fl32(d W) - fl32(lre O) ) ), d = fl32(1 - fl32(lr wd)),
// lre = fl32(lr scale).  O is [batch][n][ldo] in the state type.
template <class T>
__global__ void __launch_bounds__(kMuonThreads)
muon_update_kernel(void* W, int m, long long ld, long long stride, const void* O, long long ldo, long long so,
                   float lr, float wd, float scale) {
  constexpr int E = T::kPerChunk;
  const int r = blockIdx.x, b = blockIdx.y;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  const float lre = __fmul_rn(lr, scale);
  uint4* wr = row_chunks<T>(W, (long long)b * stride + (long long)r * ld);
  const uint4* orow = row_chunks<T>(O, (long long)b * so + (long long)r * ldo);
  for (int c = threadIdx.x; c < m / E; c += kMuonThreads) {
    const uint4 wv = load_stream(&wr[c]);
    const uint4 ov = load_stream(&orow[c]);
    float x[E], o[E];
    unpack<T>(wv, x);
    unpack<T>(ov, o);
#pragma unroll
    for (int i = 0; i < E; ++i) x[i] = __fsub_rn(__fmul_rn(d, x[i]), __fmul_rn(lre, o[i]));
    store_stream(pack<T>(x), &wr[c]);
  }
}

hipError_t launch_muon_update(void* W, gns_dtype dt, int batch, int n, int m, long long ld, long long stride,
                              const void* O, long long ldo, long long so, float lr, float wd, float scale,
                              hipStream_t s) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  return with_state_type(dt, [&](auto tag) {
    using T = decltype(tag);
    clear_stale_error();
    hipLaunchKernelGGL(muon_update_kernel<T>, dim3(n, batch), dim3(kMuonThreads), 0, s, W, m, ld, stride, O, ldo,
                       so, lr, wd, scale);
    return hipGetLastError();
  });
}

}  // namespace gns
