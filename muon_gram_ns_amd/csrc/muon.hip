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
// G, U and O are bf16; each stored value is rounded once, to nearest even, from fp32
// results computed op by op.  This file is compiled with -ffp-contract=off and uses
// explicit __fmul_rn/__fadd_rn/__fsub_rn so no multiply-add is fused.
#include "common.h"
#include "muon_kernels.h"

namespace gns {

// one workgroup per matrix row, 512 threads, 8 bf16 values (16 bytes) per access
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

__device__ __forceinline__ float lo_f32(uint32_t w) { return bf16_bits_to_f32(w & 0xffffu); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return bf16_bits_to_f32(w >> 16); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
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

// M' = bf16(fl32(mu M) + G);  U = bf16(G + fl32(mu M')) when U is given.  M and G
// share the row stride ld and matrix stride; U is [batch][n][ldu].  rowsq[b][r]
// receives the fp64 sum of squares of row r of the matrix the orthogonalisation reads
// (U, or M' without the lookahead), so its Frobenius norm needs no further pass.
__global__ void __launch_bounds__(kMuonThreads)
muon_momentum_kernel(uint16_t* M, const uint16_t* G, int n, int m, long long ld, long long stride, float mu,
                     uint16_t* U, long long ldu, long long su, double* rowsq) {
  __shared__ double sh[kMuonThreads / 64];
  const int r = blockIdx.x, b = blockIdx.y;
  double acc = 0.0;
  uint4* mr = reinterpret_cast<uint4*>(M + (size_t)b * stride + (size_t)r * ld);
  const uint4* gr = reinterpret_cast<const uint4*>(G + (size_t)b * stride + (size_t)r * ld);
  uint4* ur = U ? reinterpret_cast<uint4*>(U + (size_t)b * su + (size_t)r * ldu) : nullptr;
  for (int c = threadIdx.x; c < m / 8; c += kMuonThreads) {
    uint4 mv = load_stream(&mr[c]);
    const uint4 gv = load_stream(&gr[c]);
    uint32_t* mw = reinterpret_cast<uint32_t*>(&mv);
    const uint32_t* gw = reinterpret_cast<const uint32_t*>(&gv);
    uint4 uv;
    uint32_t* uw = reinterpret_cast<uint32_t*>(&uv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = lo_f32(gw[i]), g1 = hi_f32(gw[i]);
      const uint32_t mn = pack_bf16(__fadd_rn(__fmul_rn(mu, lo_f32(mw[i])), g0),
                                    __fadd_rn(__fmul_rn(mu, hi_f32(mw[i])), g1));
      mw[i] = mn;
      uw[i] = pack_bf16(__fadd_rn(g0, __fmul_rn(mu, lo_f32(mn))), __fadd_rn(g1, __fmul_rn(mu, hi_f32(mn))));
      const uint32_t x = ur ? uw[i] : mn;          // what the orthogonalisation reads
      const double x0 = (double)lo_f32(x), x1 = (double)hi_f32(x);
      acc += x0 * x0;
      acc += x1 * x1;
    }
    store_stream(mv, &mr[c]);
    if (ur) ur[c] = uv;      // read next by the Gram product: an ordinary store
  }
  const double t = muon_block_sum(acc, sh);
  if (threadIdx.x == 0) rowsq[(size_t)b * n + r] = t;
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

hipError_t launch_muon_momentum(uint16_t* M, const uint16_t* G, int batch, int n, int m, long long ld,
                                long long stride, float mu, uint16_t* U, long long ldu, long long su, double* rowsq,
                                float eps, float* s_out, hipStream_t s) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(muon_momentum_kernel, dim3(n, batch), dim3(kMuonThreads), 0, s, M, G, n, m, ld, stride, mu, U,
                     ldu, su, rowsq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(muon_scale_kernel, dim3(batch), dim3(kMuonThreads), 0, s, rowsq, n, eps, s_out);
  return hipGetLastError();
}

// W' = bf16( fl32( fl32(d W) - fl32(lre O) ) ), d = fl32(1 - fl32(lr wd)),
// lre = fl32(lr scale).  O is bf16 [batch][n][ldo].
__global__ void __launch_bounds__(kMuonThreads)
muon_update_kernel(uint16_t* W, int m, long long ld, long long stride, const uint16_t* O, long long ldo,
                   long long so, float lr, float wd, float scale) {
  const int r = blockIdx.x, b = blockIdx.y;
  const float d = __fsub_rn(1.0f, __fmul_rn(lr, wd));
  const float lre = __fmul_rn(lr, scale);
  uint4* wr = reinterpret_cast<uint4*>(W + (size_t)b * stride + (size_t)r * ld);
  const uint4* orow = reinterpret_cast<const uint4*>(O + (size_t)b * so + (size_t)r * ldo);
  for (int c = threadIdx.x; c < m / 8; c += kMuonThreads) {
    uint4 wv = load_stream(&wr[c]);
    const uint4 ov = load_stream(&orow[c]);
    uint32_t* ww = reinterpret_cast<uint32_t*>(&wv);
    const uint32_t* ow = reinterpret_cast<const uint32_t*>(&ov);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ww[i] = pack_bf16(__fsub_rn(__fmul_rn(d, lo_f32(ww[i])), __fmul_rn(lre, lo_f32(ow[i]))),
                        __fsub_rn(__fmul_rn(d, hi_f32(ww[i])), __fmul_rn(lre, hi_f32(ow[i]))));
    }
    store_stream(wv, &wr[c]);
  }
}

hipError_t launch_muon_update(uint16_t* W, int batch, int n, int m, long long ld, long long stride,
                              const uint16_t* O, long long ldo, long long so, float lr, float wd, float scale,
                              hipStream_t s) {
  if (batch <= 0 || n <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(muon_update_kernel, dim3(n, batch), dim3(kMuonThreads), 0, s, W, m, ld, stride, O, ldo, so, lr,
                     wd, scale);
  return hipGetLastError();
}

}  // namespace gns
