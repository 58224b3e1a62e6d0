// HBM-bound helpers of the Gram NS path: the Frobenius scale s = 1/(||X||_F + eps)
// and a scaled dtype cast.
//
// Normalisation by the Frobenius norm plus a small eps is the first step of the
// Newton-Schulz iteration ("Muon: Orthogonalized Momentum ...", section "Doing an
// SVD without an SVD"; paper.rainbus.top 方法步骤详情 Algorithm 3).  The Gram path
// never materialises the normalised X: s is kept on the device and folded into the
// epilogues of the products that read X.
//
// Reduction: each workgroup sums squares of a band of rows in fp32 (16-byte loads,
// grid-stride over the band), reduces across the workgroup in a fixed order and
// writes one partial; a second kernel (or, in Gram NS, the first Gram product's
// epilogue) adds a batch's partials in a fixed order.  No atomics, so the result is
// bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace gns {

constexpr int kRedThreads = 256;

template <typename V>
__device__ __forceinline__ V block_sum(V v, V* sh) {
  // wave reduction (fixed butterfly order), then the 4 wave sums in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh[w] = v;
  __syncthreads();
  V t = 0;
  if (threadIdx.x == 0)
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += sh[i];
  return t;   // valid in thread 0
}

int frob_partials_per_batch(int n, int m) {
  (void)m;
  int p = 1024;
  if (p > n) p = n;
  return p < 1 ? 1 : p;
}

template <class T>
__global__ void __launch_bounds__(kRedThreads)
frob_partial_kernel(const uint8_t* X, long long ldx, long long sx, int n, int m, int P, float* partials) {
  __shared__ float sh[kRedThreads / 64];
  const int p = blockIdx.x, b = blockIdx.y;
  const int rows_per = (n + P - 1) / P;
  const int r0 = p * rows_per, r1 = min(n, r0 + rows_per);
  const int cpr = m / T::kPerChunk;                        // chunks per row
  const uint8_t* base = X + (size_t)b * sx * T::kBytes;
  float acc = 0.f;
  const long long total = (long long)(r1 > r0 ? r1 - r0 : 0) * cpr;
  for (long long c = threadIdx.x; c < total; c += kRedThreads) {
    const int r = r0 + (int)(c / cpr), ch = (int)(c % cpr);
    const uint4 v = *reinterpret_cast<const uint4*>(base + ((size_t)r * ldx + (size_t)ch * T::kPerChunk) * T::kBytes);
#pragma unroll
    for (int e = 0; e < T::kPerChunk; ++e) {
      const float f = chunk_elem<T>(v, e);
      acc += f * f;
    }
  }
  const float t = block_sum(acc, sh);
  if (threadIdx.x == 0) partials[(size_t)b * P + p] = t;
}

__global__ void __launch_bounds__(kRedThreads)
frob_finish_kernel(const float* partials, int P, float eps, float* s_out) {
  __shared__ float sh[kRedThreads / 64];
  const int b = blockIdx.x;
  // each thread adds a contiguous slice in order, then the fixed tree
  const int per = (P + kRedThreads - 1) / kRedThreads;
  float acc = 0.f;
  for (int i = threadIdx.x * per; i < min(P, (int)(threadIdx.x + 1) * per); ++i) acc += partials[(size_t)b * P + i];
  const float t = block_sum(acc, sh);
  if (threadIdx.x == 0) s_out[b] = 1.0f / (sqrtf(t) + eps);
}

hipError_t launch_frob_partials(const void* X, gns_dtype dt, long long ldx, long long stride_x, int batch, int n,
                                int m, float* partials, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  const int P = frob_partials_per_batch(n, m);
  dim3 grid(P, batch);
  const uint8_t* x = reinterpret_cast<const uint8_t*>(X);
  switch (dt) {
    case GNS_BF16: clear_stale_error(); hipLaunchKernelGGL(frob_partial_kernel<TBF16>, grid, dim3(kRedThreads), 0, stream, x, ldx, stride_x, n, m, P, partials); break;
    case GNS_F16: clear_stale_error(); hipLaunchKernelGGL(frob_partial_kernel<TF16>, grid, dim3(kRedThreads), 0, stream, x, ldx, stride_x, n, m, P, partials); break;
    case GNS_F32: clear_stale_error(); hipLaunchKernelGGL(frob_partial_kernel<TF32>, grid, dim3(kRedThreads), 0, stream, x, ldx, stride_x, n, m, P, partials); break;
  }
  return hipGetLastError();
}

hipError_t launch_frob_finish(const float* partials, int P, int batch, float eps, float* s_out, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  clear_stale_error();
  hipLaunchKernelGGL(frob_finish_kernel, dim3(batch), dim3(kRedThreads), 0, stream, partials, P, eps, s_out);
  return hipGetLastError();
}

hipError_t launch_frob(const void* X, gns_dtype dt, long long ldx, long long stride_x, int batch, int n,
                       int m, float eps, float* s_out, float* partials, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  const int P = frob_partials_per_batch(n, m);
  hipError_t e = launch_frob_partials(X, dt, ldx, stride_x, batch, n, m, partials, stream);
  if (e != hipSuccess) return e;
  return launch_frob_finish(partials, P, batch, eps, s_out, stream);
}

// ---- scaled cast: Y = mul * scale[b]^pow * X, converted element by element --------
template <class TX, class TY>
__global__ void __launch_bounds__(256)
cast_scale_kernel(const uint8_t* X, long long ldx, long long sx, uint8_t* Y, long long ldy, long long sy,
                  int n, int m, float mul, const float* scale, int pow) {
  const int b = blockIdx.y;
  float f = mul;
  if (scale) for (int i = 0; i < pow; ++i) f *= scale[b];
  const long long groups = (long long)n * (m / 4);
  for (long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x; g < groups;
       g += (long long)gridDim.x * blockDim.x) {
    const int r = (int)(g / (m / 4)), c = (int)(g % (m / 4)) * 4;
    const uint8_t* xp = X + ((size_t)b * sx + (size_t)r * ldx + c) * TX::kBytes;
    uint8_t* yp = Y + ((size_t)b * sy + (size_t)r * ldy + c) * TY::kBytes;
    float v[4];
    if constexpr (TX::kBytes == 4) {
      const float4 q = *reinterpret_cast<const float4*>(xp);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      const uint2 q = *reinterpret_cast<const uint2*>(xp);
      v[0] = TX::to_f32(q.x & 0xffffu); v[1] = TX::to_f32(q.x >> 16);
      v[2] = TX::to_f32(q.y & 0xffffu); v[3] = TX::to_f32(q.y >> 16);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= f;
    if constexpr (TY::kBytes == 4) {
      *reinterpret_cast<float4*>(yp) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      *reinterpret_cast<uint2*>(yp) = make_uint2(TY::from_f32(v[0]) | (TY::from_f32(v[1]) << 16),
                                                 TY::from_f32(v[2]) | (TY::from_f32(v[3]) << 16));
    }
  }
}

template <class TX>
static hipError_t cast_to(gns_dtype ydt, dim3 grid, hipStream_t s, const uint8_t* x, long long ldx, long long sx,
                          uint8_t* y, long long ldy, long long sy, int n, int m, float mul, const float* scale, int pow) {
  switch (ydt) {
    case GNS_BF16: clear_stale_error(); hipLaunchKernelGGL((cast_scale_kernel<TX, TBF16>), grid, dim3(256), 0, s, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow); break;
    case GNS_F16: clear_stale_error(); hipLaunchKernelGGL((cast_scale_kernel<TX, TF16>), grid, dim3(256), 0, s, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow); break;
    case GNS_F32: clear_stale_error(); hipLaunchKernelGGL((cast_scale_kernel<TX, TF32>), grid, dim3(256), 0, s, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow); break;
  }
  return hipGetLastError();
}

hipError_t launch_cast_scale(const void* X, gns_dtype xdt, long long ldx, long long sx, void* Y, gns_dtype ydt,
                             long long ldy, long long sy, int batch, int n, int m, float mul, const float* scale,
                             int pow, hipStream_t stream) {
  if (batch <= 0 || n <= 0 || m <= 0) return hipSuccess;
  const long long groups = (long long)n * (m / 4);
  long long blocks = (groups + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks, batch);
  const uint8_t* x = reinterpret_cast<const uint8_t*>(X);
  uint8_t* y = reinterpret_cast<uint8_t*>(Y);
  switch (xdt) {
    case GNS_BF16: return cast_to<TBF16>(ydt, grid, stream, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow);
    case GNS_F16: return cast_to<TF16>(ydt, grid, stream, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow);
    case GNS_F32: return cast_to<TF32>(ydt, grid, stream, x, ldx, sx, y, ldy, sy, n, m, mul, scale, pow);
  }
  return hipErrorInvalidValue;
}

// ---- batched transpose: Y[b] = X[b]^T for rows x cols matrices -------------------
// Newton-Schulz runs on the short side of a matrix ("Muon: Orthogonalized Momentum
// ...", section "Doing an SVD without an SVD": a tall input is transposed first).
// 64 x 64 tiles staged through LDS with a pitch of 65 elements, so both the row-wise
// writes and the column-wise reads of a wave hit distinct banks; global loads and
// stores move 16-byte vectors along rows (rows and cols are multiples of 8, so a
// vector is wholly inside or outside the matrix).
template <class T>
__global__ void __launch_bounds__(256)
transpose_kernel(const uint8_t* X, long long ldx, long long sx, uint8_t* Y, long long ldy, long long sy, int rows,
                 int cols) {
  using U = typename std::conditional<T::kBytes == 2, uint16_t, uint32_t>::type;
  constexpr int VE = 16 / T::kBytes;                 // elements per 16-byte vector
  constexpr int NV = 16 / VE;                        // vectors per thread (16 elements)
  __shared__ U tile[64][65];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const U* xs = reinterpret_cast<const U*>(X + (size_t)b * sx * T::kBytes);
  U* ys = reinterpret_cast<U*>(Y + (size_t)b * sy * T::kBytes);
  {  // load: thread t takes row t / 4, columns 16 (t % 4) .. +15 of the tile
    const int r = t >> 2, cb = (t & 3) * 16;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int gr = r0 + r, gc = c0 + cb + v * VE;
      uint4 q = make_uint4(0, 0, 0, 0);
      if (gr < rows && gc < cols) q = *reinterpret_cast<const uint4*>(xs + (size_t)gr * ldx + gc);
      const U* e = reinterpret_cast<const U*>(&q);
#pragma unroll
      for (int i = 0; i < VE; ++i) tile[r][cb + v * VE + i] = e[i];
    }
  }
  __syncthreads();
  {  // store: thread t takes output row (= input column) t / 4, output columns 16 (t % 4) ..
    const int oc = t >> 2, rb = (t & 3) * 16;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      uint4 q;
      U* e = reinterpret_cast<U*>(&q);
#pragma unroll
      for (int i = 0; i < VE; ++i) e[i] = tile[rb + v * VE + i][oc];
      const int grow = c0 + oc, gcol = r0 + rb + v * VE;
      if (grow < cols && gcol < rows) *reinterpret_cast<uint4*>(ys + (size_t)grow * ldy + gcol) = q;
    }
  }
}

hipError_t launch_transpose(const void* X, gns_dtype dt, long long ldx, long long sx, int batch, int rows, int cols,
                            void* Y, long long ldy, long long sy, hipStream_t stream) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  const uint8_t* x = reinterpret_cast<const uint8_t*>(X);
  uint8_t* y = reinterpret_cast<uint8_t*>(Y);
  clear_stale_error();
  switch (dt) {
    case GNS_BF16: hipLaunchKernelGGL(transpose_kernel<TBF16>, grid, dim3(256), 0, stream, x, ldx, sx, y, ldy, sy, rows, cols); break;
    case GNS_F16: hipLaunchKernelGGL(transpose_kernel<TF16>, grid, dim3(256), 0, stream, x, ldx, sx, y, ldy, sy, rows, cols); break;
    case GNS_F32: hipLaunchKernelGGL(transpose_kernel<TF32>, grid, dim3(256), 0, stream, x, ldx, sx, y, ldy, sy, rows, cols); break;
  }
  return hipGetLastError();
}

// ---- sum of the K-range partial products of a split Gram product ------------------
// One float4 per thread: block 0 of tile t receives the sum of its `ranges` blocks,
// added in range order (the same order for every element and every call).
__global__ void __launch_bounds__(256)
sum_ranges_kernel(float4* part, long long quads_per_block, int ranges, long long total) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= total) return;
  const long long t = g / quads_per_block, x = g - t * quads_per_block;
  float4* base = part + (size_t)t * ranges * quads_per_block + x;
  float4 acc = base[0];
  for (int r = 1; r < ranges; ++r) {
    const float4 v = base[(size_t)r * quads_per_block];
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  base[0] = acc;
}

hipError_t launch_sum_ranges(float* part, long long tiles, int ranges, long long block_floats, hipStream_t stream) {
  if (tiles <= 0 || ranges <= 1) return hipSuccess;
  const long long quads = block_floats / 4, total = tiles * quads;
  clear_stale_error();
  hipLaunchKernelGGL(sum_ranges_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(part), quads, ranges, total);
  return hipGetLastError();
}

}  // namespace gns
