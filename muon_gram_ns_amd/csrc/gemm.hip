// MFMA GEMM kernels for gfx950: the symmetric-output product (lower-triangle tiles,
// mirrored epilogue) and the rectangular product Q X.
//
// Symmetric GEMM: only output tiles on or below the diagonal are scheduled, and each
// computed tile is also written transposed above the diagonal, which halves the
// multiply work for a symmetric result ("Dion3: Full-Stack Orthogonal Updates",
// paper.rainbus.top, 前置知识 "symmetric GEMM kernel" and 方法步骤详情 (2)).  The
// epilogue forms alpha*acc + beta*C + gamma*I in fp32 before a single rounding, and
// can emit a second output shifted by delta*I (Q_1 = Z_1 + a_1 I in Gram NS).
//
// Both kernels read their operands as rows that are contiguous along K:
//   NT  (symmetric): A is n x K, B is n x K; D = A B^T.  With B symmetric and K = n
//       this is A B, with A == B the Gram product.
//   NN  (rectangular): A is n x K, B is K x m (rows contiguous along m).  B's tile
//       is transposed in registers on its way to LDS, so the MFMA loop is shared.
// LDS holds two stages of [rows][128 bytes] tiles for A and B (K-contiguous,
// 16-byte chunks XOR-swizzled, see swz()).  Each wave owns a WM x WN sub-tile made
// of 16x16 MFMA fragments accumulated in fp32.
#include "common.h"
#include "internal.h"

namespace gns {

__device__ __forceinline__ void tri_decode(int t, int& i, int& j) {
  int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  i = r;
  j = t - r * (r + 1) / 2;
}

template <class TOut>
__device__ __forceinline__ void store1(void* base, long long off, float v) {
  if constexpr (TOut::kBytes == 4) {
    reinterpret_cast<float*>(base)[off] = v;
  } else {
    reinterpret_cast<uint16_t*>(base)[off] = (uint16_t)TOut::from_f32(v);
  }
}

template <class TOut>
__device__ __forceinline__ void store4(void* base, long long off, const float v[4]) {
  if constexpr (TOut::kBytes == 4) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    uint2 w;
    w.x = TOut::from_f32(v[0]) | (TOut::from_f32(v[1]) << 16);
    w.y = TOut::from_f32(v[2]) | (TOut::from_f32(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off) = w;
  }
}

template <class TOut>
__device__ __forceinline__ void load4(const void* base, long long off, float v[4]) {
  if constexpr (TOut::kBytes == 4) {
    float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    v[0] = TOut::to_f32(w.x & 0xffffu); v[1] = TOut::to_f32(w.x >> 16);
    v[2] = TOut::to_f32(w.y & 0xffffu); v[3] = TOut::to_f32(w.y >> 16);
  }
}

// Convert a 16-byte chunk of TB elements (times mul) to TIn elements.  Only 16-bit
// to 16-bit conversions are used, so the chunk geometry is unchanged.
template <class TIn, class TB>
__device__ __forceinline__ uint4 convert_chunk(uint4 c, float mul) {
  if constexpr (TIn::kId == TB::kId) {
    return c;
  } else {
    static_assert(TIn::kBytes == 2 && TB::kBytes == 2, "only 16-bit conversions");
    uint32_t* w = reinterpret_cast<uint32_t*>(&c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = TIn::from_f32(TB::to_f32(w[i] & 0xffffu) * mul);
      uint32_t hi = TIn::from_f32(TB::to_f32(w[i] >> 16) * mul);
      w[i] = lo | (hi << 16);
    }
    return c;
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct Tile {
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kWM = BM / WAVES_M;
  static constexpr int kWN = BN / WAVES_N;
  static constexpr int kFM = kWM / 16;
  static constexpr int kFN = kWN / 16;
  static constexpr int kLdsBytes = 2 * (BM + BN) * 128;
};

// One kernel for both products.  LOWER: symmetric output (triangle schedule +
// mirror); otherwise a plain tile grid.  NN: B is K x N (transposed on load).
template <class TIn, class TB, class TOut, int BM, int BN, int WAVES_M, int WAVES_N, bool LOWER, bool NN>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_kernel(GemmParams p) {
  using Cfg = Tile<BM, BN, WAVES_M, WAVES_N>;
  constexpr int NT = Cfg::kThreads;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  constexpr int EPC = TIn::kPerChunk;          // elements per 16-byte chunk
  constexpr int BK = 8 * EPC;                  // K elements per LDS tile row
  constexpr int A_LOADS = BM * 8 / NT;         // 16-byte chunks per thread per stage
  constexpr int B_LOADS_NT = BN * 8 / NT;
  constexpr int NN_COLS = BN / EPC;            // NN: column groups of one k-row
  constexpr int NN_BLOCKS = (BK / 4) * NN_COLS / NT;   // NN: 4(k) x EPC(n) blocks per thread
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(!NN || ((BK / 4) * NN_COLS) % NT == 0, "NN B tile/thread mismatch");
  static_assert(!LOWER || BM == BN, "symmetric tiles must be square");

  extern __shared__ __align__(16) uint4 smem[];
  uint4* As = smem;                      // [2][BM][8]
  uint4* Bs = smem + 2 * BM * 8;         // [2][BN][8]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int bz = blockIdx.y;

  int tm, tn;
  if constexpr (LOWER) {
    tri_decode(blockIdx.x, tm, tn);
  } else {
    tm = blockIdx.x / p.tiles_n;
    tn = blockIdx.x % p.tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;

  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(p.A) + (size_t)bz * p.sA * TIn::kBytes;
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(p.B) + (size_t)bz * p.sB * TB::kBytes;

  float bmul = 1.0f;
  if constexpr (NN && TIn::kId != TB::kId) {
    bmul = p.b_mul;
    if (p.scale) for (int i = 0; i < p.b_pow; ++i) bmul *= p.scale[bz];
  }

  uint4 ra[A_LOADS];
  uint4 rb[NN ? 4 * NN_BLOCKS : B_LOADS_NT];

  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + i * NT, row = c >> 3, ch = c & 7;
      const int gr = m0 + row, gk = k0 + ch * EPC;
      ra[i] = (gr < M && gk < K)
                  ? *reinterpret_cast<const uint4*>(Ab + ((size_t)gr * p.lda + gk) * TIn::kBytes)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto load_b = [&](int k0) {
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_LOADS_NT; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        const int gr = n0 + row, gk = k0 + ch * EPC;
        rb[i] = (gr < N && gk < K)
                    ? *reinterpret_cast<const uint4*>(Bb + ((size_t)gr * p.ldb + gk) * TB::kBytes)
                    : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < NN_BLOCKS; ++blk) {
        const int t = tid + blk * NT;
        const int kb = t % (BK / 4), nb = t / (BK / 4);
        const int gn = n0 + nb * EPC;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gk = k0 + kb * 4 + r;
          rb[blk * 4 + r] = (gk < K && gn < N)
                                ? *reinterpret_cast<const uint4*>(Bb + ((size_t)gk * p.ldb + gn) * TB::kBytes)
                                : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_a = [&](int stage) {
    uint4* dst = As + stage * BM * 8;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + i * NT, row = c >> 3, ch = c & 7;
      dst[row * 8 + swz(row, ch)] = ra[i];
    }
  };
  auto store_b = [&](int stage) {
    uint4* dst = Bs + stage * BN * 8;
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_LOADS_NT; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        dst[row * 8 + swz(row, ch)] = rb[i];
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < NN_BLOCKS; ++blk) {
        const int t = tid + blk * NT;
        const int kb = t % (BK / 4), nb = t / (BK / 4);
        uint4 rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) rows[r] = convert_chunk<TIn, TB>(rb[blk * 4 + r], bmul);
        if constexpr (TIn::kBytes == 2) {
          // 4 k-rows x 8 n-columns of 16-bit values -> for each column, 4 k-values
          // (8 bytes) at k offset 4*kb of row n: chunk kb/2, half kb&1.
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&rows[0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&rows[1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&rows[2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&rows[3]);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int sh = (j & 1) * 16;
            const uint32_t e0 = (w0[j >> 1] >> sh) & 0xffffu, e1 = (w1[j >> 1] >> sh) & 0xffffu;
            const uint32_t e2 = (w2[j >> 1] >> sh) & 0xffffu, e3 = (w3[j >> 1] >> sh) & 0xffffu;
            const int n = nb * 8 + j;
            uint8_t* rowp = reinterpret_cast<uint8_t*>(dst + n * 8 + swz(n, kb >> 1)) + (kb & 1) * 8;
            *reinterpret_cast<uint2*>(rowp) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
          }
        } else {
          // fp32: 4 k-rows x 4 n-columns -> each column's 4 k-values fill chunk kb.
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = nb * 4 + j;
            const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&rows[0]);
            const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&rows[1]);
            const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&rows[2]);
            const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&rows[3]);
            dst[n * 8 + swz(n, kb)] = make_uint4(r0[j], r1[j], r2[j], r3[j]);
          }
        }
      }
    }
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = (K + BK - 1) / BK;
  load_a(0);
  load_b(0);
  store_a(0);
  store_b(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt & 1;
    if (kt + 1 < KT) {
      load_a((kt + 1) * BK);
      load_b((kt + 1) * BK);
    }
    const uint4* as = As + stage * BM * 8;
    const uint4* bs = Bs + stage * BN * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 4 + (lane >> 4);
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * Cfg::kWM + i * 16 + (lane & 15);
        af[i] = as[row * 8 + swz(row, ch)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * Cfg::kWN + j * 16 + (lane & 15);
        bfr[j] = bs[row * 8 + swz(row, ch)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mfma_step<TIn>(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < KT) {
      store_a(stage ^ 1);
      store_b(stage ^ 1);
    }
    __syncthreads();
  }

  // ---- epilogue: v = alpha_eff*acc + beta*C + gamma*[diag]; D (and D2 = v + delta*[diag])
  float alpha = p.alpha;
  if (p.scale) for (int i = 0; i < p.alpha_pow; ++i) alpha *= p.scale[bz];
  uint8_t* Db = reinterpret_cast<uint8_t*>(p.D) + (size_t)bz * p.sD * TOut::kBytes;
  uint8_t* D2b = p.D2 ? reinterpret_cast<uint8_t*>(p.D2) + (size_t)bz * p.sD2 * TOut::kBytes : nullptr;
  const uint8_t* Cb = p.C ? reinterpret_cast<const uint8_t*>(p.C) + (size_t)bz * p.sC * TOut::kBytes : nullptr;

#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int gm = m0 + wm * Cfg::kWM + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int gn = n0 + wn * Cfg::kWN + j * 16 + 4 * (lane >> 4);
      if (gm >= M || gn >= N) continue;       // N % 4 == 0, so gn < N covers gn..gn+3
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][e];
      if (Cb && p.beta != 0.0f) {
        float c[4];
        load4<TOut>(Cb, (long long)gm * p.ldc + gn, c);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += p.beta * c[e];
      }
      if (p.gamma != 0.0f) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gn + e == gm) v[e] += p.gamma;
      }
      if constexpr (!LOWER) {
        store4<TOut>(Db, (long long)gm * p.ldd + gn, v);
      } else {
        const bool all_lower = gn + 3 <= gm;
        if (all_lower) {
          store4<TOut>(Db, (long long)gm * p.ldd + gn, v);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e <= gm) store1<TOut>(Db, (long long)gm * p.ldd + gn + e, v[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gn + e < gm) store1<TOut>(Db, (long long)(gn + e) * p.ldd + gm, v[e]);
        if (D2b) {
          float w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = v[e] + ((gn + e == gm) ? p.delta : 0.0f);
          if (all_lower) {
            store4<TOut>(D2b, (long long)gm * p.ldd2 + gn, w);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gn + e <= gm) store1<TOut>(D2b, (long long)gm * p.ldd2 + gn + e, w[e]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < gm) store1<TOut>(D2b, (long long)(gn + e) * p.ldd2 + gm, w[e]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Host launchers

namespace {
constexpr int kBM = 128, kBN = 128, kWavesM = 2, kWavesN = 2;
using DefTile = Tile<kBM, kBN, kWavesM, kWavesN>;

template <class TIn, class TB, class TOut, bool LOWER, bool NN>
hipError_t launch_cfg(GemmParams p, int batch, hipStream_t stream, double* flops) {
  auto kern = gemm_kernel<TIn, TB, TOut, kBM, kBN, kWavesM, kWavesN, LOWER, NN>;
  const int tm = (p.M + kBM - 1) / kBM, tn = (p.N + kBN - 1) / kBN;
  p.tiles_m = tm;
  p.tiles_n = tn;
  const long long tiles = LOWER ? (long long)tm * (tm + 1) / 2 : (long long)tm * tn;
  constexpr int BK = 8 * TIn::kPerChunk;
  const long long kpad = ((long long)(p.K + BK - 1) / BK) * BK;
  if (flops) *flops += 2.0 * (double)tiles * kBM * kBN * (double)kpad * batch;
  if (tiles == 0 || batch == 0) return hipSuccess;
  dim3 grid((unsigned)tiles, (unsigned)batch);
  clear_stale_error();
  hipLaunchKernelGGL(kern, grid, dim3(DefTile::kThreads), DefTile::kLdsBytes, stream, p);
  return hipGetLastError();
}

template <class TIn, class TB, bool LOWER, bool NN>
hipError_t dispatch_out(gns_dtype out, const GemmParams& p, int batch, hipStream_t s, double* f) {
  switch (out) {
    case GNS_BF16: return launch_cfg<TIn, TB, TBF16, LOWER, NN>(p, batch, s, f);
    case GNS_F16: return launch_cfg<TIn, TB, TF16, LOWER, NN>(p, batch, s, f);
    case GNS_F32: return launch_cfg<TIn, TB, TF32, LOWER, NN>(p, batch, s, f);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_symm(gns_dtype in, gns_dtype out, const GemmParams& p, int batch, hipStream_t s,
                       double* flops) {
  switch (in) {
    case GNS_BF16: return dispatch_out<TBF16, TBF16, true, false>(out, p, batch, s, flops);
    case GNS_F16: return dispatch_out<TF16, TF16, true, false>(out, p, batch, s, flops);
    case GNS_F32: return dispatch_out<TF32, TF32, true, false>(out, p, batch, s, flops);
  }
  return hipErrorInvalidValue;
}

bool rect_pair_supported(gns_dtype a, gns_dtype b) {
  if (a == b) return true;
  return (a == GNS_F16 && b == GNS_BF16) || (a == GNS_BF16 && b == GNS_F16);
}

hipError_t launch_rect(gns_dtype a, gns_dtype b, gns_dtype out, const GemmParams& p, int batch,
                       hipStream_t s, double* flops) {
  if (a == GNS_BF16 && b == GNS_BF16) return dispatch_out<TBF16, TBF16, false, true>(out, p, batch, s, flops);
  if (a == GNS_F16 && b == GNS_F16) return dispatch_out<TF16, TF16, false, true>(out, p, batch, s, flops);
  if (a == GNS_F32 && b == GNS_F32) return dispatch_out<TF32, TF32, false, true>(out, p, batch, s, flops);
  if (a == GNS_F16 && b == GNS_BF16) return dispatch_out<TF16, TBF16, false, true>(out, p, batch, s, flops);
  if (a == GNS_BF16 && b == GNS_F16) return dispatch_out<TBF16, TF16, false, true>(out, p, batch, s, flops);
  return hipErrorInvalidValue;
}

}  // namespace gns
