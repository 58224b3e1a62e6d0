// MFMA GEMM kernels for gfx950: the symmetric-output product (lower-triangle tiles,
// mirrored epilogue) and the rectangular product Q X.
//
// Symmetric GEMM: only output tiles on or below the diagonal are scheduled, and each
// computed tile is also written transposed above the diagonal, which halves the
// multiply work for a symmetric result ("Dion3: Full-Stack Orthogonal Updates",
// paper.rainbus.top, 前置知识 "symmetric GEMM kernel" and 方法步骤详情 (2)).  The
// epilogue forms alpha*acc + beta*C + gamma*I in fp32 before a single rounding.
//
// Both kernels read their operands as rows that are contiguous along K:
//   NT  (symmetric): A is n x K, B is n x K; D = A B^T.  With B symmetric and K = n
//       this is A B, with A == B the Gram product.
//   NN  (rectangular): A is n x K, B is K x m (rows contiguous along m).
// Two kernels share the epilogues: gemm16_kernel for fp16/bf16 operands (32x32x16
// MFMA, direct HBM -> LDS loads into a ring of k-stages) and gemm_kernel for fp32
// operands (16x16x4 MFMA, register-staged double buffer).  Each wave owns a WM x WN
// sub-tile of MFMA fragments accumulated in fp32.
#pragma once
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"


namespace gns {

// (the hardware square root is within an ulp or two; the loops correct the estimate)
__device__ __forceinline__ void tri_decode(int t, int& i, int& j) {
  int r = (int)((__builtin_amdgcn_sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  i = r;
  j = t - r * (r + 1) / 2;
}

// Tile orders that keep the workgroups running at the same time on one XCD on a few
// operand panels: tiles go in groups of G tile-rows, column by column within a group
// (32 concurrent 256 x 256 tiles then read 4 A panels and 8 B panels instead of 2
// and 16), so a k-slice fetched from HBM is reused from L2 by more tiles.
__device__ __forceinline__ void rect_tile_grouped(int t, int tiles_m, int tiles_n, int G, int& tm, int& tn) {
  const int per_group = G * tiles_n;
  const int group = t / per_group;
  const int first = group * G;
  const int gm = min(tiles_m - first, G);
  const int r = t - group * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

// The same for the lower triangle (tile t in row-major triangle order): the group of
// tile-rows R0 .. R0+gm-1 is taken column by column; columns 0 .. R0 hold gm tiles
// each, column R0+k (k >= 1) holds the gm-k tiles on or below the diagonal.
__device__ __forceinline__ void lower_tile_grouped(int t, int tiles, int G, int& tm, int& tn) {
  int r, c;
  tri_decode(t, r, c);
  const int R0 = (r / G) * G;
  const int gm = min(G, tiles - R0);
  int idx = t - R0 * (R0 + 1) / 2;
  const int full = (R0 + 1) * gm;
  if (idx < full) {
    // a whole group (every one but possibly the last) divides by the constant G
    const int q = gm == G ? idx / G : idx / gm;
    tn = q;
    tm = R0 + idx - q * gm;
  } else {
    idx -= full;
    int k = 1;
    while (idx >= gm - k) {
      idx -= gm - k;
      ++k;
    }
    tn = R0 + k;
    tm = R0 + k + idx;
  }
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i runs on XCD i % 8),
// and each XCD has its own L2.  Give XCD x one contiguous range of logical ids so the
// tiles it runs share operand panels (and, for batched problems, whole matrices).
__device__ __forceinline__ int xcd_remap(int L, int total) {
  constexpr int kXcds = 8;
  const int xcd = L % kXcds, idx = L / kXcds;
  const int per = total / kXcds, rem = total % kXcds;
  return xcd * per + min(xcd, rem) + idx;
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
    if constexpr (TIn::kId == GNS_F16 && TB::kId == GNS_BF16) {
      // bf16 -> fp32 is a bit shift (low half) or a mask (high half); the product with
      // mul is rounded to fp16 straight into the low / high half of one register
      typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        half2_t h;
        h.x = (_Float16)(__uint_as_float(w[i] << 16) * mul);
        h.y = (_Float16)(__uint_as_float(w[i] & 0xffff0000u) * mul);
        w[i] = __builtin_bit_cast(uint32_t, h);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo = TIn::from_f32(TB::to_f32(w[i] & 0xffffu) * mul);
        uint32_t hi = TIn::from_f32(TB::to_f32(w[i] >> 16) * mul);
        w[i] = lo | (hi << 16);
      }
    }
    return c;
  }
}

// Epilogue element group: row gm, columns gn .. gn+3 of the output tile.
// v = alpha' acc + beta C + gamma [diag] is written to D;
// symmetric outputs write the lower-triangle elements and their mirror images, so D
// is bitwise symmetric.  N % 4 == 0, so gn < N covers gn .. gn+3.
template <class TOut, bool LOWER>
__device__ __forceinline__ void emit_row4(const GemmParams& p, uint8_t* Db, const uint8_t* Cb,
                                          float alpha, int gm, int gn, const float* a4) {
  if (gm >= p.M || gn >= p.N) return;
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = alpha * a4[e];
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
  }
}

struct EpiPtrs {
  uint8_t* D;
  const uint8_t* C;
  float alpha;
  int c_planes, d_planes;     // 1, or 2 for a hi/lo pair of planes
};

// The Frobenius scale of batch entry bz from its partial sums of squares (at most
// 1024): lane l adds partials l, l + 64, ... in order, then an xor butterfly, whose
// result is bitwise the same in every lane (each level adds the same two values in
// either order), so every wave and workgroup forms the same s.  The loads are split
// from the sum so a kernel can issue them first and form s after its k-loop: all 16
// are issued at once, without branches (indices past n_partials load the last partial
// and count as zero).
constexpr int kPartialsPerLane = kMaxPartials / 64;
__device__ __forceinline__ void load_partials(const GemmParams& p, int bz, float (&v)[kPartialsPerLane]) {
  const int lane = threadIdx.x & 63;
  const float* q = p.partials + (size_t)bz * p.n_partials;
#pragma unroll
  for (int r = 0; r < kPartialsPerLane; ++r) v[r] = q[min(lane + 64 * r, p.n_partials - 1)];
}
__device__ __forceinline__ float scale_of_partials(const GemmParams& p, const float (&v)[kPartialsPerLane]) {
  const int lane = threadIdx.x & 63;
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < kPartialsPerLane; ++r) t += lane + 64 * r < p.n_partials ? v[r] : 0.0f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
  return 1.0f / (sqrtf(t) + p.eps);
}
// 1 when the launch has no partials
__device__ __forceinline__ float scale_from_partials(const GemmParams& p, int bz) {
  if (!p.partials) return 1.0f;
  float v[kPartialsPerLane];
  load_partials(p, bz, v);
  return scale_of_partials(p, v);
}
// tile 0 of each batch entry publishes the scale (read by later launches only)
__device__ __forceinline__ void publish_scale(const GemmParams& p, int bz, int tile, bool second, float psc) {
  if (p.partials && p.s_out && !second && tile == 0 && threadIdx.x == 0) p.s_out[bz] = psc;
}

template <class TOut>
__device__ __forceinline__ EpiPtrs epi_ptrs(const GemmParams& p, int bz, bool second, float psc) {
  EpiPtrs e;
  e.alpha = p.alpha;
  if (p.partials) {
    for (int i = 0; i < p.alpha_pow; ++i) e.alpha *= psc;
  } else if (p.scale) {
    for (int i = 0; i < p.alpha_pow; ++i) e.alpha *= p.scale[bz];
  }
  void* D = second ? p.Dp : p.D;
  const void* C = second ? p.C2 : p.C;
  e.D = reinterpret_cast<uint8_t*>(D) + (size_t)bz * p.sD * TOut::kBytes;
  e.C = C ? reinterpret_cast<const uint8_t*>(C) + (size_t)bz * p.sC * TOut::kBytes : nullptr;
  e.c_planes = second ? p.c2_planes : p.c_planes;
  e.d_planes = second ? p.dp_planes : p.d_planes;
  return e;
}

// Flat workgroup id -> (batch entry, second product of a pair, tile), with the XCD
// remap applied over all batch * tiles (* 2 for a pair) workgroups; psc is the scale
// formed from partial sums (1 without; with_scale false leaves it to the caller).
// The divisions by run-time counts are skipped when there is one K range or one
// (batch entry, product), the common cases.
struct GridPos {
  int bz, tile, ks;     // ks: K range of a split partial launch (0 otherwise)
  bool second;
  float psc;
};
__device__ __forceinline__ GridPos grid_pos(const GemmParams& p, bool with_scale = true) {
  const int splits = (p.ksplit > 1 && !p.reduce) ? p.ksplit : 1;
  const int entries = p.batch * (p.pair ? 2 : 1);
  const int total = entries * p.tiles * splits;
  const int rid0 = xcd_remap((int)blockIdx.x, total);
  GridPos g;
  int rid = rid0;
  g.ks = 0;
  if (splits > 1) {
    g.ks = __builtin_amdgcn_readfirstlane(rid0 % splits);
    rid = rid0 / splits;
  }
  int bz = 0;
  g.tile = rid;
  if (entries > 1) {
    bz = __builtin_amdgcn_readfirstlane(rid / p.tiles);
    g.tile = __builtin_amdgcn_readfirstlane(rid - bz * p.tiles);
  }
  g.second = p.pair && bz >= p.batch;
  if (g.second) bz -= p.batch;
  g.bz = bz;
  g.psc = 1.0f;
  if (with_scale) {
    g.psc = scale_from_partials(p, bz);
    publish_scale(p, bz, g.tile, g.second, g.psc);
  }
  return g;
}

// 16x16 fragments (v_mfma_f32_16x16x*, operands passed swapped): lane l owns row
// (l % 16) and columns 4 (l / 16) + e of each fragment.
template <class TOut, bool LOWER, int FM, int FN>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x4_t (&acc)[FM][FN], const GridPos& gp, int mw,
                                         int nw, int lane) {
  const int bz = gp.bz;
  const EpiPtrs e = epi_ptrs<TOut>(p, bz, gp.second, gp.psc);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float a4[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      emit_row4<TOut, LOWER>(p, e.D, e.C, e.alpha, mw + i * 16 + (lane & 15), nw + j * 16 + 4 * (lane >> 4), a4);
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
  constexpr int NN_TOTAL = (BK / 4) * NN_COLS;         // NN: 4(k) x EPC(n) blocks per tile
  constexpr int NN_BLOCKS = (NN_TOTAL + NT - 1) / NT;  // ... per thread
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(!LOWER || BM == BN, "symmetric tiles must be square");

  extern __shared__ __align__(16) uint4 smem[];
  uint4* As = smem;                      // [2][BM][8]
  uint4* Bs = smem + 2 * BM * 8;         // [2][BN][8]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // one flat grid over (batch, tile), remapped so each XCD gets a contiguous range
  const GridPos gp = grid_pos(p);
  const int bz = gp.bz, tile = gp.tile;
  int tm, tn;
  if constexpr (LOWER) {
    tri_decode(tile, tm, tn);
  } else {
    tm = tile / p.tiles_n;
    tn = tile % p.tiles_n;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;

  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(gp.second ? p.A2 : p.A) + (size_t)bz * p.sA * TIn::kBytes;
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(p.B) + (size_t)bz * p.sB * TB::kBytes;

  float bmul = 1.0f;
  if constexpr (NN && TIn::kId != TB::kId) {
    bmul = p.b_mul;
    if (p.scale) for (int i = 0; i < p.b_pow; ++i) bmul *= p.scale[bz];
  }

  uint4 ra[A_LOADS];
  uint4 rb[NN ? 4 * NN_BLOCKS : B_LOADS_NT];

  // Buffer resources over this matrix's operands: out-of-range rows/columns load as
  // zero without branches (the extents are checked to be < 2 GiB on the host).
  const auto rsA = make_rsrc(Ab, (uint32_t)(((size_t)(M - 1) * p.lda + K) * TIn::kBytes));
  const auto rsB = NN ? make_rsrc(Bb, (uint32_t)(((size_t)(K - 1) * p.ldb + N) * TB::kBytes))
                      : make_rsrc(Bb, (uint32_t)(((size_t)(N - 1) * p.ldb + K) * TB::kBytes));

  auto load_a = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int c = tid + i * NT, row = c >> 3, ch = c & 7;
      const int gr = m0 + row, gk = k0 + ch * EPC;
      const uint32_t off = (gr < M && gk < K) ? (uint32_t)(((size_t)gr * p.lda + gk) * TIn::kBytes) : kOutOfRange;
      ra[i] = buffer_load16(rsA, off);
    }
  };
  auto load_b = [&](int k0) {
    if constexpr (!NN) {
#pragma unroll
      for (int i = 0; i < B_LOADS_NT; ++i) {
        const int c = tid + i * NT, row = c >> 3, ch = c & 7;
        const int gr = n0 + row, gk = k0 + ch * EPC;
        const uint32_t off = (gr < N && gk < K) ? (uint32_t)(((size_t)gr * p.ldb + gk) * TB::kBytes) : kOutOfRange;
        rb[i] = buffer_load16(rsB, off);
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
          const uint32_t off = (t < NN_TOTAL && gk < K && gn < N)
                                   ? (uint32_t)(((size_t)gk * p.ldb + gn) * TB::kBytes) : kOutOfRange;
          rb[blk * 4 + r] = buffer_load16(rsB, off);
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
        if (NN_TOTAL % NT != 0 && t >= NN_TOTAL) break;
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

  epilogue<TOut, LOWER, FM, FN>(p, acc, gp, m0 + wm * Cfg::kWM, n0 + wn * Cfg::kWN, lane);
}


// ---------------------------------------------------------------------------------
// 16-bit kernel (fp16 / bf16 operands) on v_mfma_f32_32x32x16.  On gfx950 this MFMA
// shape runs at the full dense rate (measured 2405 TFLOP/s chip-wide), while
// v_mfma_f32_16x16x32 issues at half rate (1266 TFLOP/s), so all 16-bit products use
// 32x32 fragments.
//
// Operands go from HBM straight into LDS with buffer loads carrying the LDS flag (no
// staging registers).  They are issued through inline assembly, so the compiler does
// not track them and does not make every later LDS read wait for them; the kernel
// waits with explicit vmcnt counts for exactly the stage it is about to read, and
// the loads of younger stages stay in flight.
//
// LDS ring of STAGES slots, each one k-stage of 32 k values: the A tile as
// [BM rows][64 B] (16-byte chunks swizzled by swz64()); the B tile the same (NT) or,
// for the rectangular product, X's natural layout [BK rows (k)][BN * 2 B] with
// 16-byte chunks XOR-ed by nn_swz(k).  NN fragments are read with
// ds_read_b64_tr_b16: lane i of a 16-lane group passes the address of row k0 + i/4,
// columns n0 + 4 (i % 4) .. +3 and receives column n0 + i at rows k0 .. k0+3 -- an
// MFMA operand column (verified on gfx950).
//
// Per stage each wave runs 2 k-steps of 16; fragments alternate between two register
// sets so the LDS reads of one k-step overlap the MFMAs of the other, and the barrier
// that publishes the next stage sits between the two halves of the second k-step's
// MFMAs, which cover the first LDS reads of the next stage.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef int int4v_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ uint2 lds_read_tr16(const void* lds) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)lds);
  return __builtin_bit_cast(uint2, v);
}

// raw buffer descriptor of [base, base + bytes) in scalar registers
__device__ __forceinline__ int4v_t sgpr_rsrc(const void* base, uint32_t bytes) {
  const unsigned long long b = (unsigned long long)base;
  int4v_t r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r.y = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at voffset into LDS at lds_addr + 16 * lane;
// offsets past the end of the buffer write zeros.
__device__ __forceinline__ void dma16(int4v_t rsrc, uint32_t lds_addr, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_addr), "v"(voffset), "s"(rsrc) : "memory", "m0");
}

template <class T>
__device__ __forceinline__ void mfma32_step(f32x16_t& acc, const uint4& a, const uint4& b) {
  if constexpr (T::kId == GNS_BF16) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                 __builtin_bit_cast(bf16x8_t, a), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, b),
                                                __builtin_bit_cast(f16x8_t, a), acc, 0, 0, 0);
  }
}

// s_waitcnt immediate (gfx9 family) that waits until at most `vm` vector-memory
// instructions of this wave are outstanding, leaving the other counters alone.
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | (0x7 << 4) | (0xF << 8) | (((vm >> 4) & 0x3) << 14); }
// ... and until at most `n` LDS / scalar-memory operations are outstanding
constexpr int waitcnt_lgkm(int n) { return 0xF | (0x7 << 4) | ((n & 0xF) << 8) | (0x3 << 14); }

// Wait until at most `later` stages of LOADS loads each are outstanding (later is
// uniform, 0 .. L).  s_waitcnt takes an immediate, hence one scalar branch per count.
template <int L, int LOADS>
__device__ __forceinline__ void wait_vm_stages(int later) {
  if constexpr (L <= 0) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  } else {
    if (later >= L) __builtin_amdgcn_s_waitcnt(waitcnt_vm(L * LOADS));
    else wait_vm_stages<L - 1, LOADS>(later);
  }
}

// Workgroup barrier that is also a compiler memory barrier (no LDS access moves
// across it) but, unlike __syncthreads(), adds no waits on outstanding loads: the
// kernel waits for exactly the stage it needs before calling it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BK>
struct Tile32 {
  static constexpr int kThreads = 64 * WAVES_M * WAVES_N;
  static constexpr int kWM = BM / WAVES_M;
  static constexpr int kWN = BN / WAVES_N;
  static constexpr int kFM = kWM / 32;
  static constexpr int kFN = kWN / 32;
  static constexpr int kStages = STAGES;      // LDS ring depth
  static constexpr int kBK = BK;              // k values per stage (rows of BK * 2 bytes)
  static constexpr int kLdsBytes = kStages * (BM + BN) * kBK * 2;
};

// 64-byte LDS rows (4 chunks): 16 rows read at the same logical chunk land in 16
// distinct 16-byte slots of the 256-byte bank window (rows 4j .. 4j+3 share a window
// and sit in different quarters; j selects the chunk within the quarter).
__device__ __forceinline__ int swz64(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// physical chunk of logical chunk c in row r of a K-contiguous tile with BK values per
// row.  With 256-byte rows (BK = 128) a row fills the whole bank window, so the 16
// rows of a fragment read take slots c ^ (r mod 16): 16 distinct 16-byte slots.
template <int BK>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  if constexpr (BK == 32) return swz64(row, chunk);
  else if constexpr (BK == 64) return swz(row, chunk);
  else return chunk ^ (row & 15);
}

// 16 bytes of TOut elements <-> fp32 values
template <class TOut>
__device__ __forceinline__ void unpack16(const uint4& c, float (&v)[16 / TOut::kBytes]) {
#pragma unroll
  for (int e = 0; e < 16 / TOut::kBytes; ++e) v[e] = chunk_elem<TOut>(c, e);
}
template <class TOut>
__device__ __forceinline__ uint4 pack16(const float (&v)[16 / TOut::kBytes]) {
  uint4 r;
  uint32_t* w = reinterpret_cast<uint32_t*>(&r);
  if constexpr (TOut::kBytes == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(v[e]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = TOut::from_f32(v[2 * i]) | (TOut::from_f32(v[2 * i + 1]) << 16);
  }
  return r;
}

// Write the 16-byte vector v to row `row`, columns col .. col+VE-1, keeping only the
// elements whose column c satisfies lo <= c - col (all of them when lo <= 0) and
// c - col <= hi (all when hi >= VE - 1): full vectors take one 16-byte store.
template <class TOut>
__device__ __forceinline__ void store_vec(uint8_t* base, long long ld, int row, int col, const float (&v)[16 / TOut::kBytes],
                                          int lo, int hi) {
  constexpr int VE = 16 / TOut::kBytes;
  const long long off = (long long)row * ld + col;
  if (lo <= 0 && hi >= VE - 1) {
    *reinterpret_cast<uint4*>(base + off * TOut::kBytes) = pack16<TOut>(v);
  } else {
#pragma unroll
    for (int e = 0; e < VE; ++e)
      if (e >= lo && e <= hi) store1<TOut>(base, off + e, v[e]);
  }
}

// store_vec of v into a matrix of `planes` planes: with 2, hi = round(v) goes to
// base and lo = round(v - hi) to base + plane elements (v - hi is exact in fp32).
template <class TOut>
__device__ __forceinline__ void store_planes(uint8_t* base, long long ld, int row, int col,
                                             const float (&v)[16 / TOut::kBytes], int lo, int hi, int planes,
                                             long long plane) {
  constexpr int VE = 16 / TOut::kBytes;
  if constexpr (TOut::kBytes == 2) {
    if (planes == 2) {
      float h[VE], l[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        h[e] = TOut::to_f32(TOut::from_f32(v[e]));
        l[e] = v[e] - h[e];
      }
      store_vec<TOut>(base, ld, row, col, h, lo, hi);
      store_vec<TOut>(base + plane * TOut::kBytes, ld, row, col, l, lo, hi);
      return;
    }
  }
  store_vec<TOut>(base, ld, row, col, v, lo, hi);
}

typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
// store_vec of a whole 16-byte vector with a non-temporal store (no cache allocation)
template <class TOut>
__device__ __forceinline__ void store_vec_nt(uint8_t* base, long long ld, int row, int col,
                                             const float (&v)[16 / TOut::kBytes]) {
  const uint4 q = pack16<TOut>(v);
  const u32x4_nt x = {q.x, q.y, q.z, q.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_nt*>(base + ((long long)row * ld + col) * TOut::kBytes));
}

// Epilogue of gemm16_kernel, staged through LDS (called after a workgroup barrier:
// the operand ring is free).  Each wave takes its WM x WN sub-tile in slabs of 32
// rows (one fragment row): the raw fp32 accumulators go to a per-wave slab
// [32][WN + 4] (the padding spreads the 16 rows of a 128-bit access over distinct
// banks); the row pass forms v = alpha acc + beta C + gamma [diagonal] for 16-byte
// vectors along the output rows, stores them with coalesced 16-byte writes and puts
// v back in the slab; for a symmetric output the
// mirror pass reads the slab down its columns and writes the strictly-lower elements
// at their transposed positions.  Both triangles round the same fp32 value, so the
// output is bitwise symmetric.  Only the slab writes index the accumulators, so
// they stay in registers.
// The C vectors one lane adds in the row pass of one 32-row fragment row of a wave
// tile FN * 32 columns wide (both planes of a hi/lo pair), as whole 16-byte vectors.
template <class TOut, int FN, bool PL>
struct CRow {
  static constexpr int VE = 16 / TOut::kBytes;                 // elements per vector
  static constexpr int RV = FN * 32 / VE;                      // vectors per row
  static constexpr int IT = (32 * RV + 63) / 64;               // vectors per lane
  static constexpr int CPL = PL ? 2 : 1;
  uint4 v[IT][CPL];
};

// Load the C vectors of fragment row r0 (wave column nw).  A vector outside the matrix
// loads C's first vector instead, so every lane issues the same loads with no branch
// around them, and they all stay in flight together.
template <class TOut, int FN, bool PL>
__device__ __forceinline__ void load_c_row(const GemmParams& p, const EpiPtrs& ep, int r0, int nw, int lane,
                                           CRow<TOut, FN, PL>& cb) {
  using CR = CRow<TOut, FN, PL>;
#pragma unroll
  for (int it = 0; it < CR::IT; ++it) {
    const int t = lane + 64 * it;
    const int gm = r0 + t / CR::RV, gn = nw + (t % CR::RV) * CR::VE;
    const bool in = t < 32 * CR::RV && gm < p.M && gn < p.N;
    const uint8_t* cp = ep.C + (in ? ((long long)gm * p.ldc + gn) * TOut::kBytes : 0);
    cb.v[it][0] = *reinterpret_cast<const uint4*>(cp);
    if constexpr (PL) cb.v[it][1] = *reinterpret_cast<const uint4*>(cp + (ep.c_planes == 2 ? p.plane * TOut::kBytes : 0));
  }
}

// EARLY: the caller loaded C's first fragment row into c0 before its k-loop.
template <class TOut, bool LOWER, int FM, int FN, bool NT = false, bool PL = false, bool EARLY = false>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, f32x16_t (&acc)[FM][FN], const GridPos& gp,
                                             int mw, int nw, int lane, float* slab, const CRow<TOut, FN, PL>& c0) {
  const int bz = gp.bz;
  constexpr int WN = FN * 32;
  constexpr int S = WN + 4;
  constexpr int VE = 16 / TOut::kBytes;          // output elements per 16-byte vector
  constexpr int RV = WN / VE;                    // vectors per slab row
  constexpr int MV = 32 / VE;                    // vectors per mirrored row
  const EpiPtrs ep = epi_ptrs<TOut>(p, bz, gp.second, gp.psc);
  const bool has_c = ep.C != nullptr && p.beta != 0.0f;
  const int M = p.M, N = p.N;
  const int c_pl = PL ? ep.c_planes : 1, d_pl = PL ? ep.d_planes : 1;   // hi/lo planes (PL kernels only)
  // The C vectors of a fragment row are all loaded one fragment row ahead of the row
  // pass that adds them (the first row before the k-loop, or here), so their latency
  // overlaps the staging and stores of the row before instead of being paid once per
  // vector.
  using CR = CRow<TOut, FN, PL>;
  constexpr int IT = CR::IT, CPL = CR::CPL;
  CR cbuf[2];
  if constexpr (EARLY) cbuf[0] = c0;
  else if (has_c) load_c_row<TOut, FN, PL>(p, ep, mw, nw, lane, cbuf[0]);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r0 = mw + 32 * i;
    if (has_c && i + 1 < FM) load_c_row<TOut, FN, PL>(p, ep, r0 + 32, nw, lane, cbuf[(i + 1) & 1]);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(slab + (lane & 31) * S + j * 32 + 8 * q + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // row pass
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int t = lane + 64 * it;
      const int r = t / RV, c = (t % RV) * VE;
      const int gm = r0 + r, gn = nw + c;
      if (t >= 32 * RV || gm >= M || gn >= N) continue;   // N % 8 == 0: a vector is all in or all out
      float* sp = slab + r * S + c;
      float v[VE];
#pragma unroll
      for (int e = 0; e < VE; e += 4) {
        const float4 f = *reinterpret_cast<const float4*>(sp + e);
        v[e] = ep.alpha * f.x; v[e + 1] = ep.alpha * f.y; v[e + 2] = ep.alpha * f.z; v[e + 3] = ep.alpha * f.w;
      }
      if (has_c) {
        float cv[VE];
        unpack16<TOut>(cbuf[i & 1].v[it][0], cv);
        if constexpr (PL) {
          if (c_pl == 2) {      // C = hi + lo
            float cl[VE];
            unpack16<TOut>(cbuf[i & 1].v[it][CPL - 1], cl);
#pragma unroll
            for (int e = 0; e < VE; ++e) cv[e] += cl[e];
          }
        }
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] += p.beta * cv[e];
      }
      if (p.gamma != 0.0f) {
#pragma unroll
        for (int e = 0; e < VE; ++e)
          if (gn + e == gm) v[e] += p.gamma;
      }
      const int hi = LOWER ? gm - gn : VE - 1;   // symmetric: columns up to the diagonal
      if (hi >= 0) {
        if (NT && hi >= VE - 1 && d_pl == 1) store_vec_nt<TOut>(ep.D, p.ldd, gm, gn, v);
        else store_planes<TOut>(ep.D, p.ldd, gm, gn, v, 0, hi, d_pl, p.plane);
      }
      if constexpr (LOWER) {
#pragma unroll
        for (int e = 0; e < VE; e += 4) *reinterpret_cast<float4*>(sp + e) = make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]);
      }
    }

    if constexpr (LOWER) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // mirror pass: output row gn = nw + c, columns gm0 .. gm0+VE-1 from slab column c
#pragma unroll
      for (int it = 0; it < (WN * MV + 63) / 64; ++it) {
        const int t = lane + 64 * it;
        const int c = t / MV, rr = (t % MV) * VE;
        const int gn = nw + c, gm0 = r0 + rr;
        if (t >= WN * MV || gn >= N || gm0 >= M) continue;   // M % 8 == 0 and gm0 % VE == 0
        const int lo = gn + 1 - gm0;             // strictly lower sources: gm0 + e > gn
        if (lo > VE - 1) continue;
        float v[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] = slab[(rr + e) * S + c];
        store_planes<TOut>(ep.D, p.ldd, gn, gm0, v, lo, VE - 1, d_pl, p.plane);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// A 128 x 128 wave tile keeps 256 fp32 accumulators per lane: such configurations
// run one wave per SIMD with the full 512-register file (accumulators in AGPRs).
template <int BM, int BN, int WAVES_M, int WAVES_N>
constexpr int max_waves_per_eu() { return (BM / WAVES_M) * (BN / WAVES_N) >= 128 * 128 ? 1 : 8; }

template <class TIn, class TB, class TOut, int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int BKV, bool LOWER,
          bool NN, bool NT = false, bool PL = false, bool IDX = false>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
__attribute__((amdgpu_waves_per_eu(1, max_waves_per_eu<BM, BN, WAVES_M, WAVES_N>())))
gemm16_kernel(GemmParams p) {
  static_assert(TIn::kBytes == 2 && TB::kBytes == 2, "16-bit operands only");
  static_assert(!LOWER || (BM == BN && !NN), "symmetric tiles are square NT tiles");
  using Cfg = Tile32<BM, BN, WAVES_M, WAVES_N, STAGES, BKV>;
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int FM = Cfg::kFM, FN = Cfg::kFN;
  static_assert(FM >= 1 && FN >= 1, "wave tile must be a multiple of 32");
  constexpr int NS = Cfg::kStages, BK = Cfg::kBK;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  constexpr int A_INSTR = A_BYTES / (1024 * NW), B_INSTR = B_BYTES / (1024 * NW);   // 1 KB per wave instruction
  constexpr int LOADS = A_INSTR + B_INSTR;                                           // per wave per stage
  constexpr int NCH = BN / 8;                                                        // NN: chunks per k row
  // NN B tile: physical 16-byte chunk of logical chunk c in k-row kr is c ^ nn_swz(kr).
  // A transposing fragment read has 32 lanes on 4 consecutive k-rows x 4 chunks; with
  // 128-byte rows (BN = 64) consecutive rows already sit in opposite halves of the
  // 256-byte bank window and 2 (kr & 3) separates the rest, while rows of 256 bytes or
  // more overlay the same banks and need 4 (kr & 3) to put the 4 rows in 4 disjoint
  // 64-byte groups.
  auto nn_swz = [](int kr) { return NCH >= 16 ? 4 * (kr & 3) : 2 * (kr & 3); };
  constexpr int CPR = BK / 8;                                                        // NT: chunks per tile row
  constexpr int KS = BK / 16;                                                        // MFMA k-steps per stage
  static_assert(BK == 32 || BK == 64 || BK == 128, "stage depth");
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "tile/wave mismatch");
  static_assert(!NN || NCH >= 8, "NN tiles need >= 64 columns");
  static_assert(NS >= 2 && LOADS * (NS - 1) < 64, "ring depth / vmcnt range");

  extern __shared__ __align__(16) uint8_t smem16[];
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)smem16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // block-level indices are uniform; readfirstlane keeps them in scalar registers.
  // The Frobenius scale of a product with partial sums only enters the epilogue: up
  // to 128 x 128 tiles its loads are issued here and s is formed after the k-loop
  // (the 256 x 256 tile forms it first: a microsecond of setup is small beside its
  // products, and its registers stay for the ping-pong schedule).
  constexpr bool kDeferScale = BM <= 128;
  GridPos gp = grid_pos(p, !kDeferScale);
  const int bz = gp.bz, tile = gp.tile;
  const bool defer_scale = kDeferScale && p.partials != nullptr && !(p.ksplit > 1 && !p.reduce);
  float pv[kDeferScale ? kPartialsPerLane : 1];
  if constexpr (kDeferScale) {
    if (defer_scale) load_partials(p, bz, pv);
  }
  int tm, tn;
  constexpr int kGroup = BM >= 256 ? 4 : 8;
  if constexpr (LOWER) {
    lower_tile_grouped(tile, p.tiles_m, kGroup, tm, tn);
  } else {
    rect_tile_grouped(tile, p.tiles_m, p.tiles_n, kGroup, tm, tn);
  }
  const int m0 = __builtin_amdgcn_readfirstlane(tm * BM), n0 = __builtin_amdgcn_readfirstlane(tn * BN);
  const int M = p.M, N = p.N, K = p.K;
  // K range of this workgroup: all of K, or one range of a split partial launch
  const bool split_part = p.ksplit > 1 && !p.reduce;
  const int kbeg = split_part ? gp.ks * p.kchunk : 0;
  const int kend = split_part ? min(K, kbeg + p.kchunk) : K;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(gp.second ? p.A2 : p.A) + (size_t)bz * p.sA * 2;
  const uint8_t* Bb = reinterpret_cast<const uint8_t*>(p.B) + (size_t)bz * p.sB * 2;
  // hi/lo planes of the operands: the K loop runs once per plane pair (hi.hi, then
  // hi.lo, then lo.hi), KTp stages each
  // (only the PL instantiation reads the plane counts; the others run one pair)
  const int a_pl = PL ? (gp.second ? p.a2_planes : p.a_planes) : 1, b_pl = PL ? p.b_planes : 1;
  const int npairs = (a_pl == 2 && b_pl == 2) ? 3 : a_pl * b_pl;
  const uint32_t plane_bytes = (uint32_t)(p.plane * 2);
  // an indexed operand spans its whole source matrix (src_rows rows)
  const int a_rows_span = (IDX && !NN) ? p.src_rows : M;
  const int b_rows_span = IDX ? p.src_rows : (NN ? K : N);
  const int4v_t rsA = sgpr_rsrc(Ab, (uint32_t)(((size_t)(a_rows_span - 1) * p.lda + K + (a_pl - 1) * p.plane) * 2));
  const int4v_t rsB = NN ? sgpr_rsrc(Bb, (uint32_t)(((size_t)(b_rows_span - 1) * p.ldb + N) * 2))
                         : sgpr_rsrc(Bb, (uint32_t)(((size_t)(b_rows_span - 1) * p.ldb + K + (b_pl - 1) * p.plane) * 2));
  const int KTp = (kend - kbeg + BK - 1) / BK;       // stages per plane pair
  const int KT = KTp * npairs;
  float bmul = 1.0f;
  if constexpr (NN && TIn::kId != TB::kId) {
    bmul = p.b_mul;
    if (p.scale) for (int i = 0; i < p.b_pow; ++i) bmul *= p.scale[bz];
  }

  // Indexed X rows.  Symmetric product: each lane's operand rows are the same in every
  // stage, so their source offsets are looked up once here.  Rectangular product: the
  // B rows change with the stage, so the batch entry's row table is copied into LDS
  // after the ring (before any operand load; every wave waits for it and a barrier
  // publishes it).
  constexpr int XA = (IDX && !NN) ? A_INSTR : 1, XB = (IDX && !NN) ? B_INSTR : 1;
  uint32_t a_roff[XA], b_roff[XB];
  bool a_rok[XA], b_rok[XB];
  const int* tbl = nullptr;
  if constexpr (IDX) {
    const int* rws = p.rows + (size_t)bz * p.rows_stride;
    if constexpr (!NN) {
#pragma unroll
      for (int g = 0; g < XA; ++g) {
        const int gr = m0 + ((g * NW + wave) * 64 + lane) / CPR;
        const int pr = gr < p.rows_valid ? rws[gr] : -1;
        a_rok[g] = pr >= 0 && pr < p.src_rows;
        a_roff[g] = a_rok[g] ? (uint32_t)((size_t)pr * p.lda * 2) : 0u;
      }
#pragma unroll
      for (int g = 0; g < XB; ++g) {
        const int gr = n0 + ((g * NW + wave) * 64 + lane) / CPR;
        const int pr = gr < p.rows_valid ? rws[gr] : -1;
        b_rok[g] = pr >= 0 && pr < p.src_rows;
        b_roff[g] = b_rok[g] ? (uint32_t)((size_t)pr * p.ldb * 2) : 0u;
      }
    } else {
      const int4v_t rsT = sgpr_rsrc(rws, (uint32_t)p.rows_valid * 4u);
      const int instrs = (p.rows_valid * 4 + 1023) / 1024;
      for (int i = wave; i < instrs; i += NW)
        dma16(rsT, __builtin_amdgcn_readfirstlane(lds0 + NS * STAGE + i * 1024), (uint32_t)(i * 64 + lane) * 16u);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
      tbl = reinterpret_cast<const int*>(smem16 + NS * STAGE);
    }
  }

  // load g (0 .. LOADS-1) of k-stage kt: one direct HBM -> LDS instruction (1 KB per
  // wave) into ring slot kt % NS; loads 0 .. A_INSTR-1 fill the A tile, the rest B
  // source row of B load gb (0 .. B_INSTR-1) of stage kt of an indexed rectangular
  // product (-1: a zero row)
  auto nn_row = [&](int kt, int gb) -> int {
    if constexpr (IDX && NN) {
      const int kr = ((gb * NW + wave) * 64 + lane) / NCH;
      const int gk = kbeg + kt * BK + kr;
      return (kt < KT && gk < p.rows_valid) ? tbl[gk] : -1;
    } else {
      return -1;
    }
  };
  auto issue_load = [&](int kt, int g, int pre_row = -2) {
    // plane pair of stage kt and its K offset; stages at or past KT load nothing
    // (one pair: stages past the end have k0 >= kend, so their offsets are out of range)
    const int pi = PL ? (kt >= KTp) + (kt >= 2 * KTp) : 0;
    const int k0 = kbeg + (kt - pi * KTp) * BK;
    const bool live = PL ? kt < KT : true;
    const uint32_t a_add = (PL && pi > 0 && pi == npairs - 1 && a_pl == 2) ? plane_bytes : 0u;
    const uint32_t b_add = (PL && pi == 1 && b_pl == 2) ? plane_bytes : 0u;
    const uint32_t sb = lds0 + (kt % NS) * STAGE;
    if (g < A_INSTR) {
      const int blk = g * NW + wave;
      const int q = blk * 64 + lane;                      // LDS chunk this lane fills
      const int row = q / CPR, lc = swz_k<BK>(row, q % CPR);
      const int gr = m0 + row, gk = k0 + lc * 8;
      uint32_t off;
      if constexpr (IDX && !NN)
        off = (live && a_rok[g] && gk < kend) ? a_roff[g] + (uint32_t)gk * 2u : kOutOfRange;
      else
        off = (live && gr < M && gk < kend) ? (uint32_t)(((size_t)gr * p.lda + gk) * 2) + a_add : kOutOfRange;
      dma16(rsA, __builtin_amdgcn_readfirstlane(sb + blk * 1024), off);
    } else {
      const int blk = (g - A_INSTR) * NW + wave;
      const int q = blk * 64 + lane;
      uint32_t off;
      if constexpr (!NN) {
        const int row = q / CPR, lc = swz_k<BK>(row, q % CPR);
        const int gr = n0 + row, gk = k0 + lc * 8;
        if constexpr (IDX)
          off = (live && b_rok[g - A_INSTR] && gk < kend) ? b_roff[g - A_INSTR] + (uint32_t)gk * 2u : kOutOfRange;
        else
          off = (live && gr < N && gk < kend) ? (uint32_t)(((size_t)gr * p.ldb + gk) * 2) + b_add : kOutOfRange;
      } else {
        const int kr = q / NCH, lc = (q % NCH) ^ nn_swz(kr);
        const int gk = k0 + kr, gn = n0 + lc * 8;
        if constexpr (IDX) {
          // k-row gk of B is source row tbl[gk] (rows past rows_valid are zeros), looked
          // up here or, in the ping-pong schedule, one memory phase ahead
          const int pr = pre_row >= -1 ? pre_row : ((live && gk < p.rows_valid) ? tbl[gk] : -1);
          off = (pr >= 0 && pr < p.src_rows && gn < N) ? (uint32_t)(((size_t)pr * p.ldb + gn) * 2) : kOutOfRange;
        } else {
          off = (live && gk < kend && gn < N) ? (uint32_t)(((size_t)gk * p.ldb + gn) * 2) : kOutOfRange;
        }
      }
      dma16(rsB, __builtin_amdgcn_readfirstlane(sb + A_BYTES + blk * 1024), off);
    }
  };
  auto issue_stage = [&](int kt) {
#pragma unroll
    for (int g = 0; g < LOADS; ++g) issue_load(kt, g);
  };

  // fragments of k-step ks (16 k values) of the stage in ring slot `slot`
  auto read_frags = [&](int slot, int ks, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const uint8_t* sb = smem16 + slot * STAGE;
    const uint4* as = reinterpret_cast<const uint4*>(sb);
    const int ch = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * Cfg::kWM + i * 32 + (lane & 31);
      fa[i] = as[row * CPR + swz_k<BK>(row, ch)];
    }
    if constexpr (!NN) {
      const uint4* bs = reinterpret_cast<const uint4*>(sb + A_BYTES);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * Cfg::kWN + j * 32 + (lane & 31);
        fb[j] = bs[row * CPR + swz_k<BK>(row, ch)];
      }
    } else {
      const uint16_t* bh = reinterpret_cast<const uint16_t*>(sb + A_BYTES);
      const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int nb = wn * Cfg::kWN + j * 32 + 16 * (g & 1) + 4 * (i16 & 3);
        uint2 h[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int kr = ks * 16 + 8 * (g >> 1) + 4 * hh + (i16 >> 2);
          const int pc = (nb >> 3) ^ nn_swz(kr);
          h[hh] = lds_read_tr16(bh + kr * BN + pc * 8 + (nb & 7));
        }
        fb[j] = convert_chunk<TIn, TB>(make_uint4(h[0].x, h[0].y, h[1].x, h[1].y), bmul);
      }
    }
  };

  auto mma = [&](f32x16_t (&acc)[FM][FN], const uint4 (&fa)[FM], const uint4 (&fb)[FN], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i < i0 || i >= i1) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma32_step<TIn>(acc[i][j], fa[i], fb[j]);
    }
  };

  // wait until k-stage `next` has landed; `last` is the last stage issued so far, and
  // the (last - next) stages issued after `next` may stay in flight (vmcnt counts
  // this wave's loads, which complete in issue order)
  auto wait_for_stage = [&](int next, int last) { wait_vm_stages<NS - 1, LOADS>(last - next); };

  // Wave tiles of one fragment row: the C vectors of the epilogue are loaded here,
  // before any operand load, so their latency hides behind the k-loop.  The ring's
  // vmcnt waits stay exact: these loads are older than every ring load, and a wave's
  // loads complete in issue order.
  constexpr bool kEarlyC = FM == 1;
  CRow<TOut, FN, PL> c_early;
  if constexpr (kEarlyC) {
    const EpiPtrs ep0 = epi_ptrs<TOut>(p, bz, gp.second, gp.psc);
    if (!split_part && ep0.C != nullptr && p.beta != 0.0f)
      load_c_row<TOut, FN, PL>(p, ep0, m0 + wm * Cfg::kWM, n0 + wn * Cfg::kWN, lane, c_early);
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fp32 partial accumulators of a split product, as float4 quads:
  // [tile][range][wave][fragment][quad][lane], so every access of a wave moves 1 KB
  // of consecutive bytes
  constexpr int QUADS = FM * FN * 4;
  auto part_ptr = [&](int ks) {
    return reinterpret_cast<float4*>(p.part) + ((((size_t)bz * p.tiles + tile) * p.ksplit + ks) * NW + wave) * (QUADS * 64);
  };
  if (p.reduce) {
    // sum of the ranges in order (reduce 2: already summed into range 0 by
    // launch_sum_ranges), then the ordinary epilogue; each range's loads are all
    // issued before any is added
    const int nsum = p.reduce == 2 ? 1 : p.ksplit;
    for (int ks = 0; ks < nsum; ++ks) {
      const float4* q = part_ptr(ks);
      float4 v[QUADS];
#pragma unroll
      for (int t = 0; t < QUADS; ++t) v[t] = q[t * 64 + lane];
#pragma unroll
      for (int t = 0; t < QUADS; ++t) {
        const int f = t / 4, c = t % 4;
        f32x16_t& a = acc[f / FN][f % FN];
        a[4 * c] += v[t].x; a[4 * c + 1] += v[t].y; a[4 * c + 2] += v[t].z; a[4 * c + 3] += v[t].w;
      }
    }
  } else {
  // Small wave tiles (few MFMAs per k-step) keep a whole stage of fragments in
  // registers, twice: the LDS reads of stage kt+1 then overlap all MFMAs of stage
  // kt instead of one k-step, which is what bounds them otherwise (one 32-cycle
  // MFMA per k-step against ~130 cycles of LDS latency).
  constexpr bool kStageFrags = 2 * KS * (FM + FN) * 4 <= 128;
  // Two waves per SIMD (8 waves, WAVES_M = 2): the waves of tile row 0 (waves 0..3,
  // one per SIMD) and of tile row 1 (waves 4..7) alternate between a compute phase
  // (all MFMAs of one stage from registers) and a memory phase (all fragment reads of
  // the next stage, plus this wave's share of the direct loads of a later stage), so
  // each SIMD's MFMA pipe is fed by one wave while the other reads LDS.
  constexpr bool kPingPong = NW == 8 && WAVES_M == 2 && NS >= 3;
  if constexpr (kPingPong) {
    // Phases are separated by workgroup barriers.  Group 1 reads stage i in phase 2i
    // and multiplies it in phase 2i+1; group 0 runs one phase behind (reads in 2i+1,
    // multiplies in 2i+2).  Stage i's ring slot is therefore free after phase 2i+1,
    // and the memory phase of stage i+1 (2i+2 or 2i+3) refills it with stage i+NS.
    // At the end of phase 2i+1 every wave waits for its loads of stage i+1, which the
    // barrier then publishes before group 1 reads it in phase 2i+2; the loads of the
    // NS-2 younger stages stay in flight.  Every wave executes the same number of
    // barriers (group 0 one extra at the start, group 1 one extra at the end).
    const int grp = wm;
    uint4 fa[KS][FM], fb[KS][FN];
    constexpr int kAhead = (NS - 2) * LOADS;
    // indexed B rows: looked up one memory phase ahead, so the LDS read of the row
    // table is done by the time the loads that use it are issued
    int b_pre[(IDX && NN) ? B_INSTR : 1];
    if constexpr (IDX && NN) {
#pragma unroll
      for (int gb = 0; gb < B_INSTR; ++gb) b_pre[gb] = nn_row(NS - 1, gb);
    }
    auto memory_phase = [&](int i) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) read_frags(i % NS, ks, fa[ks], fb[ks]);
      if constexpr (IDX && NN) {
#pragma unroll
        for (int g = 0; g < A_INSTR; ++g) issue_load(i + NS - 1, g);
#pragma unroll
        for (int gb = 0; gb < B_INSTR; ++gb) issue_load(i + NS - 1, A_INSTR + gb, b_pre[gb]);
#pragma unroll
        for (int gb = 0; gb < B_INSTR; ++gb) b_pre[gb] = nn_row(i + NS, gb);
      } else {
#pragma unroll
        for (int g = 0; g < LOADS; ++g) issue_load(i + NS - 1, g);
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));   // slot i % NS may be refilled after the barrier
    };
    auto compute_phase = [&]() {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mfma32_step<TIn>(acc[i][j], fa[ks][i], fb[ks][j]);
      __builtin_amdgcn_s_setprio(0);
    };
#pragma unroll
    for (int t = 0; t + 1 < NS; ++t) issue_stage(t);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAhead));
    lds_barrier();
    if (grp == 0) lds_barrier();
    for (int i = 0; i < KT; ++i) {
      memory_phase(i);
      if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAhead));
      lds_barrier();
      compute_phase();
      if (grp == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kAhead));
      lds_barrier();
    }
    if (grp == 1) lds_barrier();
  } else if constexpr (!kStageFrags) {
    constexpr int H = (FM + 1) / 2;     // fragment rows of the last k-step before / after the barrier
    constexpr int L = (KS - 1) & 1;     // fragment set of the last k-step
    static_assert(L == 1, "the last k-step's fragments must not sit in set 0");
    constexpr int TAIL = (FM - H) * FN; // MFMAs after the barrier
    constexpr int PER = TAIL > 0 ? (LOADS + TAIL - 1) / TAIL : LOADS;
    uint4 fa[2][FM], fb[2][FN];         // two fragment sets: k-step s in set s & 1
    // Stages at or past KT are issued like the others: all their offsets are out of
    // range, so they only write zeros into ring slots whose data is never used, and
    // every iteration runs the same code (NS - 1 younger stages in flight at each wait).
#pragma unroll
    for (int t = 0; t < NS; ++t) issue_stage(t);
    wait_for_stage(0, NS - 1);
    lds_barrier();
    read_frags(0, 0, fa[0], fb[0]);

    // Stage kt (ring slot kt % NS) holds its k-step 0 fragments in set 0 on entry:
    //   k-steps 0 .. KS-2: read the fragments of the next k-step, MFMAs of this one;
    //   last k-step: MFMAs of its first fragment rows; all LDS reads of this stage are
    //   now in registers (lgkmcnt 0); wait for stage kt+1; barrier -- stage kt+1 is
    //   visible and slot kt % NS is free in every wave; read k-step 0 of stage kt+1;
    //   the remaining MFMAs, with the loads of stage kt+NS (into the freed slot)
    //   issued between them so the MFMA pipe stays busy meanwhile.
    for (int kt = 0; kt < KT; ++kt) {
      const int slot = kt % NS;
#pragma unroll
      for (int ks = 0; ks + 1 < KS; ++ks) {
        read_frags(slot, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        mma(acc, fa[ks & 1], fb[ks & 1], 0, FM);
      }
      mma(acc, fa[L], fb[L], 0, H);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      wait_for_stage(kt + 1, kt + NS - 1);
      lds_barrier();
      read_frags((kt + 1) % NS, 0, fa[0], fb[0]);
#pragma unroll
      for (int t = 0; t < (TAIL > 0 ? TAIL : 1); ++t) {
        if constexpr (TAIL > 0) {
          const int i = H + t / FN, j = t % FN;
          mfma32_step<TIn>(acc[i][j], fa[L][i], fb[L][j]);
        }
#pragma unroll
        for (int r = 0; r < PER; ++r)
          if (t * PER + r < LOADS) issue_load(kt + NS, t * PER + r);
      }
    }
  } else {
    uint4 sa[2][KS][FM], sb[2][KS][FN];
    auto read_stage = [&](int slot, uint4 (&fa)[KS][FM], uint4 (&fb)[KS][FN]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) read_frags(slot, ks, fa[ks], fb[ks]);
    };
    constexpr int MMAS = KS * FM * FN;
    constexpr int PER2 = (LOADS + MMAS - 1) / MMAS;
    // One stage: its fragments are in set S; make stage kt+1 visible (its slot was
    // filled NS-1 stages ago) and free slot kt % NS (every wave has its stage-kt
    // fragments in registers); read stage kt+1 into set S^1; the MFMAs of stage kt
    // with the loads of stage kt+NS into the freed slot issued between them.
    auto stage_iter = [&](auto set_tag, int kt) {
      constexpr int S = decltype(set_tag)::value;
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      wait_for_stage(kt + 1, kt + NS - 1);
      lds_barrier();
      read_stage((kt + 1) % NS, sa[S ^ 1], sb[S ^ 1]);
#pragma unroll
      for (int t = 0; t < MMAS; ++t) {
        const int ks = t / (FM * FN), i = (t / FN) % FM, j = t % FN;
        mfma32_step<TIn>(acc[i][j], sa[S][ks][i], sb[S][ks][j]);
#pragma unroll
        for (int r = 0; r < PER2; ++r)
          if (t * PER2 + r < LOADS) issue_load(kt + NS, t * PER2 + r);
      }
    };
#pragma unroll
    for (int t = 0; t < NS; ++t) issue_stage(t);
    wait_for_stage(0, NS - 1);
    lds_barrier();
    read_stage(0, sa[0], sb[0]);
    // pairs of stages keep the register sets compile-time; with KT odd the last pair
    // runs one stage past the end, whose loads were all out of range: its fragments
    // are zeros and its MFMAs add exact zeros
    for (int kt = 0; kt < KT; kt += 2) {
      stage_iter(std::integral_constant<int, 0>{}, kt);
      stage_iter(std::integral_constant<int, 1>{}, kt + 1);
    }
  }
  }  // k-loop
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // the trailing out-of-range loads have written their zeros
  if (split_part) {
    float4* q = part_ptr(gp.ks);
#pragma unroll
    for (int t = 0; t < QUADS; ++t) {
      const f32x16_t& a = acc[(t / 4) / FN][(t / 4) % FN];
      const int c = t % 4;
      q[t * 64 + lane] = make_float4(a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]);
    }
    return;
  }

  if constexpr (kDeferScale) {
    if (defer_scale) {
      gp.psc = scale_of_partials(p, pv);
      publish_scale(p, bz, tile, gp.second, gp.psc);
    }
  }

  // every wave is done with the operand ring: reuse it for the epilogue slabs
  static_assert(NW * 32 * (Cfg::kWN + 4) * 4 <= Cfg::kLdsBytes, "epilogue slabs exceed the LDS ring");
  lds_barrier();
  float* slab = reinterpret_cast<float*>(smem16) + wave * 32 * (Cfg::kWN + 4);
  epilogue_lds<TOut, LOWER, FM, FN, NT, PL, kEarlyC>(p, acc, gp, m0 + wm * Cfg::kWM, n0 + wn * Cfg::kWN, lane, slab,
                                                     c_early);
}

// ---------------------------------------------------------------------------------
// Host side: tile configurations and the launch of one configuration.

// Output-tile configurations: (BM, BN, waves along M, waves along N, LDS ring depth,
// k values per stage of the 16-bit kernel).
//   big:   256 x 256, 8 waves of 128 x 64 (two per SIMD, ping-pong schedule), a ring
//          of 4 stages of 32 k values (128 KB of LDS)
//   mid:   128 x 128, 4 waves of 64 x 64, 4 stages of 64 (128 KB)
//   small:  64 x 64,  4 waves of 32 x 32, 4 stages of 64 (64 KB), for problems with
//          few tiles
//   tri96:  96 x 96,  3 waves of 32 x 96, 3 stages of 64 (72 KB), lower-triangle
//          products of n of about 2048 (see pick_tile)
// Measured on MI355X (alone, fp16 operands): the 8-wave big tile beats 4 waves of
// 128 x 128 (one per SIMD) by 8-10% on 4096^3 products and by 30% on the n = 768
// products of a 128-matrix batch; with 8 waves, 3, 4 and 5 stages of 32 and 2
// stages of 64 run within 3% of each other, and 8 or 16 stages of the small tiles
// are slower than 4.
constexpr int kBigWM = 2, kBigWN = 4, kBkBig = 32, kStagesBig = 4;
constexpr int kBkMid = 64, kStagesMid = 4;
constexpr int kBkSmall = 64, kStagesSmall = 4, kStagesTri96 = 3;
enum class TileCfg { kBig = 0, kMid = 1, kSmall = 2, kTri96 = 3 };

inline long long gemm_tiles(int M, int N, int bm, int bn, bool lower) {
  const long long tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
  return lower ? tm * (tm + 1) / 2 : tm * tn;
}

// The kernels address each operand matrix (both of its planes) through a 32-bit
// buffer offset.
inline bool operand_extents_ok(const GemmParams& p, int a_bytes, int b_bytes, bool nn) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0) return true;
  const size_t lim = size_t(1) << 31;
  const int apl = std::max(p.a_planes, p.a2_planes);
  // an indexed operand spans its whole source matrix
  const int a_rows = (p.rows && !nn) ? std::max(p.src_rows, 1) : p.M;
  const int b_rows = p.rows ? std::max(p.src_rows, 1) : (nn ? p.K : p.N);
  const size_t a = ((size_t)(a_rows - 1) * p.lda + p.K + (size_t)(apl - 1) * p.plane) * a_bytes;
  const size_t b = nn ? ((size_t)(b_rows - 1) * p.ldb + p.N) * b_bytes
                      : ((size_t)(b_rows - 1) * p.ldb + p.K + (size_t)(p.b_planes - 1) * p.plane) * b_bytes;
  return a < lim && b < lim;
}

// Plane counts are 1 or 2; two planes need the 16-bit kernel, a symmetric product,
// 16-bit outputs, no K split on their operands, and a plane offset.
inline bool planes_ok(const GemmParams& p, bool k16, bool lower, bool nn, int out_bytes) {
  const int pl[7] = {p.a_planes, p.a2_planes, p.b_planes, p.c_planes, p.c2_planes, p.d_planes, p.dp_planes};
  bool any = false;
  for (int v : pl) {
    if (v != 1 && v != 2) return false;
    any = any || v == 2;
  }
  if (!any) return true;
  if (!k16 || !lower || nn || out_bytes != 2 || p.plane <= 0) return false;
  if (p.ksplit > 1 && (p.a_planes != 1 || p.b_planes != 1)) return false;
  return true;
}

// Plane pairs an operand pair runs (hi.hi, hi.lo, lo.hi).
inline int plane_pairs(int a_pl, int b_pl) { return (a_pl == 2 && b_pl == 2) ? 3 : a_pl * b_pl; }

// Pick the largest tile that still gives every CU at least one workgroup.  One
// exception, for long K: when 64 x 64 tiles would need several rounds of workgroups
// while 128 x 128 tiles fit in one, the larger tile wins (each of its k-stages costs
// about twice a small tile's for four times the flops; measured on MI355X, the
// n = 2048, K = 28672 Gram product takes 181 us on 128 x 128 tiles, one round of 136
// workgroups, against 248 us on 64 x 64 tiles, three rounds of 528).
inline TileCfg pick_tile(int M, int N, int K, int batch, bool lower) {
  constexpr long long kCUs = 256;
  constexpr int kLongK = 64 * 64;       // 64 stages of 64 k values
  const long long big = (long long)batch * gemm_tiles(M, N, 256, 256, lower);
  const long long mid = (long long)batch * gemm_tiles(M, N, 128, 128, lower);
  const long long small = (long long)batch * gemm_tiles(M, N, 64, 64, lower);
  if (big >= kCUs) return TileCfg::kBig;
  // Lower-triangle products of n of about 2048: 64 x 64 tiles (528 of them at n =
  // 2048) fill two workgroups per CU with a tail of 16, and every CU brings 16 KB per
  // stage per workgroup through its load path for 32 flop/B.  96 x 96 tiles (253 at
  // n = 2048, three waves of 32 x 96) fill one round at 48 flop/B.  Measured on MI355X:
  // the n = 2048, K = 2048 product 20.96 against 24.65 us, the Gram NS of a 2048 x 28672
  // submatrix 1.129-1.133 against 1.194-1.196 ms and the 8192 x 28672 Dion3 step at
  // f = 1/4 1.466 against 1.531 ms, bitwise the same result (every element's k order
  // does not depend on the tile).
  const long long tri96 = (long long)batch * gemm_tiles(M, N, 96, 96, lower);
  if (lower && M >= 1792 && small > 2 * kCUs && tri96 <= 2 * kCUs) return TileCfg::kTri96;
  if (mid >= kCUs) return TileCfg::kMid;
  if (K >= kLongK && small > kCUs) return TileCfg::kMid;
  return TileCfg::kSmall;
}

// hi/lo plane pairs anywhere in the product
inline bool any_planes(const GemmParams& p) {
  bool planes = false;
  for (int v : {p.a_planes, p.a2_planes, p.b_planes, p.c_planes, p.c2_planes, p.d_planes, p.dp_planes})
    planes = planes || v != 1;
  return planes;
}

constexpr double kNonTemporalOutBytes = 128.0 * (1 << 20);

template <class TIn, class TB, class TOut, int BM, int BN, int WM_, int WN_, int NS, int BKV, bool LOWER, bool NN>
hipError_t launch_one(GemmParams p, int batch, hipStream_t stream, double* flops) {
  // 16-bit operands: direct-to-LDS kernel; fp32 operands: register-staged kernel
  constexpr bool k16 = TIn::kBytes == 2 && TB::kBytes == 2;
  constexpr int threads = 64 * WM_ * WN_;
  using T32 = Tile32<BM, BN, WM_, WN_, NS, BKV>;
  constexpr int lds = k16 ? T32::kLdsBytes : Tile<BM, BN, WM_, WN_>::kLdsBytes;
  constexpr int BK = k16 ? T32::kBK : 8 * TIn::kPerChunk;    // k per stage
  // An output too large to stay in the caches is written with non-temporal stores
  // (measured on MI355X: 2-4% faster on the 128 x 768x6144 batch's products; the
  // 8 MB outputs of a 1024 x 4096 call, read again by the next launch, are faster
  // with ordinary stores).  Only the 256 x 256 tile is chosen for outputs that large.
  const int products = p.pair ? 2 : 1;
  const bool nt = (double)p.M * p.N * batch * products * TOut::kBytes >= kNonTemporalOutBytes;
  void (*base)(GemmParams);
  if constexpr (k16)
    base = gemm16_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, NS, BKV, LOWER, NN, false>;
  else
    base = gemm_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, LOWER, NN>;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(base),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  void (*kern)(GemmParams) = base;
  if constexpr (k16 && BM == 256) {
    void (*with_nt)(GemmParams) = gemm16_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, NS, BKV, LOWER, NN, true>;
    static hipError_t attr_nt = hipFuncSetAttribute(reinterpret_cast<const void*>(with_nt),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr_nt != hipSuccess) return attr_nt;
    if (nt) kern = with_nt;
  }
  // hi/lo planes: a separate instantiation (bf16 symmetric products only), so the
  // single-plane kernels carry none of its address arithmetic
  const bool planes = any_planes(p);
  // indexed X rows: separate instantiations too -- the Gram product of bf16 rows
  // (symmetric, planes handled when the output is bf16) and the rectangular product
  // with bf16 B rows, whose row table takes LDS after the ring
  int dyn_lds = lds;
  if (p.rows) {
    if (p.rows_valid < 0 || p.src_rows < 1) return hipErrorInvalidValue;
    if constexpr (k16 && LOWER && !NN && TIn::kId == GNS_BF16 && TB::kId == GNS_BF16) {
      constexpr bool PLX = TOut::kId == GNS_BF16;
      if (planes && !PLX) return hipErrorInvalidValue;
      if (p.rows_valid > p.M || p.B != p.A) return hipErrorInvalidValue;
      void (*with_idx)(GemmParams) = gemm16_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, NS, BKV, LOWER, NN, false, PLX, true>;
      static hipError_t attr_idx = hipFuncSetAttribute(reinterpret_cast<const void*>(with_idx),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (attr_idx != hipSuccess) return attr_idx;
      kern = with_idx;
    } else if constexpr (k16 && NN && !LOWER && TB::kId == GNS_BF16) {
      if (planes || p.rows_valid > p.K || p.K > kMaxIndexedRows) return hipErrorInvalidValue;
      constexpr int kMaxLds = 160 * 1024;
      dyn_lds = lds + (p.K * 4 + 1023) / 1024 * 1024;
      if (dyn_lds > kMaxLds) return hipErrorInvalidValue;
      void (*with_idx)(GemmParams) = gemm16_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, NS, BKV, LOWER, NN, false, false, true>;
      static hipError_t attr_idx = hipFuncSetAttribute(reinterpret_cast<const void*>(with_idx),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
      if (attr_idx != hipSuccess) return attr_idx;
      kern = with_idx;
    } else {
      return hipErrorInvalidValue;
    }
  } else if (planes) {
    if constexpr (k16 && LOWER && !NN && TOut::kId == GNS_BF16) {
      void (*with_pl)(GemmParams) = gemm16_kernel<TIn, TB, TOut, BM, BN, WM_, WN_, NS, BKV, LOWER, NN, false, true>;
      static hipError_t attr_pl = hipFuncSetAttribute(reinterpret_cast<const void*>(with_pl),
                                                      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (attr_pl != hipSuccess) return attr_pl;
      kern = with_pl;
    } else {
      return hipErrorInvalidValue;
    }
  }
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const long long tiles = gemm_tiles(p.M, p.N, BM, BN, LOWER);
  if (!operand_extents_ok(p, TIn::kBytes, TB::kBytes, NN)) return hipErrorInvalidValue;
  if (p.pair && (NN || !LOWER || !p.A2 || !p.Dp || (p.C && !p.C2))) return hipErrorInvalidValue;
  if (p.partials && (NN || !LOWER || p.n_partials < 1 || p.n_partials > kMaxPartials)) return hipErrorInvalidValue;
  if (p.ksplit > 1 && (!k16 || !LOWER || NN || p.pair || !p.part || p.kchunk % BK)) return hipErrorInvalidValue;
  if (!planes_ok(p, k16, LOWER, NN, TOut::kBytes)) return hipErrorInvalidValue;
  const int splits = (p.ksplit > 1 && !p.reduce) ? p.ksplit : 1;
  if (flops && !p.reduce) {
    // issued: K padded to whole stages (split ranges are whole stages but the last),
    // once per plane pair
    const long long kpad = ((long long)(p.K + BK - 1) / BK) * BK;
    const int pairs = plane_pairs(p.a_planes, p.b_planes) + (p.pair ? plane_pairs(p.a2_planes, p.b_planes) : 0);
    *flops += 2.0 * (double)tiles * BM * BN * (double)kpad * batch * pairs;
  }
  if (tiles == 0 || batch == 0) return hipSuccess;
  p.batch = batch;
  p.tiles = (int)tiles;
  clear_stale_error();
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * batch * products * splits)), dim3(threads), dyn_lds, stream, p);
  return hipGetLastError();
}

template <class TIn, class TB, class TOut, bool LOWER, bool NN>
hipError_t launch_cfg(GemmParams p, int batch, hipStream_t stream, double* flops) {
  const TileCfg cfg = pick_tile(p.M, p.N, p.K, p.pair ? 2 * batch : batch, LOWER);
  switch (cfg) {
    case TileCfg::kBig:
      return launch_one<TIn, TB, TOut, 256, 256, kBigWM, kBigWN, kStagesBig, kBkBig, LOWER, NN>(
          p, batch, stream, flops);
    case TileCfg::kMid:
      // A B operand converted on load (bf16 -> fp16) is converted by every wave that
      // reads it: 4 waves side by side along N (1 x 4, 128 x 32 each) convert each
      // fragment once, where 2 x 2 waves convert it twice.  Measured on MI355X on the
      // 1024 x 4096 restart product: 19.0 against 20.4 us; with an fp16 B operand the
      // 2 x 2 layout is faster (17.3 against 18.3 us).
      if constexpr (NN && TIn::kId != TB::kId)
        return launch_one<TIn, TB, TOut, 128, 128, 1, 4, kStagesMid, kBkMid, LOWER, NN>(p, batch, stream,
                                                                                             flops);
      else
        return launch_one<TIn, TB, TOut, 128, 128, 2, 2, kStagesMid, kBkMid, LOWER, NN>(p, batch, stream,
                                                                                             flops);
    case TileCfg::kSmall:
      return launch_one<TIn, TB, TOut, 64, 64, 2, 2, kStagesSmall, kBkSmall, LOWER, NN>(p, batch, stream, flops);
    case TileCfg::kTri96:
      // 3 stages (72 KB): two workgroups share a CU when a paired launch doubles the grid
      if constexpr (LOWER && TIn::kBytes == 2)
        return launch_one<TIn, TB, TOut, 96, 96, 3, 1, kStagesTri96, kBkSmall, LOWER, NN>(p, batch, stream, flops);
      else
        return launch_one<TIn, TB, TOut, 64, 64, 2, 2, kStagesSmall, kBkSmall, LOWER, NN>(p, batch, stream, flops);
  }
  return hipErrorInvalidValue;
}

// K split of the symmetric product: a matrix with K >= 16384 whose output has 32 to
// 127 tiles of 256 x 256 is cut into S ranges of at least 2048 values, S as large as
// the CUs allow for one matrix (at most 8).  The n = 2048, K = 28672 Gram product of
// the Dion3 workload (36 tiles) runs on 7 ranges.  A matrix with fewer than 32 such
// tiles (n <= 1792) splits on tiles of 128 x 128 instead, when it has at least 32 of
// those: the n = 1024, K = 28672 Gram product then runs on 36 tiles x 7 ranges
// instead of 136 unsplit 64 x 64 tiles that leave half the CUs idle.  With fewer
// tiles each workgroup of the sum would read too many partial tiles.  The plan
// depends on n and K only, never on the batch size, so a matrix gets the same
// summation order, and the same bits, alone and in any batch.
constexpr int kSplitMinK = 16384, kSplitMinChunk = 2048, kSplitMinTiles = 32;
struct SymmSplit {
  int S = 1;         // number of K ranges (1: no split)
  int kchunk = 0;    // K values per range, a whole number of stages
  int tile = 256;    // output tile edge
};
inline SymmSplit symm_split_plan(int n, int K) {
  SymmSplit r;
  if (K < kSplitMinK) return r;
  long long tiles = gemm_tiles(n, n, 256, 256, true);
  int bk = kBkBig;
  if (tiles < kSplitMinTiles) {
    tiles = gemm_tiles(n, n, 128, 128, true);
    if (tiles < kSplitMinTiles) return r;
    r.tile = 128;
    bk = kBkMid;
  }
  const long long S = std::min<long long>(std::min<long long>(256 / tiles, 8), K / kSplitMinChunk);
  if (S < 2) return SymmSplit{};
  r.kchunk = (int)(((K + S - 1) / S + bk - 1) / bk * bk);
  r.S = (K + r.kchunk - 1) / r.kchunk;
  return r;
}

// Three launches: the partial products (one workgroup per tile and K range), the sum
// of each tile's ranges into its first range (element-parallel, fixed order), and the
// epilogue over the summed tiles.
template <class TIn, class TOut, int BM, int WM_, int WN_, int NS, int BKV>
hipError_t launch_symm_split_cfg(GemmParams p, int batch, float* part, hipStream_t stream, double* flops) {
  p.part = part;
  p.reduce = 0;
  hipError_t e = launch_one<TIn, TIn, TOut, BM, BM, WM_, WN_, NS, BKV, true, false>(p, batch, stream, flops);
  if (e != hipSuccess) return e;
  const long long tiles = gemm_tiles(p.M, p.N, BM, BM, true) * batch;
  e = launch_sum_ranges(part, tiles, p.ksplit, BM * BM, stream);
  if (e != hipSuccess) return e;
  p.reduce = 2;
  p.rows = nullptr;      // the epilogue launch reads no operand
  return launch_one<TIn, TIn, TOut, BM, BM, WM_, WN_, NS, BKV, true, false>(p, batch, stream, flops);
}

template <class TIn, class TOut>
hipError_t launch_symm_split(GemmParams p, int batch, float* part, int tile, hipStream_t stream, double* flops) {
  if (tile == 128)
    return launch_symm_split_cfg<TIn, TOut, 128, 2, 2, kStagesMid, kBkMid>(p, batch, part, stream, flops);
  return launch_symm_split_cfg<TIn, TOut, 256, kBigWM, kBigWN, kStagesBig, kBkBig>(p, batch, part,
                                                                                                 stream, flops);
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

}  // namespace gns
