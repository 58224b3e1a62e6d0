// Launcher of the symmetric-output (lower-triangle tile) MFMA GEMM; see gemm_kernel.h.
#include <algorithm>

#include "gemm_kernel.h"

namespace gns {

// Split-K plan of a symmetric product.  With fewer output tiles than CUs, K is cut
// into up to 8 ranges of at least 32 ring stages each, so that tiles x ranges covers
// the 256 CUs; the largest tile configuration that gets there wins (larger tiles
// need fewer operand bytes per flop).  Each range costs a write-through of its fp32
// partial and a read-back by the last workgroup (memory round trips of a few us), so
// short ranges lose: measured on MI355X, 8-stage ranges made the 1024 x 4096 Gram NS
// call 19% slower than no split, 32-stage ranges 4% faster.  The plan depends on the
// total tile count, hence on the batch size.
SymmPlan plan_symm(int n, int K, int batch, bool may_split) {
  constexpr long long kCUs = 256;
#ifndef GNS_SPLIT_MIN_STAGES
#define GNS_SPLIT_MIN_STAGES 32
#endif
  constexpr int kMaxSplits = 8, kMinStages = GNS_SPLIT_MIN_STAGES;
  SymmPlan pl;
#ifdef GNS_FORCE_TILE
  const TileCfg base = static_cast<TileCfg>(GNS_FORCE_TILE);
#else
  const TileCfg base = pick_tile(n, n, batch, true);
#endif
  auto tiles_of = [&](TileCfg c) { return gemm_tiles(n, n, tile_edge(c), tile_edge(c), true); };
  pl.cfg = static_cast<int>(base);
  pl.tiles = tiles_of(base);
  if (!may_split || n <= 0 || K <= 0 || batch <= 0 || (long long)batch * pl.tiles >= kCUs) return pl;
  auto splits_for = [&](TileCfg c) {
    const long long T = (long long)batch * tiles_of(c);
    const long long KT = (K + stage_k(c) - 1) / stage_k(c);
    long long s = (kCUs + T - 1) / T;
    s = std::min<long long>(s, kMaxSplits);
    s = std::min<long long>(s, KT / kMinStages);
    return (int)std::max<long long>(s, 1);
  };
  TileCfg chosen = base;
  int s = splits_for(base);
#ifndef GNS_FORCE_TILE
  for (TileCfg c : {TileCfg::kBig, TileCfg::kMid, TileCfg::kSmall}) {
    const int sc = splits_for(c);
    if (sc >= 2 && (long long)batch * tiles_of(c) * sc >= kCUs) {
      chosen = c;
      s = sc;
      break;
    }
  }
#endif
  if (s < 2) return pl;
  const int KT = (K + stage_k(chosen) - 1) / stage_k(chosen);
  const int per = (KT + s - 1) / s;
  s = (KT + per - 1) / per;                    // no empty K range
  if (s < 2) return pl;
  const long long e = tile_edge(chosen);
  pl.cfg = static_cast<int>(chosen);
  pl.splits = s;
  pl.kt_per_split = per;
  pl.tiles = tiles_of(chosen);
  pl.partial_floats = (size_t)batch * pl.tiles * s * e * e;
  pl.counters = (int)(batch * pl.tiles);
  return pl;
}

hipError_t launch_symm(gns_dtype in, gns_dtype out, const GemmParams& p, int batch, hipStream_t s,
                       double* flops) {
  switch (in) {
    case GNS_BF16: return dispatch_out<TBF16, TBF16, true, false>(out, p, batch, s, flops);
    case GNS_F16: return dispatch_out<TF16, TF16, true, false>(out, p, batch, s, flops);
    case GNS_F32: return dispatch_out<TF32, TF32, true, false>(out, p, batch, s, flops);
  }
  return hipErrorInvalidValue;
}

}  // namespace gns
