// Launcher of the symmetric-output (lower-triangle tile) MFMA GEMM; see gemm_kernel.h.
#include "gemm_kernel.h"

namespace gns {

hipError_t launch_symm(gns_dtype in, gns_dtype out, const GemmParams& p, int batch, hipStream_t s,
                       double* flops) {
  switch (in) {
    case GNS_BF16: return dispatch_out<TBF16, TBF16, true, false>(out, p, batch, s, flops);
    case GNS_F16: return dispatch_out<TF16, TF16, true, false>(out, p, batch, s, flops);
    case GNS_F32: return dispatch_out<TF32, TF32, true, false>(out, p, batch, s, flops);
  }
  return hipErrorInvalidValue;
}

size_t symm_split_bytes(int batch, int n, int K, gns_dtype in) {
  if (in == GNS_F32) return 0;
  const SymmSplit sp = symm_split_plan(n, K);
  if (sp.S < 2 || batch < 1) return 0;
  return (size_t)batch * gemm_tiles(n, n, sp.tile, sp.tile, true) * sp.S * sp.tile * sp.tile * sizeof(float);
}

hipError_t launch_symm_ws(gns_dtype in, gns_dtype out, const GemmParams& p, int batch, float* part, size_t part_bytes,
                          hipStream_t s, double* flops) {
  const SymmSplit sp = (in == GNS_F32 || p.pair) ? SymmSplit{} : symm_split_plan(p.M, p.K);
  if (sp.S < 2 || !part || part_bytes < symm_split_bytes(batch, p.M, p.K, in))
    return launch_symm(in, out, p, batch, s, flops);
  GemmParams q = p;
  q.ksplit = sp.S;
  q.kchunk = sp.kchunk;
  if (in == GNS_BF16) {
    switch (out) {
      case GNS_BF16: return launch_symm_split<TBF16, TBF16>(q, batch, part, sp.tile, s, flops);
      case GNS_F16: return launch_symm_split<TBF16, TF16>(q, batch, part, sp.tile, s, flops);
      case GNS_F32: return launch_symm_split<TBF16, TF32>(q, batch, part, sp.tile, s, flops);
    }
  } else {
    switch (out) {
      case GNS_BF16: return launch_symm_split<TF16, TBF16>(q, batch, part, sp.tile, s, flops);
      case GNS_F16: return launch_symm_split<TF16, TF16>(q, batch, part, sp.tile, s, flops);
      case GNS_F32: return launch_symm_split<TF16, TF32>(q, batch, part, sp.tile, s, flops);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gns
