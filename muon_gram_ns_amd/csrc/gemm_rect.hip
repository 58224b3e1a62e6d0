// Launcher of the rectangular MFMA GEMM (B transposed on load); see gemm_kernel.h.
#include "gemm_kernel.h"

namespace gns {

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
