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

}  // namespace gns
