// Launchers of the Muon step's element-wise passes (muon.hip).  Matrices share the
// state type dt (bf16, f16 or fp32), row-major with 8 | m and 8 | row stride; every
// launch covers the whole batch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gns.h"

namespace gns {

// M <- fl(fl32(mu M) + G) in place; with U non-null also U = fl(G + fl32(mu M'))
// ([batch][n][ldu], matrix stride su).  M and G: row stride ld, matrix stride stride.
// The fp64 sums of squares of the rows of the matrix the orthogonalisation reads (U,
// or M' without U) go to rowsq ([batch][n] doubles) and, with rowsq32 non-null, rounded
// to fp32 to rowsq32 ([batch][n]), the partial sums a Gram product forms its Frobenius
// scale from.  With s_out non-null a second launch also forms s_out[b] =
// 1 / (||X_b||_F + eps) from the fp64 sums.
hipError_t launch_muon_momentum(void* M, const void* G, gns_dtype dt, int batch, int n, int m, long long ld,
                                long long stride, float mu, void* U, long long ldu, long long su, double* rowsq,
                                float* rowsq32, float eps, float* s_out, hipStream_t s);

// W <- fl(fl32(d W) - fl32(fl32(lr scale) O)), d = fl32(1 - fl32(lr wd)), in place;
// O: [batch][n][ldo] in the state type, matrix stride so.
hipError_t launch_muon_update(void* W, gns_dtype dt, int batch, int n, int m, long long ld, long long stride,
                              const void* O, long long ldo, long long so, float lr, float wd, float scale,
                              hipStream_t s);

}  // namespace gns
