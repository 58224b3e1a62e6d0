// Launchers of the Muon step's element-wise passes (muon.hip).  Matrices are bf16,
// row-major with 8 | m and 8 | row stride; every launch covers the whole batch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gns {

// M <- bf16(fl32(mu M) + G) in place; with U non-null also U = bf16(G + fl32(mu M'))
// ([batch][n][ldu], matrix stride su).  M and G: row stride ld, matrix stride stride.
// Also s_out[b] = 1 / (||X_b||_F + eps) of the matrix the orthogonalisation reads (U,
// or M' without U), from fp64 row sums of squares kept in rowsq ([batch][n] doubles).
hipError_t launch_muon_momentum(uint16_t* M, const uint16_t* G, int batch, int n, int m, long long ld,
                                long long stride, float mu, uint16_t* U, long long ldu, long long su, double* rowsq,
                                float eps, float* s_out, hipStream_t s);

// W <- bf16(fl32(d W) - fl32(fl32(lr scale) O)), d = fl32(1 - fl32(lr wd)), in place;
// O: bf16 [batch][n][ldo], matrix stride so.
hipError_t launch_muon_update(uint16_t* W, int batch, int n, int m, long long ld, long long stride,
                              const uint16_t* O, long long ldo, long long so, float lr, float wd, float scale,
                              hipStream_t s);

}  // namespace gns
