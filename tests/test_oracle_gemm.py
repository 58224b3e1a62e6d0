"""Pins for the oracle's GEMM definitions: explicit triple loops on tiny inputs."""
import numpy as np

from oracle import symm_gemm_ref, rect_gemm_ref


def test_symm_gemm_ref_loops():
    rng = np.random.default_rng(0)
    n, k = 5, 3
    A, B, C = rng.standard_normal((n, k)), rng.standard_normal((n, k)), rng.standard_normal((n, n))
    got = symm_gemm_ref(A, B, C, alpha=0.7, beta=-1.3, gamma=2.0)
    for i in range(n):
        for j in range(n):
            r, c = max(i, j), min(i, j)          # the lower-triangle element is the one formed
            v = 0.7 * sum(A[r, t] * B[c, t] for t in range(k)) - 1.3 * C[r, c] + (2.0 if r == c else 0.0)
            assert abs(got[i, j] - v) < 1e-12
    assert np.array_equal(got, got.T)


def test_rect_gemm_ref_loops():
    rng = np.random.default_rng(1)
    n, k, m = 4, 3, 6
    A, B, C = rng.standard_normal((n, k)), rng.standard_normal((k, m)), rng.standard_normal((n, m))
    got = rect_gemm_ref(A, B, C, alpha=1.5, beta=0.25)
    for i in range(n):
        for j in range(m):
            v = 1.5 * sum(A[i, t] * B[t, j] for t in range(k)) + 0.25 * C[i, j]
            assert abs(got[i, j] - v) < 1e-12
