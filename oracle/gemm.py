"""Reference definitions of the two GEMM entry points, float64.

Symmetric-output GEMM ("Dion3: Full-Stack Orthogonal Updates", paper.rainbus.top,
前置知识 symmetric GEMM kernel; 方法步骤详情 (2)): only the lower triangle (with the
diagonal) of alpha A B^T + beta C + gamma I is formed, and it is copied to the upper
triangle, so the result is exactly symmetric even when A B^T is not.  C is read
from its lower triangle.

Rectangular GEMM: alpha A B + beta C.

Parity status: pinned by explicit triple loops on tiny inputs (tests).
"""
from __future__ import annotations

import numpy as np


def symm_gemm_ref(A, B, C=None, alpha=1.0, beta=0.0, gamma=0.0):
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    if A.ndim == 3:
        return np.stack([symm_gemm_ref(A[i], B[i], None if C is None else C[i], alpha, beta, gamma)
                         for i in range(A.shape[0])])
    full = alpha * (A @ B.T) + gamma * np.eye(A.shape[0])
    if C is not None and beta != 0.0:
        full = full + beta * np.asarray(C, np.float64)
    lower = np.tril(full)
    return lower + np.tril(lower, -1).T


def rect_gemm_ref(A, B, C=None, alpha=1.0, beta=0.0):
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    out = alpha * np.matmul(A, B)
    if C is not None and beta != 0.0:
        out = out + beta * np.asarray(C, np.float64)
    return out
