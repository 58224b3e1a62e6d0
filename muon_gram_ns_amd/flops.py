"""FLOP accounting for Newton-Schulz variants (host arithmetic, no GPU).

Cost formulas stated on "Dion3: Full-Stack Orthogonal Updates" (paper.rainbus.top):
  * standard NS: 2 T (2 alpha + 1) n^3 (section 研究动机);
  * standard NS with symmetric kernels: T (3 alpha + 1) n^3, plain: (20 alpha + 10) n^3
    at T = 5, Gram NS: (4T + 3 alpha - 3) n^3 (实验结果 table, Algorithm 3 total cost);
  * each restart adds 3 (alpha - 1) n^3 (局限与改进).
Here alpha = m / n and "n^3" counts a symmetric n x n product once (lower half).

Exact algorithmic counts of the schedules libgns runs (what `achieved` TFLOP/s uses):
a symmetric n x n output with inner dimension K costs n (n + 1) K flops (lower
triangle incl. diagonal, 2K each); a rectangular n x K by K x m product 2 n K m.
"""
from __future__ import annotations


def pages_gram(T: int, alpha: float) -> float:
    return 4 * T + 3 * alpha - 3


def pages_standard_symmetric(T: int, alpha: float) -> float:
    return T * (3 * alpha + 1)


def pages_standard_plain(T: int, alpha: float) -> float:
    return 2 * T * (2 * alpha + 1)


def pages_restart_extra(alpha: float) -> float:
    return 3 * (alpha - 1)


def standard_ns_nominal(n: int, m: int, T: int = 5) -> float:
    """Dense standard NS, every product counted in full: 2 T (2 alpha + 1) n^3."""
    return 2.0 * T * (2.0 * m + n) * n * n


def sym(n: int, K: int) -> float:
    return float(n) * (n + 1) * K


def rect(n: int, K: int, m: int) -> float:
    return 2.0 * n * K * m


def gram_schedule(n: int, m: int, T: int = 5, restart_after=(2,)) -> float:
    """Algorithmic flops of libgns's Gram NS schedule for one n x m matrix."""
    restarts = {s + 1 for s in restart_after if 1 <= s < T}
    f = sym(n, m)                                     # R0 = X X^T
    q_identity = True
    for t in range(1, T + 1):
        if t in restarts:
            f += rect(n, n, m) + sym(n, m)            # X <- Q X ; R = X X^T
            q_identity = True
        f += sym(n, n)                                # Z = c R R + b R (Q = Z + aI free)
        if not q_identity:
            f += sym(n, n)                            # Q <- Q (Z + a I)
        q_identity = False
        if t < T and (t + 1) not in restarts:
            f += 2 * sym(n, n)                        # Y = R (Z + a I) ; R = (Z + a I) Y
    return f + rect(n, n, m)                          # O = Q X


def standard_schedule(n: int, m: int, T: int = 5) -> float:
    """Algorithmic flops of libgns's standard NS schedule (symmetric products halved)."""
    return T * (sym(n, m) + sym(n, n) + rect(n, n, m))
