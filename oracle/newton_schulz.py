"""Standard and Gram Newton-Schulz orthogonalisation, float64, written from the pages.

Sources:
  * "Muon: Orthogonalized Momentum and Why It Trains LLMs 2x Cheaper", section
    "Doing an SVD without an SVD": the odd quintic phi(x) = a x + b x^3 + c x^5 acts
    on each singular value; coefficients (3.4445, -4.7750, 2.0315); five steps;
    the input is divided by (Frobenius norm + 1e-7); a matrix with more rows than
    columns is transposed so the iteration runs on the short side.
  * "Dion3：全栈正交更新" (paper.rainbus.top), section 前置知识 (Newton-Schulz
    iteration): one step applies the odd quintic to X, which is the matrix
    a X + b (X X^T) X + c (X X^T)^2 X.
  * Same page, section 核心方法 (theorem 2): writing each odd step as
    p_t(x) = x h_t(x^2) with h_t(r) = a_t + b_t r + c_t r^2, the composition
    p_T o ... o p_1 (x) equals q_T x, where r_0 = x^2, q_0 = 1, z_t = h_t(r_{t-1}),
    r_t = r_{t-1} z_t^2, q_t = q_{t-1} z_t.  Lifted to matrices with R_0 = X X^T this
    is Gram Newton-Schulz.
  * Same page, section 方法步骤详情 (Algorithm 3): R_0 = X X^T, Q_0 = I; each step
    Z_t = b_t R + c_t R^2, Q_t = Q Z_t + a_t Q, R updated from Z_t; a restart before
    step 3 sets X <- Q_2 X, recomputes R = X X^T and resets Q = I; the output is Q_T X.
    The page's R-update formula is garbled; the reading used here follows theorem 2:
    R_t = (Z_t + a_t I) R_{t-1} (Z_t + a_t I).

Parity status:
  * newton_schulz: pinned (SVD closed form U phi^T(Sigma) V^T; diagonal and
    orthonormal-row closed forms; permutation equivariance; transposition).
  * gram_newton_schulz: pinned against newton_schulz (equal in exact arithmetic,
    with or without restart) and the negative-eigenvalue divergence the pages report.
"""
from __future__ import annotations

import numpy as np

JORDAN_ABC = (3.4445, -4.7750, 2.0315)
EPS = 1e-7


def _coeffs(abc, steps):
    """Per-step (a_t, b_t, c_t): one triple used for every step, or a table of them."""
    arr = np.asarray(abc, dtype=np.float64)
    if arr.ndim == 1:
        return [tuple(arr)] * steps
    assert arr.shape == (steps, 3)
    return [tuple(row) for row in arr]


def quintic(x, abc=JORDAN_ABC):
    """phi(x) = a x + b x^3 + c x^5 on scalars or arrays."""
    a, b, c = abc
    x = np.asarray(x, dtype=np.float64)
    return a * x + b * x ** 3 + c * x ** 5


def quintic_composed(x, steps=5, abc=JORDAN_ABC):
    """phi_T o ... o phi_1 applied to scalars (the action on singular values)."""
    y = np.asarray(x, dtype=np.float64)
    for t in _coeffs(abc, steps):
        y = quintic(y, t)
    return y


def normalize(x, eps=EPS):
    """X / (||X||_F + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.sum(x * x)) + eps)


def _short_side(x):
    """(Y, flipped): Y = X when X has no more rows than columns, else Y = X^T, so
    that the iteration works with the smaller Gram matrix Y Y^T."""
    return (x.T, True) if x.shape[0] > x.shape[1] else (x, False)


def _odd_step_factor(gram, a, b, c):
    """h(G) = a I + b G + c G^2 for the Gram matrix G = Y Y^T.

    An odd quintic p(y) = a y + b y^3 + c y^5 factors as p(y) = h(y^2) y with
    h(r) = a + b r + c r^2 (the factorisation behind theorem 2).  For a matrix Y,
    p acts on every singular value, which is the left multiplication
    p(Y) = h(Y Y^T) Y.  The factor is built here as a I + G (b I + c G)."""
    eye = np.eye(gram.shape[0])
    return a * eye + gram @ (b * eye + c * gram)


def newton_schulz(x, steps=5, abc=JORDAN_ABC, eps=EPS):
    """Standard quintic Newton-Schulz on one matrix (the oracle of record).

    Each step replaces Y by p_t(Y) = h_t(Y Y^T) Y, i.e. applies the odd quintic
    p_t to every singular value of Y, starting from the Frobenius-normalised input
    on its short side; T = `steps` steps with the per-step (a_t, b_t, c_t)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 3:
        return np.stack([newton_schulz(xi, steps, abc, eps) for xi in x])
    y, flipped = _short_side(normalize(x, eps))
    for a, b, c in _coeffs(abc, steps):
        y = _odd_step_factor(y @ y.T, a, b, c) @ y
    return y.T if flipped else y


def gram_newton_schulz_schedule(steps=5, restart_after=(2,)):
    """Which steps are preceded by a restart: a restart 'after step s' happens
    before step s+1 (the pages' 'restart at t = 3' is restart_after=(2,))."""
    return {s + 1 for s in restart_after if 1 <= s < steps}


def gram_newton_schulz(x, steps=5, abc=JORDAN_ABC, eps=EPS, restart_after=(2,),
                       perturb_r0=None, trace=None):
    """Gram Newton-Schulz (Algorithm 3 with the theorem-2 R update), float64.

    perturb_r0: optional function R0 -> R0' applied to the first Gram matrix (used to
      inject a spurious negative eigenvalue).
    trace: optional list; receives (t, min eigenvalue of R before step t, max |Q|)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 3:
        return np.stack([gram_newton_schulz(xi, steps, abc, eps, restart_after,
                                            perturb_r0, trace) for xi in x])
    xn, transposed = _short_side(normalize(x, eps))
    n = xn.shape[0]
    eye = np.eye(n)
    restarts = gram_newton_schulz_schedule(steps, restart_after)
    R = xn @ xn.T
    if perturb_r0 is not None:
        R = perturb_r0(R)
    Q = eye.copy()
    for t, (a, b, c) in enumerate(_coeffs(abc, steps), start=1):
        if t in restarts:
            xn = Q @ xn
            R = xn @ xn.T
            Q = eye.copy()
        if trace is not None:
            trace.append((t, float(np.linalg.eigvalsh(R).min()), float(np.abs(Q).max())))
        Z = b * R + c * (R @ R)
        Q = Q @ Z + a * Q
        Zf = Z + a * eye
        R = Zf @ R @ Zf
    out = Q @ xn
    return out.T if transposed else out
