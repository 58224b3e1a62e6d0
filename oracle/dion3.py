"""Dion3 row-subsampled update with error feedback, written from the pages.

Sources:
  * "Dion3：全栈正交更新" (paper.rainbus.top), section 方法步骤详情, Algorithm 4:
    M <- M + G; pick the k = ceil(f n) rows of largest l1 norm (index set S);
    orthogonalise the submatrix M[S, :] with Gram NS; decay the weights
    W <- (1 - lr wd) W; update the selected weight rows W[S, :] <- W[S, :] - lr O;
    error feedback decays only the selected momentum rows, M[S, :] <- mu M[S, :].
  * Same page, section 前置知识 (error feedback): M <- mu M_hat + (M - M_hat), where
    M_hat keeps only the selected rows; unselected rows keep their value.
  * Same page, 核心方法: the learning rate is rescaled as lr = eta / sqrt(f).
  * "Dion3: Full-Stack Orthogonal Updates" (m.montaan.com): f = 1 is Muon.

Storage model (the pages leave rounding open; the reading stated here is the one the
GPU path follows): W, M, G are stored in one format, the caller's state dtype (bf16,
f16 or f32).  Every stored result is rounded once to that format (nearest, ties to
even).  The element-wise updates are carried out in fp32 op by op (numpy float32
arithmetic, each operation correctly rounded, no fused multiply-add).  Row scores are
sums in float64 of the stored (rounded) values.  The orthogonalised rows O are stored
in the state format before the weight update reads them.

Storage modes:
  storage="bf16"  bf16 bit patterns (uint16), the model above;
  storage="f16"   numpy float16 arrays, the model above;
  storage="f32"   numpy float32 arrays, the model above;
  storage="f64"   float64 arrays, no rounding anywhere (used to pin f = 1 against Muon
                  exactly).

Parity status: select_topk pinned by brute force; accumulate / error_feedback /
weight_update pinned by their bit-level definitions and invariants; dion3_step
pinned by the f = 1 == Muon identity and the error-feedback invariants;
dion3_step_rows pinned by its invariants, by the all-rows case and by equality with
dion3_step on the top-k set; dion3_step_cols pinned by column-norm selection, its
column invariants and the Newton-Schulz oracle on the gathered columns.
"""
from __future__ import annotations

import math
import numpy as np

from .bf16 import bf16_to_f64, f64_to_bf16_rne
from .newton_schulz import newton_schulz, JORDAN_ABC, EPS


def k_from_fraction(f, n: int) -> int:
    """k = ceil(f n), computed exactly (f may be a float such as 0.25 or 1/8)."""
    from fractions import Fraction
    return int(math.ceil(Fraction(f).limit_denominator(1 << 20) * n))


def _codec(storage):
    """(decode: stored values -> float64 exactly, encode: float64 -> stored values with
    one rounding to nearest, ties to even) of a state format."""
    if storage == "bf16":
        return bf16_to_f64, f64_to_bf16_rne
    def narrow(dtype):
        def enc(x):
            with np.errstate(over="ignore"):         # values past the format's range become inf
                return np.asarray(x, dtype=np.float64).astype(dtype)
        return enc
    if storage == "f16":
        return lambda a: np.asarray(a, dtype=np.float16).astype(np.float64), narrow(np.float16)
    if storage == "f32":
        return lambda a: np.asarray(a, dtype=np.float32).astype(np.float64), narrow(np.float32)
    raise ValueError(f"storage must be bf16, f16 or f32, not {storage!r}")


def accumulate(m, g, storage="bf16"):
    """M <- fl(M + G) in the state format.  The fp64 sum of two stored values rounded
    once more to the format equals the correctly rounded sum (binary64 has at least
    2p + 2 bits for p = 8, 11 and 24), which is also what rounding the fp32 sum gives."""
    dec, enc = _codec(storage)
    return enc(dec(m) + dec(g))


def row_scores(m, norm="l1", storage="bf16"):
    """Per-row score of the stored momentum: sum_j |M_ij| (l1) or sum_j M_ij^2 (l2),
    each the correctly rounded float64 value of the exact sum (math.fsum)."""
    dec, _ = _codec(storage)
    x = dec(m)
    terms = np.abs(x) if norm == "l1" else x * x      # squares of stored values are exact in fp64
    return np.array([math.fsum(row) for row in terms], dtype=np.float64)


def select_topk(scores, k: int):
    """Indices of the k largest scores, ties broken toward the lower index, returned
    in ascending index order."""
    scores = [float(s) for s in scores]
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return np.array(sorted(order[:k]), dtype=np.int64)


def gather_rows(m_bits, S):
    return np.asarray(m_bits)[np.asarray(S)]


def error_feedback(m, S, mu, storage="bf16"):
    """M[S, :] <- fl(fl32(mu) * M[S, :]) in the state format; other rows unchanged."""
    dec, enc = _codec(storage)
    out = np.array(m, copy=True)
    mu32 = np.float32(mu)
    rows = dec(out[S]).astype(np.float32)
    out[S] = enc((mu32 * rows).astype(np.float64))
    return out


def weight_update(w, S, o, lr, wd, storage="bf16"):
    """Decoupled weight decay on all rows and the orthogonalised update on rows S.

    d = fl32(1 - fl32(lr * wd));
    W[S]     <- fl( fl32( fl32(d * W[S]) - fl32(lr * O) ) )
    W[not S] <- W                   if wd == 0
                fl( fl32(d * W) )   otherwise
    (fl: one rounding to the state format.)  o: the update rows, [k, m] float values
    (as stored by the caller, e.g. in the state format)."""
    dec, enc = _codec(storage)
    out = np.array(w, copy=True)
    lr32, wd32 = np.float32(lr), np.float32(wd)
    d = np.float32(np.float32(1.0) - lr32 * wd32)
    o32 = np.asarray(o, dtype=np.float64).astype(np.float32)
    if wd32 != 0:
        allw = dec(out).astype(np.float32)
        out = enc((d * allw).astype(np.float64))
    wsel = dec(np.asarray(w)[S]).astype(np.float32)
    upd = (d * wsel) - (lr32 * o32)
    out[S] = enc(upd.astype(np.float64))
    return out


def dion3_step(w, m, g, k, lr, wd=0.0, mu=0.95, norm="l1", steps=5, abc=JORDAN_ABC,
               eps=EPS, storage="bf16", orthogonalize=None):
    """One Dion3 step.  Returns (W', M', S, O) where O is the orthogonalised
    submatrix (float64) of the selected rows.

    storage="bf16": w, m, g are uint16 bf16 bit patterns, results likewise;
    storage="f16" / "f32": numpy float16 / float32 arrays, results likewise;
    storage="f64":  w, m, g are float64 arrays and nothing is rounded.
    orthogonalize: function X -> O (default: standard Newton-Schulz, the oracle of
    record for Gram NS, which it equals in exact arithmetic)."""
    ortho = orthogonalize or (lambda x: newton_schulz(x, steps, abc, eps))
    if storage == "f64":
        m1 = np.asarray(m, np.float64) + np.asarray(g, np.float64)
        terms = np.abs(m1) if norm == "l1" else m1 * m1
        scores = np.array([math.fsum(r) for r in terms])
        S = select_topk(scores, k)
        O = ortho(m1[S])
        w1 = (1.0 - lr * wd) * np.asarray(w, np.float64)
        w1[S] = w1[S] - lr * O
        m2 = m1.copy()
        m2[S] = mu * m1[S]
        return w1, m2, S, O
    m1 = accumulate(m, g, storage)
    scores = row_scores(m1, norm, storage)
    S = select_topk(scores, k)
    w2, m2, O = _update_rows(w, m1, S, lr, wd, mu, ortho, storage)
    return w2, m2, S, O


def _update_rows(w, m1, S, lr, wd, mu, ortho, storage="bf16"):
    """The part of a step after the row set S is known: orthogonalise M[S, :],
    store O in the state format, decay + row update of W, error feedback on M[S, :]."""
    dec, enc = _codec(storage)
    X = dec(gather_rows(m1, S))
    O = ortho(X)
    O_stored = dec(enc(O))
    w2 = weight_update(w, S, O_stored, lr, wd, storage)
    m2 = error_feedback(m1, S, mu, storage)
    return w2, m2, O


def dion3_step_rows(w, m, g, S, lr, wd=0.0, mu=0.95, steps=5, abc=JORDAN_ABC, eps=EPS, orthogonalize=None,
                    storage="bf16"):
    """One Dion3 step on a row set S chosen by the caller instead of the top-k rows.

    The pages report that rows picked at random train about as well as the rows of
    largest l1 norm, and that a set S chosen without looking at M lets a data-parallel
    step exchange only M[S, :] ("Dion3：全栈正交更新", paper.rainbus.top, 局限与改进 and
    the future-work paragraph after it; the random draw itself is the caller's).
    Everything else is Algorithm 4 as in dion3_step: M <- M + G, orthogonalise
    M[S, :], decay + row update of W, error feedback on M[S, :].  w, m, g: stored
    values as in dion3_step (storage bf16, f16 or f32).  S: distinct row indices,
    ascending.  Returns (W', M', O).

    Parity: pinned by its invariants, by S = all rows giving the orthogonalised
    accumulated momentum, and by equality with dion3_step when S is its top-k set."""
    S = np.asarray(S, dtype=np.int64)
    n = np.asarray(m).shape[0]
    if S.ndim != 1 or S.size == 0 or np.any(np.diff(S) <= 0) or S[0] < 0 or S[-1] >= n:
        raise ValueError("S must hold distinct row indices in [0, N), ascending")
    ortho = orthogonalize or (lambda x: newton_schulz(x, steps, abc, eps))
    m1 = accumulate(m, g, storage)
    return _update_rows(w, m1, S, lr, wd, mu, ortho, storage)


def dion3_step_cols(w, m, g, k, lr, wd=0.0, mu=0.95, norm="l1", steps=5, abc=JORDAN_ABC, eps=EPS,
                    orthogonalize=None, storage="bf16"):
    """One Dion3 step that subsamples columns instead of rows.

    The pages let the fraction f select rows or columns ("Dion3：全栈正交更新",
    paper.rainbus.top, 核心方法 and 方法步骤详情 (3); "Dion3: Full-Stack Orthogonal
    Updates", m.montaan.com).  Selecting the k columns of largest norm of M, orthogonalising
    M[:, S], updating W[:, S] and decaying M[:, S] is the row rule applied to the
    transposes, which is how it is written here.  w, m, g: N x m stored values as in
    dion3_step (storage bf16, f16 or f32).  Returns (W', M', S, O) with O the k x N transpose of the orthogonalised
    N x k submatrix (row j is the update of column S[j]).

    Parity: pinned by column-norm selection against brute force, by the invariants on
    the unselected and selected columns, and by O against the Newton-Schulz oracle on
    the gathered columns."""
    T = lambda a: np.ascontiguousarray(np.asarray(a).T)
    wt, mt, S, O = dion3_step(T(w), T(m), T(g), k, lr, wd, mu, norm, steps, abc, eps, storage, orthogonalize)
    return T(wt), T(mt), S, O
