"""Seeded synthetic inputs shared by the oracle and the GPU path.

This module holds NO arithmetic of the method (no normalisation, no Newton-Schulz,
no Gram products, no row scores).  It only draws random matrices with the shapes,
value distributions and singular-value spectra of the workloads the Dion3 pages
describe, and rounds them ONCE to the stored dtype.  Both the CPU oracle and the
HIP path receive the very same bytes.

Stored dtypes:
  * "f32"  -> numpy float32 array
  * "f16"  -> numpy float16 array
  * "bf16" -> numpy uint16 array holding bfloat16 bit patterns

The rounding to bf16 uses torch's CPU conversion (round to nearest even), a library
routine; fp64 -> fp32 uses numpy's conversion (also round to nearest even).  The
construction is what defines the workload, so any fixed deterministic rounding is
acceptable here; the bytes produced are the input.

Randomness: numpy PCG64 seeded per workload (1000 + workload index).
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_rng", "to_storage", "haar",
    "kron_mixed_operator", "kron_mixed_orthonormal", "low_rank_matrix", "gns_batch", "dion3_state",
    "random_symmetric", "random_matrix", "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str          # what the workload is, with its sizes
    index: int         # position in the list of workloads (seed = 1000 + index)
    batch: int
    n: int             # rows (short side)
    m: int             # columns (long side)
    dtype: str         # stored dtype of the momentum matrices ("f32" | "bf16")
    spectrum: str      # "inv" (sigma_i = 1/i) | "invsqrt" (sigma_i = i^-1/2) | "gauss"
    noise: float       # std of additive entrywise Gaussian noise
    factors: str       # "haar" (QR of a Gaussian) | "kron" (two-level Kronecker-Haar)


# The five workloads of the Dion3/Gram-NS hot path.  The Dion3 workload's matrix is
# 8192 x 28672 (n = rows of the momentum matrix that are subsampled).
WORKLOADS = [
    Workload("gns_64x256_f32", 0, 1, 64, 256, "f32", "inv", 1e-3, "haar"),
    Workload("gns_1024x4096_bf16", 1, 1, 1024, 4096, "bf16", "inv", 1e-3, "haar"),
    Workload("gns_32x4096x4096_bf16", 2, 32, 4096, 4096, "bf16", "invsqrt", 0.0, "kron"),
    Workload("gns_128x768x6144_bf16", 3, 128, 768, 6144, "bf16", "inv", 1e-3, "kron"),
    Workload("dion3_8192x28672_bf16", 4, 1, 8192, 28672, "bf16", "gauss", 0.0, "none"),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp64 array once to the stored dtype ("f32" or "bf16" bit patterns)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(x32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact; a bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def haar(rng: np.random.Generator, m: int, n: int | None = None) -> np.ndarray:
    """m x n matrix with orthonormal columns, Haar distributed (QR of a Gaussian,
    with the signs of R's diagonal moved into Q)."""
    n = m if n is None else n
    g = rng.standard_normal((m, n))
    q, r = np.linalg.qr(g)
    d = np.sign(np.diag(r))
    d[d == 0] = 1.0
    return q * d[None, :]


def _split(m: int) -> tuple[int, int]:
    p = int(np.sqrt(m))
    while m % p:
        p -= 1
    return p, m // p


def kron_mixed_operator(rng: np.random.Generator, m: int):
    """A random m x m orthogonal operator (A1 (x) B1) P (A2 (x) B2), where A*, B* are
    Haar factors of size ~sqrt(m) and P is a random permutation, returned as a
    function y -> op @ y for y of shape (m, k).  The operator is dense and
    incoherent like a Haar matrix but costs O(m^1.5 k) to apply instead of the
    O(m^3) of forming a Haar matrix by QR, which matters for large batches."""
    p, q = _split(m)
    a1, a2 = haar(rng, p), haar(rng, p)
    b1, b2 = haar(rng, q), haar(rng, q)
    perm = rng.permutation(m)

    import torch
    ta1, ta2, tb1, tb2 = (torch.from_numpy(x) for x in (a1, a2, b1, b2))

    def apply_kron(a, b, y):  # (a (x) b) @ y, y of shape (p*q, k)
        k = y.shape[1]
        t = (a @ y.reshape(p, q * k)).reshape(p, q, k)          # along the p index
        return torch.matmul(b, t).reshape(p * q, k)               # along the q index

    def op(y):
        y = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float64))
        return apply_kron(ta1, tb1, apply_kron(ta2, tb2, y)[perm]).numpy()
    return op


def kron_mixed_orthonormal(rng: np.random.Generator, m: int, n: int) -> np.ndarray:
    """The first n columns of a kron_mixed_operator: m x n, orthonormal columns."""
    e = np.zeros((m, n))
    e[np.arange(n), np.arange(n)] = 1.0
    return kron_mixed_operator(rng, m)(e)


def _spectrum(kind: str, n: int) -> np.ndarray:
    i = np.arange(1, n + 1, dtype=np.float64)
    if kind == "inv":
        return 1.0 / i
    if kind == "invsqrt":
        return 1.0 / np.sqrt(i)
    raise ValueError(kind)


def low_rank_matrix(rng, n, m, spectrum, noise, factors) -> np.ndarray:
    """U diag(sigma) V^T (+ noise), U n x n orthogonal, V m x n orthonormal columns."""
    sig = _spectrum(spectrum, n) if isinstance(spectrum, str) else np.asarray(spectrum, np.float64)
    if factors == "haar":
        u, v = haar(rng, n), haar(rng, m, n)
        x = (u * sig[None, :]) @ v.T
    elif factors == "kron":
        u_op = kron_mixed_operator(rng, n)
        v = kron_mixed_orthonormal(rng, m, n)
        x = u_op(sig[:, None] * v.T)
    else:
        raise ValueError(factors)
    if noise:
        x = x + noise * rng.standard_normal((n, m))
    return x


def gns_batch(w: Workload | str | int, batch: int | None = None, seed: int | None = None,
              n: int | None = None, m: int | None = None) -> np.ndarray:
    """A batch of momentum matrices of a Gram-NS workload, in its stored dtype.

    batch/n/m override the workload's sizes (reduced-size parity cases keep the
    workload's construction); the default seed is 1000 + workload index.
    Returns shape [B, n, m]."""
    w = w if isinstance(w, Workload) else workload(w)
    batch = w.batch if batch is None else batch
    n = w.n if n is None else n
    m = w.m if m is None else m
    rng = make_rng(1000 + w.index if seed is None else seed)
    out = [to_storage(low_rank_matrix(rng, n, m, w.spectrum, w.noise, w.factors), w.dtype)
           for _ in range(batch)]
    return np.stack(out)


def dion3_state(n: int = 8192, m: int = 28672, seed: int | None = None, std: float = 0.02):
    """(W, G, M0) for a Dion3 step, each n x m bf16 bit patterns, entries N(0, std^2)."""
    rng = make_rng(1000 + 4 if seed is None else seed)
    outs = []
    for _ in range(3):
        x = rng.standard_normal((n, m), dtype=np.float32) * np.float32(std)
        outs.append(to_storage(x, "bf16"))
    return tuple(outs)


def random_symmetric(rng, n, dtype="f32", scale=None) -> np.ndarray:
    """A random symmetric n x n matrix (G + G^T) * scale with G Gaussian, stored.
    The default scale 1/sqrt(2n) keeps its spectrum near [-2, 2]."""
    g = rng.standard_normal((n, n))
    s = (g + g.T) * (1.0 / np.sqrt(2.0 * n) if scale is None else scale)
    return to_storage(s, dtype)


def random_matrix(rng, n, m, dtype="f32", scale=1.0) -> np.ndarray:
    """An n x m matrix of N(0, scale^2) entries, stored."""
    return to_storage(scale * rng.standard_normal((n, m)), dtype)
