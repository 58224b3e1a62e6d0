"""Pins for the oracle's standard and Gram Newton-Schulz (float64), against what the
pages and the mathematics fix, not against the oracle's own formulas:

* SVD closed form: an odd matrix polynomial acts on each singular value as the
  scalar polynomial ("Muon: Orthogonalized Momentum ...", 'Doing an SVD without an
  SVD'), so NS(X) = U phi^T(Sigma / (||X||_F + eps)) V^T, computed here with numpy's
  SVD and scalar arithmetic.
* closed forms for diagonal and orthonormal-row inputs, permutation equivariance,
  transposition, zero input, the output band the blog states.
* Gram NS equals standard NS in exact arithmetic, with and without restart, and for
  per-step coefficient tables (Dion3 page, 核心方法 theorem 2 / 方法步骤详情).
* a spurious negative eigenvalue of -4e-4 (the pages' figure) makes the
  restart-free iteration diverge even in float64, and the restart prevents it.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import (JORDAN_ABC, EPS, newton_schulz, gram_newton_schulz, quintic_composed)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def scalar_phi_T(x, steps=5, abc=(3.4445, -4.7750, 2.0315)):
    # written independently of the oracle: Horner form of a x + b x^3 + c x^5
    a, b, c = abc
    for _ in range(steps):
        x2 = x * x
        x = x * (a + x2 * (b + c * x2))
    return x


def test_constants_match_pages():
    assert tuple(JORDAN_ABC) == tuple(GOLD["ns_coefficients"]["value"])
    assert EPS == GOLD["ns_eps"]["value"]


@pytest.mark.parametrize("shape", [(8, 8), (16, 40), (40, 16), (64, 256), (33, 97)])
@pytest.mark.parametrize("seed", [0, 1])
def test_svd_closed_form(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-6, 0, size=(shape[0], 1)))
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    fro = np.sqrt(np.sum(s ** 2))
    expected = (u * scalar_phi_T(s / (fro + 1e-7))) @ vt
    got = newton_schulz(x)
    assert rel(got, expected) < 1e-10


def test_diagonal_closed_form():
    d = np.array([3.0, 1.0, 0.5, 0.01, 1e-4])
    x = np.zeros((5, 12))
    x[np.arange(5), np.arange(5)] = d
    got = newton_schulz(x)
    dn = d / (np.sqrt(np.sum(d * d)) + 1e-7)
    expected = np.zeros_like(x)
    expected[np.arange(5), np.arange(5)] = scalar_phi_T(dn)
    assert rel(got, expected) < 1e-12


def test_orthonormal_rows_scale():
    rng = np.random.default_rng(3)
    q, _ = np.linalg.qr(rng.standard_normal((256, 64)))
    x = q.T                                       # 64 x 256, orthonormal rows, sigma = 1
    got = newton_schulz(x)
    c = scalar_phi_T(np.array([1.0 / (8.0 + 1e-7)]))[0]   # ||x||_F = sqrt(64) = 8
    assert rel(got, c * x) < 1e-12
    assert 0.68 < c < 0.70


def test_rank_one_closed_form():
    rng = np.random.default_rng(4)
    u = rng.standard_normal(20)
    v = rng.standard_normal(50)
    x = np.outer(u, v)
    got = newton_schulz(x)
    uu, vv = u / np.linalg.norm(u), v / np.linalg.norm(v)
    s = np.linalg.norm(x)
    expected = scalar_phi_T(np.array([s / (s + 1e-7)]))[0] * np.outer(uu, vv)
    assert rel(got, expected) < 1e-12


def test_permutation_and_transpose_equivariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((24, 70))
    p = rng.permutation(24)
    q = rng.permutation(70)
    base = newton_schulz(x)
    assert rel(newton_schulz(x[p][:, q]), base[p][:, q]) < 1e-12
    assert rel(newton_schulz(x.T), base.T) < 1e-12


def test_zero_input_gives_zero():
    assert np.all(newton_schulz(np.zeros((4, 9))) == 0.0)
    assert np.all(gram_newton_schulz(np.zeros((4, 9))) == 0.0)


def test_output_band_stated_by_blog():
    lo, hi = GOLD["output_singular_value_band"]["value"]
    # singular values of a normalised input lie in (0, 1]; over the range where the
    # iteration has converged the outputs stay near [0.7, 1.3] (the blog's "roughly")
    grid = np.linspace(2e-3, 1.0, 20001)
    out = quintic_composed(grid)
    assert out.min() > lo - 0.05 and out.max() < hi


@pytest.mark.parametrize("shape", [(16, 64), (32, 32), (48, 20), (64, 256)])
@pytest.mark.parametrize("restart_after", [(), (2,), (1, 3), (1, 2, 3, 4)])
def test_gram_equals_standard_fp64(shape, restart_after):
    rng = np.random.default_rng(7)
    n, m = shape
    k = min(n, m)
    u, _ = np.linalg.qr(rng.standard_normal((n, k)))
    v, _ = np.linalg.qr(rng.standard_normal((m, k)))
    x = (u * (1.0 / np.arange(1, k + 1))) @ v.T
    assert rel(gram_newton_schulz(x, restart_after=restart_after), newton_schulz(x)) < 1e-10


def test_gram_equals_standard_per_step_table():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((20, 60))
    table = np.array([[3.4, -4.7, 2.0], [3.0, -3.5, 1.2], [2.5, -2.0, 0.6],
                      [1.9, -1.3, 0.4], [1.875, -1.25, 0.375]])
    a = newton_schulz(x, abc=table)
    b = gram_newton_schulz(x, abc=table, restart_after=(2,))
    assert rel(b, a) < 1e-10
    s = np.linalg.svd(x, compute_uv=False)
    sn = s / (np.sqrt(np.sum(s * s)) + 1e-7)
    y = sn.copy()
    for (p, q, r) in table:
        y = p * y + q * y ** 3 + r * y ** 5
    assert np.allclose(np.sort(np.linalg.svd(a, compute_uv=False)), np.sort(np.abs(y)), rtol=1e-10)


def test_batched_matches_loop():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 10, 30))
    got = newton_schulz(x)
    for i in range(3):
        assert rel(got[i], newton_schulz(x[i])) < 1e-15


def _with_negative_eigenvalue(value):
    def perturb(R):
        w, v = np.linalg.eigh(R)
        w = w.copy()
        w[0] = value
        return (v * w) @ v.T
    return perturb


def test_negative_eigenvalue_diverges_without_restart():
    neg = GOLD["spurious_negative_eigenvalue"]["value"]
    rng = np.random.default_rng(10)
    u, _ = np.linalg.qr(rng.standard_normal((32, 32)))
    v, _ = np.linalg.qr(rng.standard_normal((128, 32)))
    x = (u * np.linspace(1.0, 1e-3, 32)) @ v.T
    good = newton_schulz(x)
    no_restart = gram_newton_schulz(x, restart_after=(), perturb_r0=_with_negative_eigenvalue(neg))
    with_restart = gram_newton_schulz(x, restart_after=(2,), perturb_r0=_with_negative_eigenvalue(neg))
    # theorem 2's scalar recursion with r0 = -4e-4: r <- r h(r)^2 reaches about
    # -2.8e9 in five steps while q = prod h(r) grows by ~2.6e6
    r, q = neg, 1.0
    for _ in range(5):
        h = 3.4445 - 4.7750 * r + 2.0315 * r * r
        r, q = r * h * h, q * h
    assert r < -1e9 and q > 1e6
    s_bad = np.linalg.svd(no_restart, compute_uv=False)
    s_ok = np.linalg.svd(with_restart, compute_uv=False)
    # the perturbed direction is the one of X's smallest singular value; the output
    # there is q_T * sigma_min(normalised X), far outside the healthy band
    sig_min = 1e-3 / (np.linalg.norm(x) + 1e-7)
    assert abs(s_bad.max() / (q * sig_min) - 1) < 1e-8
    assert s_bad.max() > 100
    assert s_ok.max() < 1.3           # bounded: the restart flushed the spurious eigenvalue
    assert rel(with_restart, good) < 0.05


def test_restart_trace_resets_q():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((16, 64))
    tr = []
    gram_newton_schulz(x, restart_after=(2,), trace=tr)
    steps = [t for t, _, _ in tr]
    assert steps == [1, 2, 3, 4, 5]
    # Q is the identity entering step 1 and entering step 3 (after the restart)
    assert tr[0][2] == 1.0 and tr[2][2] == 1.0
    assert tr[1][2] > 1.0
