"""Pins for the oracle's Muon step (the Muon blog's step listing and its notes on
weight decay and update-scale matching):

* Dion3 with f = 1 is Muon (Dion3 summary, m.montaan.com): without the lookahead,
  three float64 Muon steps equal three Dion3 steps that select every row;
* the momentum and lookahead against their closed forms on dyadic inputs, where
  every operation is exact (U = (1 + mu) G + mu^2 M), and against torch's CPU float32
  arithmetic with one bf16 rounding;
* the scale against the page's 0.2 sqrt(max(d_out, d_in)), and its stated purpose:
  with an exactly orthogonal update, the scaled update has RMS 0.2 for wide and tall
  matrices alike;
* the decoupled decay: a zero gradient and zero momentum leave W <- (1 - lr wd) W.
"""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import (muon_scale, momentum, decay_and_update, muon_step, dion3_step, bf16_to_f64,
                    f64_to_bf16_rne)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def tbf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def test_f_equals_one_dion3_is_muon_without_lookahead():
    rng = np.random.default_rng(31)
    n, m, mu, lr = 12, 40, 0.95, 0.01
    w0 = rng.standard_normal((n, m))
    w_d, state_d = w0.copy(), np.zeros((n, m))
    w_m, state_m = w0.copy(), np.zeros((n, m))
    for _ in range(3):
        g = rng.standard_normal((n, m))
        w_d, state_d, S, O_d = dion3_step(w_d, state_d, g, k=n, lr=lr, wd=0.0, mu=mu, storage="f64")
        # scale 1: Dion3's update carries no RMS factor
        w_m, state_m, O_m = muon_step(w_m, state_m, g, lr, wd=0.0, mu=mu, nesterov=False, scale=1.0,
                                      storage="f64")
        assert np.allclose(O_m, O_d, rtol=0, atol=1e-12)
        assert np.allclose(w_m, w_d, rtol=0, atol=1e-12)


def test_momentum_closed_form_on_dyadic_inputs():
    """M, G in {-3..3}/8 and mu = 1/2: every product and sum is exact in float32 and
    bf16, so M' = mu M + G and U = G + mu M' = (1 + mu) G + mu^2 M hold bit for bit."""
    assert GOLD["muon_nesterov_lookahead"]["value"] == "U = G + mu * M_updated"
    rng = np.random.default_rng(32)
    m = rng.integers(-3, 4, size=(16, 24)) / 8.0
    g = rng.integers(-3, 4, size=(16, 24)) / 8.0
    mb, gb = f64_to_bf16_rne(m), f64_to_bf16_rne(g)
    m1, u = momentum(mb, gb, 0.5, nesterov=True)
    assert np.array_equal(bf16_to_f64(m1), 0.5 * m + g)
    assert np.array_equal(bf16_to_f64(u), 1.5 * g + 0.25 * m)
    m1p, up = momentum(mb, gb, 0.5, nesterov=False)
    assert np.array_equal(m1p, m1) and np.array_equal(up, m1)


def test_momentum_rounding_matches_torch_float32():
    w, g, m = synth.dion3_state(n=64, m=128, seed=33)
    mu = 0.95
    m1, u = momentum(m, g, mu, nesterov=True)
    mu32 = torch.tensor(np.float32(mu))
    ref_m = (mu32 * tbf(m).float() + tbf(g).float()).to(torch.bfloat16)
    ref_u = (tbf(g).float() + mu32 * ref_m.float()).to(torch.bfloat16)
    assert np.array_equal(m1, ref_m.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(u, ref_u.view(torch.int16).numpy().view(np.uint16))


def test_scale_is_page_formula_on_the_long_side():
    c = GOLD["muon_update_scale"]["value"]
    assert abs(float(muon_scale(64, 256)) - c * 16.0) <= 1e-6
    assert muon_scale(256, 64) == muon_scale(64, 256)          # max(d_out, d_in)
    assert abs(float(muon_scale(100, 100)) - c * 10.0) <= 1e-6
    assert abs(float(muon_scale(768, 6144)) - c * np.sqrt(6144.0)) <= 1e-5


def test_scaled_update_has_rms_point_two():
    """With the exact polar factor as the orthogonaliser (full rank), the update
    lr scale O has RMS 0.2 lr whatever the shape: the page's reason for the scale."""
    c = GOLD["muon_update_scale"]["value"]
    rng = np.random.default_rng(34)

    def polar(x):
        u, _, vt = np.linalg.svd(x, full_matrices=False)
        return u @ vt

    for n, m in [(32, 128), (128, 32), (48, 48)]:
        w = np.zeros((n, m))
        g = rng.standard_normal((n, m))
        lr = 0.01
        w1, _, _ = muon_step(w, np.zeros((n, m)), g, lr, mu=0.0, nesterov=False, storage="f64",
                             orthogonalize=polar)
        rms = np.sqrt(np.mean((w1 / lr) ** 2))
        assert abs(rms - c) <= 1e-12


def test_zero_gradient_is_pure_decay():
    assert GOLD["muon_decay_before_update"]["value"] is True
    w, _, _ = synth.dion3_state(n=32, m=64, seed=35)
    z = np.zeros_like(w)
    lr, wd = 0.02, 0.1
    w1, m1, O = muon_step(w, z, z, lr, wd=wd, mu=0.95)
    assert np.array_equal(m1, z) and not np.any(O)
    d = torch.tensor(np.float32(1.0) - np.float32(lr) * np.float32(wd))
    ref = (d * tbf(w).float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(w1, ref)
    w2, _, _ = muon_step(w, z, z, lr, wd=0.0, mu=0.95)
    assert np.array_equal(w2, w)


def test_decay_and_update_rounding_matches_torch_float32():
    w, g, _ = synth.dion3_state(n=40, m=96, seed=36)
    o = bf16_to_f64(g) * 10.0
    lr, wd, sc = 0.02, 0.1, float(muon_scale(40, 96))
    got = decay_and_update(w, o, lr, wd, sc)
    lr32, wd32, sc32 = (torch.tensor(np.float32(v)) for v in (lr, wd, sc))
    d = torch.tensor(np.float32(1.0)) - lr32 * wd32
    ref = (d * tbf(w).float() - (lr32 * sc32) * torch.from_numpy(o.astype(np.float32))).to(torch.bfloat16)
    assert np.array_equal(got, ref.view(torch.int16).numpy().view(np.uint16))


# ---- the same model in the f16 and f32 state formats ---------------------------------

TORCH_OF = {"f16": torch.float16, "f32": torch.float32}


@pytest.mark.parametrize("storage", ["f16", "f32"])
@pytest.mark.parametrize("nesterov", [False, True])
def test_momentum_matches_torch_state_formats(storage, nesterov):
    rng = np.random.default_rng(71)
    m = synth.to_storage(rng.standard_normal((24, 200)) * 0.02, storage)
    g = synth.to_storage(rng.standard_normal((24, 200)) * 0.02, storage)
    m_new, u = momentum(m, g, 0.95, nesterov, storage)
    f, dt = torch.float32, TORCH_OF[storage]
    mu = torch.tensor(0.95, dtype=f)
    mt, gt = torch.from_numpy(m).float(), torch.from_numpy(g).float()
    ref_m = (mu * mt + gt).to(dt)
    assert np.array_equal(m_new.view(np.uint8), ref_m.numpy().view(np.uint8))
    ref_u = (gt + mu * ref_m.float()).to(dt) if nesterov else ref_m
    assert np.array_equal(u.view(np.uint8), ref_u.numpy().view(np.uint8))


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_decay_and_update_matches_torch_state_formats(storage):
    rng = np.random.default_rng(72)
    w = synth.to_storage(rng.standard_normal((24, 200)) * 0.02, storage)
    o = synth.to_storage(rng.standard_normal((24, 200)) * 0.1, storage).astype(np.float64)
    lr, wd, sc = 0.02, 0.1, float(muon_scale(24, 200))
    out = decay_and_update(w, o, lr, wd, sc, storage)
    f = torch.float32
    lr_t, wd_t, sc_t = (torch.tensor(v, dtype=f) for v in (lr, wd, sc))
    d = torch.tensor(1.0, dtype=f) - lr_t * wd_t
    ref = (d * torch.from_numpy(w).float() - (lr_t * sc_t) * torch.from_numpy(o).to(f)).to(TORCH_OF[storage])
    assert np.array_equal(out.view(np.uint8), ref.numpy().view(np.uint8))


def test_muon_step_f32_within_rounding_of_the_unrounded_step():
    rng = np.random.default_rng(73)
    w, m, g = (synth.to_storage(rng.standard_normal((48, 160)) * 0.02, "f32") for _ in range(3))
    w32, m32, o32 = muon_step(w, m, g, 0.02, wd=0.1, storage="f32")
    w64, m64, o64 = muon_step(w.astype(np.float64), m.astype(np.float64), g.astype(np.float64), 0.02, wd=0.1,
                              storage="f64")
    assert w32.dtype == np.float32 and m32.dtype == np.float32
    # a few fp32 roundings of the terms (fp32 mu, the product, the sum), bounded by the
    # terms' magnitudes, not the result's (mu M and G may cancel)
    u = 2.0 ** -24
    m_bound = 4 * u * (0.95 * np.abs(m.astype(np.float64)) + np.abs(g.astype(np.float64)))
    assert np.all(np.abs(m32 - m64) <= m_bound)
    assert np.allclose(o32, o64, rtol=0, atol=1e-5)
    sc = float(muon_scale(48, 160))
    w_bound = 4 * u * (np.abs(w.astype(np.float64)) + 0.02 * sc * np.abs(o64)) + 0.02 * sc * 1e-5
    assert np.all(np.abs(w32 - w64) <= w_bound)
