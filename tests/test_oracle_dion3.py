"""Pins for the oracle's Dion3 step:

* top-k selection against brute force over all k-subsets on tiny inputs with ties;
* bf16 accumulate / error feedback / weight update against torch's CPU bf16 and fp32
  arithmetic (independent library routines);
* the error-feedback invariant (unselected momentum rows untouched, selected rows
  decayed by mu) from the Dion3 page, 前置知识 (error feedback) / Algorithm 4;
* f = 1 reproduces Muon's momentum recursion M <- mu M + G exactly (float64),
  stated on the Dion3 summary page (m.montaan.com);
* the step on a caller-chosen row set (random selection): its invariants, the
  all-rows case against the Newton-Schulz oracle, and equality with the top-k step
  when given the top-k set.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import (accumulate, row_scores, select_topk, error_feedback, weight_update,
                    dion3_step, newton_schulz, bf16_to_f64, f64_to_bf16_rne, k_from_fraction)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def tbf(bits):
    return torch.from_numpy(np.asarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_of(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def brute_topk(scores, k):
    n = len(scores)
    valid = []
    for S in itertools.combinations(range(n), k):
        s = set(S)
        ok = all((scores[i] > scores[j]) or (scores[i] == scores[j] and i < j)
                 for i in s for j in range(n) if j not in s)
        if ok:
            valid.append(S)
    assert len(valid) == 1
    return np.array(valid[0])


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = 9
    scores = rng.integers(0, 4, size=n).astype(np.float64)   # many ties
    for k in (1, 3, 5, 9):
        assert np.array_equal(select_topk(scores, k), brute_topk(list(scores), k))


def test_k_rule():
    assert k_from_fraction(0.25, 8192) == 2048
    assert k_from_fraction(1 / 8, 8192) == 1024
    assert k_from_fraction(0.3, 10) == 3
    assert k_from_fraction(0.31, 10) == 4
    assert k_from_fraction(1.0, 77) == 77


def test_accumulate_matches_torch_bf16_add():
    rng = np.random.default_rng(1)
    m = synth.to_storage(rng.standard_normal((64, 300)) * 0.02, "bf16")
    g = synth.to_storage(rng.standard_normal((64, 300)) * np.exp(rng.uniform(-20, 5, (64, 300))), "bf16")
    ref = bits_of(tbf(m) + tbf(g))          # torch: fp32 add, one rounding to bf16
    assert np.array_equal(accumulate(m, g), ref)


def test_row_scores():
    rng = np.random.default_rng(2)
    m = synth.to_storage(rng.standard_normal((32, 1000)) * 0.02, "bf16")
    x = bf16_to_f64(m)
    assert np.allclose(row_scores(m, "l1"), np.abs(x).sum(1), rtol=1e-13, atol=0)
    assert np.allclose(row_scores(m, "l2"), (x * x).sum(1), rtol=1e-13, atol=0)
    small = synth.to_storage(np.array([[1.0, -2.0, 0.5], [0.0, 0.0, -3.0]]), "bf16")
    assert list(row_scores(small, "l1")) == [3.5, 3.0]
    assert list(row_scores(small, "l2")) == [5.25, 9.0]


def test_error_feedback_matches_torch():
    rng = np.random.default_rng(3)
    m = synth.to_storage(rng.standard_normal((40, 256)) * 0.02, "bf16")
    S = np.array([0, 3, 7, 39])
    out = error_feedback(m, S, 0.95)
    ref = tbf(m).clone()
    ref[S] = (torch.tensor(0.95, dtype=torch.float32) * tbf(m)[S].float()).to(torch.bfloat16)
    assert np.array_equal(out, bits_of(ref))
    rest = np.setdiff1d(np.arange(40), S)
    assert np.array_equal(out[rest], m[rest])


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_weight_update_matches_torch(wd):
    rng = np.random.default_rng(4)
    w = synth.to_storage(rng.standard_normal((30, 128)) * 0.02, "bf16")
    S = np.array([1, 2, 10, 29])
    o = bf16_to_f64(synth.to_storage(rng.standard_normal((4, 128)) * 0.1, "bf16"))
    lr = 0.02
    out = weight_update(w, S, o, lr, wd)
    f = torch.float32
    lr_t, wd_t = torch.tensor(lr, dtype=f), torch.tensor(wd, dtype=f)
    d = torch.tensor(1.0, dtype=f) - lr_t * wd_t
    wt = tbf(w).float()
    ref = (d * wt).to(torch.bfloat16) if wd else tbf(w).clone()
    upd = d * wt[S] - lr_t * torch.from_numpy(o).to(f)
    ref[S] = upd.to(torch.bfloat16)
    assert np.array_equal(out, bits_of(ref))


def test_dion3_error_feedback_invariants():
    w, g, m = synth.dion3_state(n=48, m=256, seed=5)
    k = k_from_fraction(0.25, 48)
    w2, m2, S, O = dion3_step(w, m, g, k, lr=0.02, wd=0.0, mu=0.95)
    m1 = accumulate(m, g)
    rest = np.setdiff1d(np.arange(48), S)
    assert np.array_equal(m2[rest], m1[rest])               # unselected rows keep M + G
    assert np.array_equal(m2[S], error_feedback(m1, S, 0.95)[S])
    assert np.array_equal(w2[rest], w[rest])                 # wd = 0: unselected W untouched
    assert len(S) == k and np.all(np.diff(S) > 0)
    # the selected rows are those with the largest l1 norms of M + G
    sc = np.abs(bf16_to_f64(m1)).sum(1)
    assert sc[S].min() >= sc[rest].max()
    assert np.allclose(O, newton_schulz(bf16_to_f64(m1[S])), rtol=0, atol=1e-15)


def test_f_equals_one_is_muon():
    assert GOLD["f_equals_one_is_muon"]["value"] is True
    rng = np.random.default_rng(6)
    n, mm, mu, lr = 12, 40, 0.95, 0.01
    w = rng.standard_normal((n, mm))
    state = np.zeros((n, mm))
    w_muon, m_muon = w.copy(), np.zeros((n, mm))
    for step in range(3):
        g = rng.standard_normal((n, mm))
        w, state, S, O = dion3_step(w, state, g, k=n, lr=lr, wd=0.0, mu=mu, storage="f64")
        m_muon = mu * m_muon + g                 # Muon's heavy-ball momentum
        o_muon = newton_schulz(m_muon)
        w_muon = w_muon - lr * o_muon
        assert np.array_equal(S, np.arange(n))
        assert np.allclose(O, o_muon, rtol=0, atol=1e-12)
        assert np.allclose(w, w_muon, rtol=0, atol=1e-12)


# ---- a caller-chosen row set (random selection, the pages' alternative to top-k) ----

def test_dion3_step_rows_invariants_random_set():
    w, g, m = synth.dion3_state(n=64, m=256, seed=21)
    rng = np.random.default_rng(22)
    S = np.sort(rng.choice(64, size=16, replace=False))
    w2, m2, O = oracle.dion3_step_rows(w, m, g, S, lr=0.02, wd=0.0, mu=0.95)
    m1 = accumulate(m, g)
    rest = np.setdiff1d(np.arange(64), S)
    assert np.array_equal(m2[rest], m1[rest])                  # unselected: M + G only
    assert np.array_equal(w2[rest], w[rest])                    # wd = 0: unselected W untouched
    # selected momentum rows decay by mu, rounded once (torch's own bf16 arithmetic)
    ref_m = (torch.tensor(np.float32(0.95)) * tbf(m1[S]).float()).to(torch.bfloat16)
    assert np.array_equal(m2[S], bits_of(ref_m))
    # O is the orthogonalised selected submatrix, and W[S] gets -lr O in one rounding
    assert np.allclose(O, newton_schulz(bf16_to_f64(m1[S])), rtol=0, atol=1e-15)
    o_b = tbf(f64_to_bf16_rne(O)).float()
    ref_w = (tbf(w[S]).float() - torch.tensor(np.float32(0.02)) * o_b).to(torch.bfloat16)
    assert np.array_equal(w2[S], bits_of(ref_w))


def test_dion3_step_rows_all_rows_orthogonalises_accumulated_momentum():
    w, g, m = synth.dion3_state(n=24, m=96, seed=23)
    w2, m2, O = oracle.dion3_step_rows(w, m, g, np.arange(24), lr=0.01, wd=0.0, mu=0.9)
    m1 = accumulate(m, g)
    assert np.allclose(O, newton_schulz(bf16_to_f64(m1)), rtol=0, atol=1e-15)
    assert np.array_equal(m2, error_feedback(m1, np.arange(24), 0.9))


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_rows_on_topk_set_equals_dion3_step(wd):
    w, g, m = synth.dion3_state(n=40, m=128, seed=24)
    w_a, m_a, S, O_a = dion3_step(w, m, g, 10, lr=0.02, wd=wd, mu=0.95, norm="l2")
    w_b, m_b, O_b = oracle.dion3_step_rows(w, m, g, S, lr=0.02, wd=wd, mu=0.95)
    assert np.array_equal(w_a, w_b) and np.array_equal(m_a, m_b) and np.array_equal(O_a, O_b)


@pytest.mark.parametrize("S", [[3, 1], [1, 1, 2], [-1, 2], [0, 8], []])
def test_dion3_step_rows_rejects_bad_sets(S):
    w, g, m = synth.dion3_state(n=8, m=16, seed=25)
    with pytest.raises(ValueError):
        oracle.dion3_step_rows(w, m, g, S, lr=0.01)


# ---- column selection (the pages' "rows or columns") ----

@pytest.mark.parametrize("norm", ["l1", "l2"])
def test_dion3_step_cols_selects_columns_by_norm_and_keeps_invariants(norm):
    w, g, m = synth.dion3_state(n=96, m=40, seed=31)       # tall: 96 rows, 40 columns
    k = k_from_fraction(0.25, 40)
    w2, m2, S, O = oracle.dion3_step_cols(w, m, g, k, lr=0.02, wd=0.0, mu=0.95, norm=norm)
    m1 = accumulate(m, g)
    x = bf16_to_f64(m1)
    col = np.abs(x).sum(0) if norm == "l1" else (x * x).sum(0)
    rest = np.setdiff1d(np.arange(40), S)
    assert len(S) == k and np.all(np.diff(S) > 0)
    assert col[S].min() > col[rest].max()                     # the k columns of largest norm
    assert np.array_equal(m2[:, rest], m1[:, rest])          # unselected columns: M + G only
    assert np.array_equal(w2[:, rest], w[:, rest])           # wd = 0: unselected W columns untouched
    ref_m = (torch.tensor(np.float32(0.95)) * tbf(m1[:, S]).float()).to(torch.bfloat16)
    assert np.array_equal(m2[:, S], bits_of(ref_m))
    # O (k x N) is the transpose of the orthogonalised N x k column submatrix
    assert np.allclose(O.T, newton_schulz(x[:, S]), rtol=0, atol=1e-14)
    o_b = tbf(f64_to_bf16_rne(O.T)).float()
    ref_w = (tbf(w[:, S]).float() - torch.tensor(np.float32(0.02)) * o_b).to(torch.bfloat16)
    assert np.array_equal(w2[:, S], bits_of(ref_w))


# ---- the same element-wise model in the f16 and f32 state formats -----------------

TORCH_OF = {"f16": torch.float16, "f32": torch.float32}
NP_OF = {"f16": np.float16, "f32": np.float32}


def t_of(a, storage):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=NP_OF[storage]))


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_state_codec_rounds_once_to_nearest_even(storage):
    """The oracle's encode (float64 -> stored format) against torch's float64 ->
    float16/float32 conversion, and on hand-built midpoints of neighbouring stored
    values, which must go to the neighbour with the even significand."""
    from oracle.dion3 import _codec
    dec, enc = _codec(storage)
    rng = np.random.default_rng(11)
    hi = 15 if storage == "f16" else 120
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-hi - 12, hi + 1, 20000))
    ref = torch.from_numpy(x).to(TORCH_OF[storage]).numpy()
    got = enc(x)
    assert got.dtype == NP_OF[storage]
    assert np.array_equal(got.view(np.uint16 if storage == "f16" else np.uint32),
                          ref.view(np.uint16 if storage == "f16" else np.uint32))
    # midpoints between neighbours: a = stored value with an even significand, b its
    # successor (odd); (a + b) / 2 is exact in float64 and must round back to a
    ui = np.uint16 if storage == "f16" else np.uint32
    bits = (rng.integers(1, 0x7000 if storage == "f16" else 0x7e000000, 4000) & ~1).astype(ui)
    a = dec(bits.view(NP_OF[storage]))
    b = dec((bits + 1).view(NP_OF[storage]))
    mid = (a + b) / 2
    assert np.array_equal(enc(mid).view(ui), bits)
    assert np.array_equal(enc(-mid).view(ui), bits | ui(0x8000 if storage == "f16" else 0x80000000))
    # every finite stored value decodes and encodes back to itself
    if storage == "f16":
        allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
        v = allb.view(np.float16)
        fin = np.isfinite(v)
        assert np.array_equal(enc(dec(v[fin])).view(np.uint16), allb[fin])


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_accumulate_matches_torch_add(storage):
    rng = np.random.default_rng(21)
    m = synth.to_storage(rng.standard_normal((64, 300)) * 0.02, storage)
    g = synth.to_storage(rng.standard_normal((64, 300)) * np.exp(rng.uniform(-12, 3, (64, 300))), storage)
    ref = (t_of(m, storage) + t_of(g, storage)).numpy()     # torch: one rounding to the format
    assert np.array_equal(accumulate(m, g, storage).view(np.uint8), ref.view(np.uint8))


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_row_scores_state_formats(storage):
    small = synth.to_storage(np.array([[1.0, -2.0, 0.5], [0.0, 0.0, -3.0]]), storage)
    assert list(row_scores(small, "l1", storage)) == [3.5, 3.0]
    assert list(row_scores(small, "l2", storage)) == [5.25, 9.0]
    rng = np.random.default_rng(22)
    m = synth.to_storage(rng.standard_normal((16, 700)) * 0.02, storage)
    x = t_of(m, storage).double()
    assert np.allclose(row_scores(m, "l1", storage), x.abs().sum(1).numpy(), rtol=1e-13, atol=0)
    assert np.allclose(row_scores(m, "l2", storage), (x * x).sum(1).numpy(), rtol=1e-13, atol=0)


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_error_feedback_matches_torch_state_formats(storage):
    rng = np.random.default_rng(23)
    m = synth.to_storage(rng.standard_normal((40, 256)) * 0.02, storage)
    S = np.array([0, 3, 7, 39])
    out = error_feedback(m, S, 0.95, storage)
    ref = t_of(m, storage).clone()
    ref[S] = (torch.tensor(0.95, dtype=torch.float32) * t_of(m, storage)[S].float()).to(TORCH_OF[storage])
    assert np.array_equal(out.view(np.uint8), ref.numpy().view(np.uint8))
    rest = np.setdiff1d(np.arange(40), S)
    assert np.array_equal(out[rest].view(np.uint8), m[rest].view(np.uint8))


@pytest.mark.parametrize("storage", ["f16", "f32"])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_weight_update_matches_torch_state_formats(storage, wd):
    rng = np.random.default_rng(24)
    w = synth.to_storage(rng.standard_normal((30, 128)) * 0.02, storage)
    S = np.array([1, 2, 10, 29])
    o = synth.to_storage(rng.standard_normal((4, 128)) * 0.1, storage).astype(np.float64)
    lr = 0.02
    out = weight_update(w, S, o, lr, wd, storage)
    f = torch.float32
    lr_t, wd_t = torch.tensor(lr, dtype=f), torch.tensor(wd, dtype=f)
    d = torch.tensor(1.0, dtype=f) - lr_t * wd_t
    wt = t_of(w, storage).float()
    ref = (d * wt).to(TORCH_OF[storage]) if wd else t_of(w, storage).clone()
    upd = d * wt[S] - lr_t * torch.from_numpy(o).to(f)
    ref[S] = upd.to(TORCH_OF[storage])
    assert np.array_equal(out.view(np.uint8), ref.numpy().view(np.uint8))


@pytest.mark.parametrize("storage", ["f16", "f32"])
def test_dion3_step_state_formats_invariants(storage):
    """The error-feedback invariants of Algorithm 4 in the f16 and f32 formats, and the
    f32 step within fp32 rounding of the unrounded (float64) step on the same state."""
    rng = np.random.default_rng(25)
    n, mm = 48, 256
    w = synth.to_storage(rng.standard_normal((n, mm)) * 0.02, storage)
    m = synth.to_storage(rng.standard_normal((n, mm)) * 0.02, storage)
    g = synth.to_storage(rng.standard_normal((n, mm)) * 0.02, storage)
    k = k_from_fraction(0.25, n)
    w2, m2, S, O = dion3_step(w, m, g, k, lr=0.02, wd=0.0, mu=0.95, storage=storage)
    m1 = accumulate(m, g, storage)
    rest = np.setdiff1d(np.arange(n), S)
    assert m2.dtype == NP_OF[storage] and w2.dtype == NP_OF[storage]
    assert np.array_equal(m2[rest].view(np.uint8), m1[rest].view(np.uint8))
    assert np.array_equal(w2[rest].view(np.uint8), w[rest].view(np.uint8))
    sc = np.abs(m1.astype(np.float64)).sum(1)
    assert sc[S].min() >= sc[rest].max()
    assert np.allclose(O, newton_schulz(m1[S].astype(np.float64)), rtol=0, atol=1e-15)
    if storage == "f32":
        w64, m64, S64, O64 = dion3_step(w.astype(np.float64), m.astype(np.float64), g.astype(np.float64), k,
                                        lr=0.02, wd=0.0, mu=0.95, storage="f64")
        assert np.array_equal(S, S64)
        assert np.allclose(w2, w64, rtol=2e-7, atol=1e-9)
        assert np.allclose(m2, m64, rtol=2e-7, atol=1e-9)
