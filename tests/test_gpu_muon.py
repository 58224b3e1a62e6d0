"""GPU parity of the Muon step (muon_step_batched) against the oracle.

Bit-exact: the momentum M after each step, and W given the GPU's own O (the decay
and the scaled update are element-wise with one rounding).  Within tolerance: O
(relative Frobenius <= 2e-2 against float64 standard NS of the oracle's U), and W
against the oracle's full step (elementwise within one bf16 rounding plus lr scale
times O's tolerance).  Shapes cover a ragged batch, a tall matrix, square matrices
(which run standard NS, the aspect-ratio-1 fallback), rows with a stride wider than m,
and the 1024 x 4096 workload, with and without the lookahead and the weight decay.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import bf16_to_f64, muon_scale, decay_and_update
from gpu_helpers import to_dev, to_f64, rel_fro, announce, bits

pytestmark = pytest.mark.gpu


def states(B, n, m, seed):
    ws, gs, ms = zip(*(synth.dion3_state(n=n, m=m, seed=seed + b) for b in range(B)))
    return np.stack(ws), np.stack(gs), np.stack(ms)


def w_within_bound(w_gpu_bits, w_ref_bits, lr_eff, o_ref, o_tol=2e-2):
    """Elementwise: one bf16 rounding of the larger magnitude plus lr scale times the
    allowed error of O (o_tol max |O|)."""
    a, b = bf16_to_f64(w_gpu_bits), bf16_to_f64(w_ref_bits)
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + lr_eff * o_tol * np.abs(o_ref).max()
    ratio = np.abs(a - b) / bound
    print(f"W: max |dW|/bound = {ratio.max():.3f}")
    return bool(np.all(ratio <= 1.0))


@pytest.mark.parametrize("B,n,m,nesterov,wd", [(1, 64, 256, True, 0.0), (3, 136, 200, False, 0.1),
                                              (2, 256, 64, True, 0.1), (1, 1024, 4096, True, 0.0),
                                              (2, 256, 256, True, 0.1), (2, 256, 256, False, 0.0),
                                              (1, 1032, 512, True, 0.1)])
def test_muon_step_matches_oracle(gns_mod, B, n, m, nesterov, wd):
    """Shapes cover the Gram path fed by the momentum pass's row sums (n <= 1024: wide,
    tall through the transpose, square through standard NS) and, at n = 1032, the
    separate scale launch."""
    announce(f"muon step B={B} {n}x{m} nesterov={nesterov} wd={wd}")
    w, g, mo = states(B, n, m, seed=200 + n)
    lr, mu = 0.02, 0.95
    W, M, G = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    O = gns_mod.muon_step(W, M, G, lr, weight_decay=wd, mu=mu, nesterov=nesterov, return_O=True)
    Wb, Mb, Ob = bits(W), bits(M), bits(O)
    sc = float(muon_scale(n, m))
    for b in range(B):
        w_ref, m_ref, o_ref = oracle.muon_step(w[b], mo[b], g[b], lr, wd=wd, mu=mu, nesterov=nesterov)
        assert np.array_equal(Mb[b], m_ref)
        e = rel_fro(bf16_to_f64(Ob[b]), o_ref)
        print(f"entry {b}: O rel err {e:.3e}")
        assert e <= 2e-2
        # the update given the GPU's own O is exact
        assert np.array_equal(Wb[b], decay_and_update(w[b], bf16_to_f64(Ob[b]), lr, wd, sc))
        assert w_within_bound(Wb[b], w_ref, lr * sc, o_ref)


@pytest.mark.parametrize("B,n,m", [(3, 128, 512), (2, 1024, 16384)])
def test_muon_batched_equals_single_entries(gns_mod, B, n, m):
    """A batch gives each entry bitwise the step of that entry alone, also at K = 16384
    where the Gram products split K (the split depends on the shape only)."""
    announce(f"muon batched == single {B}x{n}x{m}")
    w, g, mo = states(B, n, m, seed=300)
    W, M, G = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    O = gns_mod.muon_step(W, M, G, 0.02, weight_decay=0.1, return_O=True)
    for b in range(B):
        Wi, Mi, Gi = to_dev(w[b], "bf16"), to_dev(mo[b], "bf16"), to_dev(g[b], "bf16")
        Oi = gns_mod.muon_step(Wi, Mi, Gi, 0.02, weight_decay=0.1, return_O=True)
        assert np.array_equal(bits(Oi), bits(O)[b])
        assert np.array_equal(bits(Wi), bits(W)[b])
        assert np.array_equal(bits(Mi), bits(M)[b])


def test_muon_three_steps(gns_mod):
    """Three steps in a row: M stays bit-exact (it does not depend on O), each step's
    O and W stay within their bounds of the oracle's step on the GPU's previous W."""
    announce("muon three steps")
    n, m = 128, 384
    w, _, mo = synth.dion3_state(n=n, m=m, seed=310)
    W, M = to_dev(w, "bf16"), to_dev(mo, "bf16")
    m_ref = mo
    sc = float(muon_scale(n, m))
    for step in range(3):
        _, g, _ = synth.dion3_state(n=n, m=m, seed=320 + step)
        w_prev = bits(W)
        O = gns_mod.muon_step(W, M, to_dev(g, "bf16"), 0.01, weight_decay=0.1, mu=0.9, return_O=True)
        w_ref, m_ref, o_ref = oracle.muon_step(w_prev, m_ref, g, 0.01, wd=0.1, mu=0.9)
        assert np.array_equal(bits(M), m_ref)
        assert rel_fro(to_f64(O), o_ref) <= 2e-2
        assert w_within_bound(bits(W), w_ref, 0.01 * sc, o_ref)


def test_muon_zero_gradient_is_pure_decay(gns_mod):
    announce("muon zero gradient")
    w, _, _ = synth.dion3_state(n=64, m=128, seed=330)
    z = np.zeros_like(w)
    W, M, G = to_dev(w, "bf16"), to_dev(z, "bf16"), to_dev(z, "bf16")
    O = gns_mod.muon_step(W, M, G, 0.02, weight_decay=0.1, return_O=True)
    w_ref, m_ref, _ = oracle.muon_step(w, z, z, 0.02, wd=0.1)
    assert not bits(O).any() and not bits(M).any()
    assert np.array_equal(bits(W), w_ref)


def test_muon_explicit_scale(gns_mod):
    announce("muon explicit scale")
    w, g, mo = synth.dion3_state(n=64, m=256, seed=340)
    W, M, G = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    O = gns_mod.muon_step(W, M, G, 0.02, scale=1.0, nesterov=False, return_O=True)
    assert np.array_equal(bits(W), decay_and_update(w, bf16_to_f64(bits(O)), 0.02, 0.0, 1.0))
    w_ref, _, o_ref = oracle.muon_step(w, mo, g, 0.02, nesterov=False, scale=1.0)
    assert rel_fro(to_f64(O), o_ref) <= 2e-2
    assert w_within_bound(bits(W), w_ref, 0.02, o_ref)


@pytest.mark.parametrize("nesterov", [False, True])
def test_muon_step_on_strided_rows(gns_mod, nesterov):
    """W, M, G are column slices of wider buffers (row stride 320 for m = 256): the
    momentum and update passes and, without the lookahead, the Gram NS read them in
    place at that stride.  Same bars as the contiguous case; the padding columns are
    left untouched."""
    import torch
    announce(f"muon strided rows nesterov={nesterov}")
    n, m, ld = 128, 256, 320
    w, g, mo = synth.dion3_state(n=n, m=m, seed=350)
    pad = np.full((n, ld - m), 0x3F80, dtype=np.uint16)        # bf16 1.0
    wide = lambda a: to_dev(np.concatenate([a, pad], axis=1), "bf16")
    Wf, Mf, Gf = wide(w), wide(mo), wide(g)
    W, M, G = Wf[:, :m], Mf[:, :m], Gf[:, :m]
    assert W.stride() == (ld, 1)
    O = gns_mod.muon_step(W, M, G, 0.02, weight_decay=0.1, nesterov=nesterov, return_O=True)
    torch.cuda.synchronize()
    w_ref, m_ref, o_ref = oracle.muon_step(w, mo, g, 0.02, wd=0.1, nesterov=nesterov)
    assert np.array_equal(bits(M), m_ref)
    assert rel_fro(to_f64(O), o_ref) <= 2e-2
    sc = float(muon_scale(n, m))
    assert np.array_equal(bits(W), decay_and_update(w, bf16_to_f64(bits(O)), 0.02, 0.1, sc))
    for full in (Wf, Mf, Gf):
        assert np.array_equal(bits(full[:, m:]), pad)


def test_muon_scale_must_be_positive(gns_mod):
    """scale=None selects 0.2 sqrt(max(n, m)); an explicit scale must be positive (an
    explicit 0 or a negative value is refused, not turned into the default)."""
    w, g, mo = synth.dion3_state(n=64, m=128, seed=360)
    W, M, G = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    for bad in (0.0, -1.0):
        with pytest.raises(ValueError):
            gns_mod.muon_step(W, M, G, 0.02, scale=bad)
    assert np.array_equal(bits(W), w) and np.array_equal(bits(M), mo)
