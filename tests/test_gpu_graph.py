"""The ABI allocates nothing and issues only kernels on the caller's stream, so a call
can be captured in a HIP graph.  Each captured call is replayed several times, with
eager calls and synchronisations in between; every replay must give the same bits as
the eager call, and the replayed results are checked against the oracle on their own:
the orthogonalised outputs within 2e-2 of float64 standard Newton-Schulz, the Dion3
row sets and momenta bit-exact through a chain of steps, and the weights within O's
tolerance of the oracle's step from the same state."""
import numpy as np
import pytest

import synth
import oracle
from oracle import bf16_to_f64, newton_schulz
from gpu_helpers import to_dev, to_f64, bits, announce, rel_fro

pytestmark = pytest.mark.gpu


def w_within_bound(w_gpu_bits, w_ref_bits, lr_eff, o_ref, o_tol=2e-2):
    """Elementwise: one bf16 rounding of the larger magnitude plus lr (times the Muon
    scale) times the allowed error of O."""
    a, b = bf16_to_f64(w_gpu_bits), bf16_to_f64(w_ref_bits)
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + lr_eff * o_tol * np.abs(o_ref).max()
    return bool(np.all(np.abs(a - b) <= bound))


def ns_parity(out_bits, st):
    """Every matrix of a replayed bf16 output against the oracle."""
    for b in range(st.shape[0]):
        e = rel_fro(bf16_to_f64(out_bits[b]), newton_schulz(bf16_to_f64(st[b])))
        assert e <= 2e-2, (b, e)


@pytest.mark.parametrize("fn", ["orthogonalize", "newton_schulz"])
def test_graph_replays_match_eager(gns_mod, fn):
    import torch
    announce(f"graph capture {fn}")
    st = synth.gns_batch("gns_1024x4096_bf16", batch=2, n=512, m=2048, seed=21)
    X = to_dev(st, "bf16")
    f = getattr(gns_mod, fn)
    ref = bits(f(X))
    out = torch.empty_like(X)
    for _ in range(3):
        f(X, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        f(X, out=out)
    for _ in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), ref)
        f(X)                          # eager work between replays
        torch.cuda.synchronize()
    ns_parity(bits(out), st)


@pytest.mark.parametrize("method", ["orthogonalize", "newton_schulz"])
def test_graphed_call_owns_buffers_and_follows_input(gns_mod, method):
    """graphed_* captures one call on its own workspace and output; a replay after the
    input is refilled in place gives the eager result for the new contents, bitwise,
    also after an eager call that needs a larger shared workspace."""
    import torch
    announce(f"graphed {method}")
    st1 = synth.gns_batch("gns_1024x4096_bf16", batch=2, n=256, m=1024, seed=31)
    st2 = synth.gns_batch("gns_1024x4096_bf16", batch=2, n=256, m=1024, seed=32)
    X = to_dev(st1, "bf16")
    eager = getattr(gns_mod, method)
    g = getattr(gns_mod, f"graphed_{method}")(X)
    ref1 = bits(eager(to_dev(st1, "bf16")))
    ref2 = bits(eager(to_dev(st2, "bf16")))
    for rep in range(3):
        assert np.array_equal(bits(g.replay()), ref1)
        torch.cuda.synchronize()
        big = to_dev(synth.gns_batch("gns_1024x4096_bf16", batch=1, n=512, m=2048, seed=33), "bf16")
        eager(big)                    # grows the shared workspace; the graph's is its own
        torch.cuda.synchronize()
    ns_parity(bits(g.replay()), st1)
    X.copy_(to_dev(st2, "bf16"))
    for rep in range(2):
        assert np.array_equal(bits(g.replay()), ref2)
        torch.cuda.synchronize()
    ns_parity(bits(g.replay()), st2)


def test_graphed_dion3_steps_match_eager_steps(gns_mod):
    """Three replays of a captured Dion3 step equal three eager steps from the same
    state, bitwise (W, M and S), with the gradient refilled in place between steps."""
    import torch
    announce("graphed dion3")
    w, g0, m = synth.dion3_state(n=512, m=2048, seed=41)
    grads = [synth.dion3_state(n=512, m=2048, seed=50 + i)[1] for i in range(3)]
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    k, lr = 128, 0.02
    We, Me = tb(w), tb(m)
    Se = []
    for gr in grads:
        Se.append(gns_mod.dion3_step(We, Me, tb(gr), k, lr, 0.1, 0.95, score_norm=2).cpu().numpy())
    Wg, Mg, Gg = tb(w), tb(m), tb(g0)
    step = gns_mod.graphed_dion3_step(Wg, Mg, Gg, k, lr, 0.1, 0.95, score_norm=2, return_O=True)
    assert np.array_equal(bits(Wg), w.view(np.uint16)) and np.array_equal(bits(Mg), m.view(np.uint16))
    w_prev, m_prev = w, m
    for i, gr in enumerate(grads):
        Gg.copy_(tb(gr))
        S, O = step.replay()
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), Se[i])
        # the oracle's step from the replay's previous state: S and M bit-exact (they
        # do not depend on O), O within 2e-2, W within O's tolerance
        w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w_prev, m_prev, gr, k, lr, wd=0.1, mu=0.95, norm="l2")
        assert np.array_equal(S.cpu().numpy(), S_ref)
        assert np.array_equal(bits(Mg), m_ref)
        assert rel_fro(to_f64(O), O_ref) <= 2e-2
        assert w_within_bound(bits(Wg), w_ref, lr, O_ref)
        w_prev, m_prev = bits(Wg), bits(Mg)
    assert np.array_equal(bits(Wg), bits(We))
    assert np.array_equal(bits(Mg), bits(Me))


def test_graphed_dion3_with_device_scalars_follows_a_schedule(gns_mod):
    """One capture with lr, weight decay and mu in device memory; three replays with a
    different (lr, wd, mu) written before each equal three eager dion3_step calls with
    those host values, bitwise (W, M and S)."""
    import torch
    announce("graphed dion3 with device scalars")
    w, g0, m = synth.dion3_state(n=512, m=2048, seed=42)
    grads = [synth.dion3_state(n=512, m=2048, seed=60 + i)[1] for i in range(3)]
    sched = [(0.02, 0.1, 0.95), (0.015, 0.0, 0.9), (0.01, 0.05, 0.95)]
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    k = 128
    We, Me = tb(w), tb(m)
    Se = []
    for gr, (lr, wd, mu) in zip(grads, sched):
        Se.append(gns_mod.dion3_step(We, Me, tb(gr), k, lr, wd, mu, score_norm=1).cpu().numpy())
    Wg, Mg, Gg = tb(w), tb(m), tb(g0)
    step = gns_mod.graphed_dion3_step(Wg, Mg, Gg, k, 0.5, 0.5, 0.5, score_norm=1, device_scalars=True,
                                      return_O=True)
    w_prev, m_prev = w, m
    for i, (gr, (lr, wd, mu)) in enumerate(zip(grads, sched)):
        Gg.copy_(tb(gr))
        step.set_scalars(lr, wd, mu)
        S, O = step.replay()
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), Se[i])
        w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w_prev, m_prev, gr, k, lr, wd=wd, mu=mu, norm="l1")
        assert np.array_equal(S.cpu().numpy(), S_ref)
        assert np.array_equal(bits(Mg), m_ref)
        assert rel_fro(to_f64(O), O_ref) <= 2e-2
        assert w_within_bound(bits(Wg), w_ref, lr, O_ref)
        w_prev, m_prev = bits(Wg), bits(Mg)
    assert np.array_equal(bits(Wg), bits(We))
    assert np.array_equal(bits(Mg), bits(Me))


def test_graphed_muon_steps_match_eager_steps(gns_mod):
    """Three replays of a captured Muon step on a batch of three equal three eager
    steps from the same state, bitwise (W, M and O), with the gradient refilled in
    place between steps."""
    import torch
    announce("graphed muon")
    st = [synth.dion3_state(n=256, m=1024, seed=60 + b) for b in range(3)]
    w = np.stack([s[0] for s in st])
    m = np.stack([s[2] for s in st])
    grads = [np.stack([synth.dion3_state(n=256, m=1024, seed=70 + 3 * i + b)[1] for b in range(3)]) for i in range(3)]
    tb = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    We, Me = tb(w), tb(m)
    Oe = []
    for gr in grads:
        Oe.append(bits(gns_mod.muon_step(We, Me, tb(gr), 0.02, weight_decay=0.1, mu=0.95, return_O=True)))
    Wg, Mg, Gg = tb(w), tb(m), tb(grads[0])
    step = gns_mod.graphed_muon_step(Wg, Mg, Gg, 0.02, weight_decay=0.1, mu=0.95, return_O=True)
    assert np.array_equal(bits(Wg), w.view(np.uint16)) and np.array_equal(bits(Mg), m.view(np.uint16))
    w_prev, m_prev = w, m
    sc = float(oracle.muon_scale(256, 1024))
    for i, gr in enumerate(grads):
        Gg.copy_(tb(gr))
        O = step.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(O), Oe[i])
        # the oracle's step from the previous state: M bit-exact, O within 2e-2, W within
        # O's tolerance
        Wb, Mb, Ob = bits(Wg), bits(Mg), bits(O)
        for b in range(3):
            w_ref, m_ref, o_ref = oracle.muon_step(w_prev[b], m_prev[b], gr[b], 0.02, wd=0.1, mu=0.95)
            assert np.array_equal(Mb[b], m_ref)
            assert rel_fro(bf16_to_f64(Ob[b]), o_ref) <= 2e-2
            assert w_within_bound(Wb[b], w_ref, 0.02 * sc, o_ref)
        w_prev, m_prev = Wb, Mb
    assert np.array_equal(bits(Wg), bits(We))
    assert np.array_equal(bits(Mg), bits(Me))
