"""GPU parity of the Dion3 and Muon steps on f16 and fp32 states against the oracle.

The state type is the caller's (W, M, G in one dtype); the oracle follows the same
rounding model in that format (one rounding to the state type after each fp32
operation, fp64 row scores of the stored values, O stored in the state type).
Bit-exact: the accumulated momentum M, the selected set S (the oracle's scores have a
margin at the k-th row far above any fp64 summation-order difference, so S is
unique), the error feedback on M, the weight update given the same O, and the
unselected rows of W.  Within tolerance: O (relative Frobenius <= 2e-2 against float64
standard NS of the oracle's gathered rows) and the selected rows of W (one rounding in
the state type plus lr times O's tolerance).
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import accumulate, row_scores, select_topk, error_feedback, weight_update, k_from_fraction
from gpu_helpers import to_dev, to_f64, rel_fro, announce

pytestmark = pytest.mark.gpu

NP = {"f16": np.float16, "f32": np.float32}
ULP = {"f16": 2.0 ** -10, "f32": 2.0 ** -23}     # one rounding, relative to the magnitude


def state(n, m, seed, dt):
    rng = np.random.default_rng(seed)
    return tuple(synth.to_storage(rng.standard_normal((n, m)) * 0.02, dt) for _ in range(3))


def host(x, dt):
    return x.detach().cpu().numpy().astype(NP[dt])


def same(a, b):
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def unique_topk(scores, k):
    """The k-th and (k+1)-th largest scores differ by far more than fp64 summation order
    can move a score (about 1e-13 relative here), so the top-k set is unique."""
    s = np.sort(scores)[::-1]
    return k == len(s) or (s[k - 1] - s[k]) > 1e-9 * s[k - 1]


def w_within_bound(wg, wr, lr, o_ref, dt, o_tol=2e-2):
    a, b = wg.astype(np.float64), wr.astype(np.float64)
    bound = ULP[dt] * np.maximum(np.abs(a), np.abs(b)) + lr * o_tol * np.abs(o_ref).max()
    ratio = np.abs(a - b) / bound
    print(f"W: max |dW|/bound = {ratio.max():.3f}")
    return bool(np.all(ratio <= 1.0))


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("norm", [1, 2])
def test_accumulate_score_state_types(gns_mod, dt, norm):
    announce(f"dion3 accumulate_score {dt} norm={norm}")
    _, g, m = state(96, 1000 - 1000 % 8, 31, dt)
    M, G = to_dev(m, dt), to_dev(g, dt)
    score, sumsq = gns_mod.dion3_accumulate_score(M, G, norm)
    m1 = accumulate(m, g, dt)
    assert same(host(M, dt), m1)
    assert np.allclose(score.cpu().numpy(), row_scores(m1, "l1" if norm == 1 else "l2", dt), rtol=1e-13, atol=0)
    assert np.allclose(sumsq.cpu().numpy(), row_scores(m1, "l2", dt), rtol=1e-13, atol=0)


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_gather_feedback_state_types(gns_mod, dt):
    announce(f"dion3 gather_feedback {dt}")
    torch = __import__("torch")
    _, _, m = state(200, 512, 32, dt)
    S = np.array(sorted(np.random.default_rng(3).choice(200, 37, replace=False)), dtype=np.int32)
    M = to_dev(m, dt)
    X = gns_mod.dion3_gather_feedback(M, torch.from_numpy(S).cuda(), 0.95)
    assert same(host(X, dt), m[S])
    assert same(host(M, dt), error_feedback(m, S, 0.95, dt))


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("o_dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_apply_update_state_types(gns_mod, dt, o_dt, wd):
    announce(f"dion3 apply_update {dt} O={o_dt} wd={wd}")
    torch = __import__("torch")
    w, _, _ = state(160, 768, 33, dt)
    rng = np.random.default_rng(4)
    S = np.array(sorted(rng.choice(160, 40, replace=False)), dtype=np.int32)
    o_st = synth.to_storage(rng.standard_normal((40, 768)) * 0.01, o_dt)
    o = synth.bf16_bits_to_f32(o_st).astype(np.float64) if o_dt == "bf16" else o_st.astype(np.float64)
    W = to_dev(w, dt)
    gns_mod.dion3_apply_update(W, torch.from_numpy(S).cuda(), to_dev(o_st, o_dt), 0.02, wd)
    assert same(host(W, dt), weight_update(w, S, o, 0.02, wd, dt))


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("norm", [1, 2])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_state_types(gns_mod, dt, norm, wd):
    announce(f"dion3 step {dt} 512x2048 norm={norm} wd={wd}")
    w, g, m = state(512, 2048, 34, dt)
    k = k_from_fraction(0.25, 512)
    lr = 0.01 / np.sqrt(0.25)
    nm = "l1" if norm == 1 else "l2"
    assert unique_topk(row_scores(accumulate(m, g, dt), nm, dt), k)
    W, M, G = to_dev(w, dt), to_dev(m, dt), to_dev(g, dt)
    S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm, return_O=True)
    assert O.dtype == W.dtype
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, k, lr, wd=wd, mu=0.95, norm=nm, storage=dt)
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert same(host(M, dt), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2
    wg = host(W, dt)
    assert w_within_bound(wg, w_ref, lr, O_ref, dt)
    rest = np.setdiff1d(np.arange(512), S_ref)
    assert same(wg[rest], w_ref[rest])
    # the update given the GPU's own O is bit-exact
    assert same(wg, weight_update(w, S_ref, to_f64(O), lr, wd, dt))


@pytest.mark.parametrize("k", [60, 125])
def test_dion3_step_f32_any_k_rows_in_place_falls_back(gns_mod, k):
    """A k that is not a multiple of 8 (padded submatrix), and rows_in_place on an fp32
    state, which reads the rows through the gathered copy: the same bits as without."""
    announce(f"dion3 step f32 any k={k}, rows_in_place requested")
    w, g, m = state(256, 1024, 35, "f32")
    runs = []
    for rip in (False, True):
        W, M, G = to_dev(w, "f32"), to_dev(m, "f32"), to_dev(g, "f32")
        sched = gns_mod.default_schedule(rows_in_place=rip)
        S, O = gns_mod.dion3_step(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, schedule=sched,
                                  return_O=True)
        runs.append((S.cpu().numpy(), host(O, "f32"), host(W, "f32"), host(M, "f32")))
    assert all(same(a, b) for a, b in zip(runs[0], runs[1]))
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, k, 0.02, wd=0.1, mu=0.95, norm="l2", storage="f32")
    assert np.array_equal(runs[0][0], S_ref)
    assert same(runs[0][3], m_ref)
    assert rel_fro(runs[0][1].astype(np.float64), O_ref) <= 2e-2


def test_dion3_step_rows_f32(gns_mod):
    announce("dion3 step_rows f32 random set")
    torch = __import__("torch")
    w, g, m = state(384, 1536, 36, "f32")
    S = np.array(sorted(np.random.default_rng(5).choice(384, 96, replace=False)), dtype=np.int32)
    W, M, G = to_dev(w, "f32"), to_dev(m, "f32"), to_dev(g, "f32")
    O = torch.empty((96, 1536), dtype=torch.float32, device="cuda")
    gns_mod.dion3_step_rows(W, M, G, torch.from_numpy(S).cuda(), 0.02, weight_decay=0.0, mu=0.9, O=O)
    w_ref, m_ref, O_ref = oracle.dion3_step_rows(w, m, g, S, 0.02, wd=0.0, mu=0.9, storage="f32")
    assert same(host(M, "f32"), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2
    assert same(host(W, "f32"), weight_update(w, S, to_f64(O), 0.02, 0.0, "f32"))


def test_dion3_step_cols_f32(gns_mod):
    announce("dion3 step_cols f32 1024x256")
    w, g, m = state(1024, 256, 37, "f32")
    k = 64
    assert unique_topk(row_scores(accumulate(m, g, "f32").T, "l2", "f32"), k)
    W, M, G = to_dev(w, "f32"), to_dev(m, "f32"), to_dev(g, "f32")
    S, O = gns_mod.dion3_step_cols(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step_cols(w, m, g, k, 0.02, wd=0.1, mu=0.95, norm="l2",
                                                        storage="f32")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert same(host(M, "f32"), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2
    wt = weight_update(np.ascontiguousarray(w.T), S_ref, to_f64(O), 0.02, 0.1, "f32")
    assert same(host(W, "f32"), np.ascontiguousarray(wt.T))


def test_dion3_step_batched_f16_equals_single(gns_mod):
    announce("dion3 step_batched f16 3 x 256x1024")
    torch = __import__("torch")
    sts = [state(256, 1024, 40 + b, "f16") for b in range(3)]
    k = 64
    Wb = torch.stack([to_dev(s[0], "f16") for s in sts])
    Gb = torch.stack([to_dev(s[1], "f16") for s in sts])
    Mb = torch.stack([to_dev(s[2], "f16") for s in sts])
    Sb, Ob = gns_mod.dion3_step_batched(Wb, Mb, Gb, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
    for b, (w, g, m) in enumerate(sts):
        W, M, G = to_dev(w, "f16"), to_dev(m, "f16"), to_dev(g, "f16")
        S, O = gns_mod.dion3_step(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
        assert np.array_equal(S.cpu().numpy(), Sb[b].cpu().numpy())
        assert same(host(O, "f16"), host(Ob[b], "f16"))
        assert same(host(W, "f16"), host(Wb[b], "f16"))
        assert same(host(M, "f16"), host(Mb[b], "f16"))


# ---- the Muon step on f16 and fp32 states ---------------------------------------------

@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("B,n,m,nesterov,wd", [(2, 136, 200, True, 0.1), (1, 256, 64, False, 0.0),
                                              (2, 128, 128, True, 0.0)])
def test_muon_step_state_types(gns_mod, dt, B, n, m, nesterov, wd):
    announce(f"muon step {dt} B={B} {n}x{m} nesterov={nesterov} wd={wd}")
    rng = np.random.default_rng(60 + n + m)
    w, g, mo = (np.stack([synth.to_storage(rng.standard_normal((n, m)) * 0.02, dt) for _ in range(B)])
                for _ in range(3))
    lr, mu = 0.02, 0.95
    W, M, G = to_dev(w, dt), to_dev(mo, dt), to_dev(g, dt)
    O = gns_mod.muon_step(W, M, G, lr, weight_decay=wd, mu=mu, nesterov=nesterov, return_O=True)
    assert O.dtype == W.dtype
    Wh, Mh, Oh = host(W, dt), host(M, dt), host(O, dt)
    sc = float(oracle.muon_scale(n, m))
    for b in range(B):
        w_ref, m_ref, o_ref = oracle.muon_step(w[b], mo[b], g[b], lr, wd=wd, mu=mu, nesterov=nesterov, storage=dt)
        assert same(Mh[b], m_ref)
        assert rel_fro(Oh[b].astype(np.float64), o_ref) <= 2e-2
        assert same(Wh[b], oracle.decay_and_update(w[b], Oh[b].astype(np.float64), lr, wd, sc, dt))
        assert w_within_bound(Wh[b], w_ref, lr * sc, o_ref, dt)
