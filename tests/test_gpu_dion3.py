"""GPU parity of the Dion3 step against the oracle.

Bit-exact: the accumulated momentum M, the selected row set S (ascending), the error
feedback on M, and the weight update given the same (seeded) O.  Within tolerance:
the orthogonalised submatrix O (relative Frobenius <= 2e-2 against float64 standard
NS of the oracle's gathered rows) and the selected rows of W after a full step (they
depend on O: elementwise within one bf16 rounding plus lr times O's tolerance);
unselected rows of W are bit-exact.  The step on a caller-chosen row set (random
selection) is held to the same bars, and to bitwise equality with the top-k step
when given the top-k set.
"""
import numpy as np
import pytest

import synth
import oracle
from oracle import (accumulate, row_scores, select_topk, error_feedback, weight_update, newton_schulz,
                    bf16_to_f64, f64_to_bf16_rne, k_from_fraction)
from gpu_helpers import to_dev, to_f64, rel_fro, announce, bits

pytestmark = pytest.mark.gpu


def w_within_bound(w_gpu_bits, w_ref_bits, lr, o_ref, o_tol=2e-2):
    """W after a step depends on O, which is only required within o_tol (relative).
    Elementwise bound: one bf16 rounding of the larger magnitude, plus lr times the
    allowed error of O (o_tol * max |O|).  Near W ~ lr O the result crosses zero,
    where an ulp count would be meaningless, hence an absolute bound."""
    a, b = bf16_to_f64(w_gpu_bits), bf16_to_f64(w_ref_bits)
    # one bf16 ulp is at most 2^-7 of the magnitude (8 significant bits)
    bound = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + lr * o_tol * np.abs(o_ref).max()
    ratio = np.abs(a - b) / bound
    print(f"W: max |dW|/bound = {ratio.max():.3f}, changed elements {(a != b).mean():.4f}")
    return bool(np.all(ratio <= 1.0))


@pytest.mark.parametrize("norm", [1, 2])
def test_accumulate_score_bit_exact(gns_mod, norm):
    announce(f"dion3 accumulate_score norm={norm}")
    w, g, m = synth.dion3_state(n=300, m=1024, seed=11)
    M = to_dev(m, "bf16")
    score, sumsq = gns_mod.dion3_accumulate_score(M, to_dev(g, "bf16"), norm)
    m1 = accumulate(m, g)
    assert np.array_equal(bits(M), m1)
    ref = row_scores(m1, "l1" if norm == 1 else "l2")
    assert np.allclose(score.cpu().numpy(), ref, rtol=1e-13, atol=0)
    assert np.allclose(sumsq.cpu().numpy(), row_scores(m1, "l2"), rtol=1e-13, atol=0)


@pytest.mark.parametrize("N,k", [(1, 1), (9, 4), (1000, 250), (8192, 2048), (8192, 1024), (20000, 3)])
def test_topk_bit_exact_with_ties(gns_mod, N, k):
    announce(f"dion3 topk N={N} k={k}")
    rng = np.random.default_rng(N + k)
    scores = rng.integers(0, 50, size=N).astype(np.float64) * 0.125   # many exact ties
    torch = __import__("torch")
    S = gns_mod.dion3_select_topk(torch.from_numpy(scores).cuda(), k).cpu().numpy()
    assert np.array_equal(S, select_topk(scores, k))


def test_topk_distinct_scores(gns_mod):
    announce("dion3 topk distinct")
    rng = np.random.default_rng(5)
    scores = rng.random(8192) * 100
    torch = __import__("torch")
    for k in (1, 17, 2048, 8192):
        S = gns_mod.dion3_select_topk(torch.from_numpy(scores).cuda(), k).cpu().numpy()
        assert np.array_equal(S, select_topk(scores, k))


@pytest.mark.parametrize("kind", ["equal", "zero", "two_values", "row_l2", "row_l1", "inf_and_zero"])
@pytest.mark.parametrize("N,k", [(8192, 2048), (3000, 3000), (777, 776), (20000, 5000)])
def test_topk_shared_bits_and_early_stop(gns_mod, kind, N, k):
    """Scores whose bit patterns share their leading bits (one magnitude, all equal,
    two values), the workload's row sums, and +inf among zeros."""
    announce(f"dion3 topk {kind} N={N} k={k}")
    rng = np.random.default_rng(N + k)
    if kind == "equal":
        scores = np.full(N, 3.5)
    elif kind == "zero":
        scores = np.zeros(N)
    elif kind == "two_values":
        scores = np.where(rng.random(N) < 0.5, 1.0, 2.0)
    elif kind in ("row_l2", "row_l1"):
        x = rng.normal(0.0, 0.02, size=(N, 256))
        scores = (x * x).sum(1) if kind == "row_l2" else np.abs(x).sum(1)
    else:
        scores = rng.random(N)
        scores[rng.random(N) < 0.3] = np.inf
        scores[rng.random(N) < 0.2] = 0.0
    torch = __import__("torch")
    S = gns_mod.dion3_select_topk(torch.from_numpy(scores).cuda(), k).cpu().numpy()
    assert np.array_equal(S, select_topk(scores, k))


def test_gather_feedback_bit_exact(gns_mod):
    announce("dion3 gather_feedback")
    _, _, m = synth.dion3_state(n=200, m=512, seed=12)
    S = np.array(sorted(np.random.default_rng(1).choice(200, 37, replace=False)), dtype=np.int32)
    torch = __import__("torch")
    M = to_dev(m, "bf16")
    X = gns_mod.dion3_gather_feedback(M, torch.from_numpy(S).cuda(), 0.95)
    assert np.array_equal(bits(X), m[S])
    assert np.array_equal(bits(M), error_feedback(m, S, 0.95))


@pytest.mark.parametrize("wd", [0.0, 0.1])
@pytest.mark.parametrize("o_dt", ["bf16", "f32"])
def test_apply_update_bit_exact(gns_mod, wd, o_dt):
    announce(f"dion3 apply_update wd={wd} O={o_dt}")
    w, _, _ = synth.dion3_state(n=160, m=768, seed=13)
    rng = np.random.default_rng(2)
    S = np.array(sorted(rng.choice(160, 40, replace=False)), dtype=np.int32)
    o_st = synth.to_storage(rng.standard_normal((40, 768)) * 0.01, o_dt)
    o = synth.bf16_bits_to_f32(o_st).astype(np.float64) if o_dt == "bf16" else o_st.astype(np.float64)
    torch = __import__("torch")
    W = to_dev(w, "bf16")
    gns_mod.dion3_apply_update(W, torch.from_numpy(S).cuda(), to_dev(o_st, o_dt), 0.02, wd)
    assert np.array_equal(bits(W), weight_update(w, S, o, 0.02, wd))


@pytest.mark.parametrize("norm", [1, 2])
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_small(gns_mod, norm, wd):
    announce(f"dion3 step 512x2048 norm={norm} wd={wd}")
    w, g, m = synth.dion3_state(n=512, m=2048, seed=14)
    k = k_from_fraction(0.25, 512)
    lr = 0.01 / np.sqrt(0.25)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, k, lr, wd=wd, mu=0.95, norm="l1" if norm == 1 else "l2")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2
    wg = bits(W)
    assert w_within_bound(wg, w_ref, lr, O_ref)
    rest = np.setdiff1d(np.arange(512), S_ref)
    assert np.array_equal(wg[rest], w_ref[rest])     # unselected rows do not depend on O


def test_dion3_step_repeatable(gns_mod):
    """The same step from the same state gives the same bits (S, O, W, M), ten times."""
    announce("dion3 step repeatable 1024x4096")
    w, g, m = synth.dion3_state(n=1024, m=4096, seed=15)
    k = k_from_fraction(0.25, 1024)
    runs = []
    for _ in range(10):
        W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
        S, O = gns_mod.dion3_step(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
        runs.append((S.cpu().numpy(), bits(O), bits(W), bits(M)))
    for r in runs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(r, runs[0]))


@pytest.fixture(scope="module")
def dion3_full():
    """The 8192 x 28672 workload's seeded state, the oracle's accumulated momentum and
    its row scores (l1 and l2), computed once for the module."""
    announce("dion3 8192x28672: generating inputs")
    w, g, m = synth.dion3_state()
    announce("dion3 8192x28672: oracle accumulate")
    m1 = accumulate(m, g)
    announce("dion3 8192x28672: oracle row scores")
    return {"w": w, "g": g, "m": m, "m1": m1, "l2": row_scores(m1, "l2"), "l1": row_scores(m1, "l1")}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("f,norm", [(0.25, 2), (0.125, 2), (0.25, 1)])
def test_dion3_step_full_size(gns_mod, dion3_full, f, norm):
    """The 8192 x 28672 workload at f = 1/4 and 1/8 with l2 row scores (the configured
    score) and at f = 1/4 with the pages' l1 score: S, M and the unselected W rows
    bit-exact; O within 2e-2 of float64 standard NS on the oracle's selected rows;
    the selected W rows within one bf16 rounding plus lr times O's tolerance of the
    oracle's update."""
    d = dion3_full
    w, g, m, m1 = d["w"], d["g"], d["m"], d["m1"]
    k = k_from_fraction(f, 8192)
    lr = 0.01 / np.sqrt(f)
    announce(f"dion3 step 8192x28672 f={f} norm=l{norm}")
    S_ref = select_topk(d["l2" if norm == 2 else "l1"], k)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=norm, return_O=True)
    assert np.array_equal(S.cpu().numpy(), S_ref)
    announce(f"dion3 8192x28672 f={f}: comparing M and the unselected W rows")
    assert np.array_equal(bits(M), error_feedback(m1, S_ref, 0.95))
    wg = bits(W)
    rest = np.setdiff1d(np.arange(8192), S_ref)
    assert np.array_equal(wg[rest], w[rest])
    announce(f"dion3 8192x28672 f={f}: oracle Newton-Schulz on the {k} selected rows")
    O_ref = newton_schulz(bf16_to_f64(m1[S_ref]))
    e = rel_fro(to_f64(O), O_ref)
    print(f"f={f} l{norm} O rel err {e:.3e}")
    assert e <= 2e-2
    announce(f"dion3 8192x28672 f={f}: selected W rows against the oracle's update")
    w_ref_sel = weight_update(w[S_ref], np.arange(k), bf16_to_f64(f64_to_bf16_rne(O_ref)), lr, 0.0)
    assert w_within_bound(wg[S_ref], w_ref_sel, lr, O_ref)
    if f == 0.25 and norm == 2:
        announce("dion3 8192x28672 f=0.25: the same step with the rows read in place")
        W2, M2, G2 = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
        S2, O2 = gns_mod.dion3_step(W2, M2, G2, k, lr, weight_decay=0.0, mu=0.95, score_norm=norm, return_O=True,
                                    schedule=gns_mod.default_schedule(rows_in_place=True))
        assert np.array_equal(S2.cpu().numpy(), S_ref)
        assert np.array_equal(bits(O2), bits(O)) and np.array_equal(bits(W2), wg)
        assert np.array_equal(bits(M2), bits(M))


@pytest.mark.parametrize("N,m,f,norm,wd", [(1000, 2048, 0.125, 2, 0.0), (1000, 2048, 0.125, 1, 0.1),
                                           (200, 520, 0.3, 2, 0.1)])
def test_dion3_step_any_k(gns_mod, N, m, f, norm, wd):
    """k = ceil(f N) that is not a multiple of 8 (k = 125 and 60): the submatrix is
    padded with zero rows inside the library.  S and M bit-exact, O within 2e-2, W
    within O's tolerance and bit-exact on unselected rows when wd = 0."""
    k = k_from_fraction(f, N)
    assert k % 8 != 0
    announce(f"dion3 step {N}x{m} f={f} (k={k}) norm={norm} wd={wd}")
    w, g, mo = synth.dion3_state(n=N, m=m, seed=38)
    lr = 0.01 / np.sqrt(f)
    W, M, G = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, mo, g, k, lr, wd=wd, mu=0.95, norm="l1" if norm == 1 else "l2")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    e = rel_fro(to_f64(O), O_ref)
    print(f"O rel err {e:.3e}")
    assert e <= 2e-2
    wg = bits(W)
    assert w_within_bound(wg, w_ref, lr, O_ref)
    if wd == 0.0:
        rest = np.setdiff1d(np.arange(N), S_ref)
        assert np.array_equal(wg[rest], w_ref[rest])
    # the same step without O_out takes the same path through the workspace
    W2, M2, G2 = to_dev(w, "bf16"), to_dev(mo, "bf16"), to_dev(g, "bf16")
    S2 = gns_mod.dion3_step(W2, M2, G2, k, lr, weight_decay=wd, mu=0.95, score_norm=norm)
    assert np.array_equal(S2.cpu().numpy(), S_ref)
    assert np.array_equal(bits(W2), wg) and np.array_equal(bits(M2), bits(M))


@pytest.mark.timeout(600)
def test_dion3_step_batched_long_k_equals_single(gns_mod):
    """Two 1024 x 16384 states at k = 1024: the submatrices' Gram products have
    K = 16384 and split K.  The batched step equals the single steps bitwise (the split
    does not depend on the batch size), and entry 0 matches the oracle."""
    import torch
    announce("dion3 step batched 2x1024x16384 k=1024 (long K)")
    B, N, m, k, lr = 2, 1024, 16384, 1024, 0.02
    states = [synth.dion3_state(n=N, m=m, seed=80 + b) for b in range(B)]
    stack = lambda i: torch.stack([to_dev(st[i], "bf16") for st in states])
    W, G, M = stack(0), stack(1), stack(2)
    S, O = gns_mod.dion3_step_batched(W, M, G, k, lr, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
    for b, (w, g, mm) in enumerate(states):
        W1, M1, G1 = to_dev(w, "bf16"), to_dev(mm, "bf16"), to_dev(g, "bf16")
        S1, O1 = gns_mod.dion3_step(W1, M1, G1, k, lr, weight_decay=0.1, mu=0.95, score_norm=2, return_O=True)
        assert np.array_equal(S1.cpu().numpy(), S[b].cpu().numpy())
        assert np.array_equal(bits(O1), bits(O[b]))
        assert np.array_equal(bits(W1), bits(W[b])) and np.array_equal(bits(M1), bits(M[b]))
    announce("dion3 step batched 2x1024x16384: oracle on entry 0")
    w, g, mm = states[0]
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, mm, g, k, lr, wd=0.1, mu=0.95, norm="l2")
    assert np.array_equal(S[0].cpu().numpy(), S_ref)
    assert np.array_equal(bits(M[0]), m_ref)
    e = rel_fro(to_f64(O[0]), O_ref)
    print(f"O rel err {e:.3e}")
    assert e <= 2e-2


def test_dion3_step_tall_submatrix(gns_mod):
    """k > m: the gathered k x m rows form a tall matrix, orthogonalised through its
    transpose (the iteration runs on the short side)."""
    announce("dion3 step 1024x256 k=512 (tall submatrix)")
    w, g, m = synth.dion3_state(n=1024, m=256, seed=16)
    k, lr = 512, 0.02
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=1, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, k, lr, wd=0.0, mu=0.95, norm="l1")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    e = rel_fro(to_f64(O), O_ref)
    print(f"tall O rel err {e:.3e}")
    assert e <= 2e-2
    assert w_within_bound(bits(W), w_ref, lr, O_ref)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_batched_matches_oracle_and_single(gns_mod, wd):
    """A batch of 3 same-shape states: per entry S and M bit-exact against the oracle,
    O within 2e-2, W within the bound of the single test; and every entry bitwise equal
    to dion3_step on that entry alone (batching changes no arithmetic)."""
    import torch
    announce(f"dion3 step batched 3x512x1024 wd={wd}")
    B, N, m, k, lr = 3, 512, 1024, 128, 0.02
    states = [synth.dion3_state(n=N, m=m, seed=60 + b) for b in range(B)]
    stack = lambda i: torch.stack([to_dev(st[i], "bf16") for st in states])
    W, G, M = stack(0), stack(1), stack(2)
    S, O = gns_mod.dion3_step_batched(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=2, return_O=True)
    Sb, Ob, Wb, Mb = S.cpu().numpy(), bits(O.reshape(B * k, m)), bits(W.reshape(B * N, m)), bits(M.reshape(B * N, m))
    for b, (w, g, mm) in enumerate(states):
        w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, mm, g, k, lr, wd=wd, mu=0.95, norm="l2")
        assert np.array_equal(Sb[b], S_ref)
        assert np.array_equal(Mb[b * N:(b + 1) * N], m_ref)
        assert rel_fro(to_f64(O[b]), O_ref) <= 2e-2
        assert w_within_bound(Wb[b * N:(b + 1) * N], w_ref, lr, O_ref)
        W1, M1, G1 = to_dev(w, "bf16"), to_dev(mm, "bf16"), to_dev(g, "bf16")
        S1, O1 = gns_mod.dion3_step(W1, M1, G1, k, lr, weight_decay=wd, mu=0.95, score_norm=2, return_O=True)
        assert np.array_equal(S1.cpu().numpy(), Sb[b])
        assert np.array_equal(bits(O1), Ob[b * k:(b + 1) * k])
        assert np.array_equal(bits(W1), Wb[b * N:(b + 1) * N])
        assert np.array_equal(bits(M1), Mb[b * N:(b + 1) * N])


def _rows_tensor(S_np):
    torch = __import__("torch")
    return torch.from_numpy(np.asarray(S_np, dtype=np.int32)).cuda()


def _bf16_empty(k, m):
    torch = __import__("torch")
    return torch.empty((k, m), dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_rows_random_set(gns_mod, wd):
    """A step on a random row set (the pages' alternative to top-k): M bit-exact, O
    within 2e-2, W within O's tolerance and bit-exact on unselected rows."""
    announce(f"dion3 step on a random row set 512x2048 wd={wd}")
    w, g, m = synth.dion3_state(n=512, m=2048, seed=17)
    S_np = np.sort(np.random.default_rng(18).choice(512, size=128, replace=False))
    lr = 0.02
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    O = gns_mod.dion3_step_rows(W, M, G, _rows_tensor(S_np), lr, weight_decay=wd, mu=0.95, O=_bf16_empty(128, 2048))
    w_ref, m_ref, O_ref = oracle.dion3_step_rows(w, m, g, S_np, lr, wd=wd, mu=0.95)
    assert np.array_equal(bits(M), m_ref)
    e = rel_fro(to_f64(O), O_ref)
    print(f"O rel err {e:.3e}")
    assert e <= 2e-2
    wg = bits(W)
    assert w_within_bound(wg, w_ref, lr, O_ref)
    rest = np.setdiff1d(np.arange(512), S_np)
    assert np.array_equal(wg[rest], w_ref[rest])


def test_dion3_step_rows_on_topk_set_is_dion3_step(gns_mod):
    """Given the set dion3_step picks, the caller-set step gives bitwise the same W, M, O."""
    announce("dion3 step_rows on the top-k set 1024x4096")
    w, g, m = synth.dion3_state(n=1024, m=4096, seed=19)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, 256, 0.02, weight_decay=0.1, mu=0.95, score_norm=1, return_O=True)
    W2, M2, G2 = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    O2 = gns_mod.dion3_step_rows(W2, M2, G2, S, 0.02, weight_decay=0.1, mu=0.95, O=_bf16_empty(256, 4096))
    assert np.array_equal(bits(O), bits(O2))
    assert np.array_equal(bits(W), bits(W2)) and np.array_equal(bits(M), bits(M2))


def test_dion3_step_rows_index_out_of_range_is_a_zero_row(gns_mod):
    """An index outside [0, N) reads as a zero row and updates nothing, so the step
    equals the oracle's step on the valid indices (a zero row of X stays zero under
    the iteration and does not change the Frobenius norm)."""
    announce("dion3 step_rows with an out-of-range index 256x1024")
    w, g, m = synth.dion3_state(n=256, m=1024, seed=20)
    valid = np.sort(np.random.default_rng(21).choice(256, size=15, replace=False))
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    O = gns_mod.dion3_step_rows(W, M, G, _rows_tensor(np.append(valid, 256)), 0.02, mu=0.95, O=_bf16_empty(16, 1024))
    w_ref, m_ref, O_ref = oracle.dion3_step_rows(w, m, g, valid, 0.02, wd=0.0, mu=0.95)
    assert np.array_equal(bits(M), m_ref)
    o = to_f64(O)
    assert np.all(o[15] == 0)
    assert rel_fro(o[:15], O_ref) <= 2e-2
    rest = np.setdiff1d(np.arange(256), valid)
    assert np.array_equal(bits(W)[rest], w[rest])


@pytest.mark.timeout(600)
def test_dion3_step_rows_full_size_random_set(gns_mod):
    """The 8192 x 28672 state with 2048 random rows (f = 1/4): M bit-exact against the
    oracle's accumulate + error feedback, unselected W rows untouched."""
    announce("dion3 step_rows 8192x28672 random k=2048: generating inputs")
    w, g, m = synth.dion3_state()
    S_np = np.sort(np.random.default_rng(26).choice(8192, size=2048, replace=False))
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    announce("dion3 step_rows 8192x28672: GPU step")
    gns_mod.dion3_step_rows(W, M, G, _rows_tensor(S_np), 0.02, mu=0.95)
    announce("dion3 step_rows 8192x28672: oracle accumulate + error feedback")
    assert np.array_equal(bits(M), error_feedback(accumulate(m, g), S_np, 0.95))
    rest = np.setdiff1d(np.arange(8192), S_np)
    assert np.array_equal(bits(W)[rest], w[rest])


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_dion3_step_dev_scalars_equals_host_scalars(gns_mod, wd):
    """lr, weight decay and mu read from device memory give bitwise the step with the
    same host values (S, O, W, M)."""
    announce(f"dion3 step with device scalars 512x2048 wd={wd}")
    torch = __import__("torch")
    w, g, m = synth.dion3_state(n=512, m=2048, seed=27)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, 128, 0.02, weight_decay=wd, mu=0.9, score_norm=2, return_O=True)
    W2, M2, G2 = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    sc = torch.tensor([0.02, wd, 0.9], dtype=torch.float32, device="cuda")
    S2, O2 = gns_mod.dion3_step_dev_scalars(W2, M2, G2, 128, sc, score_norm=2, O=_bf16_empty(128, 2048))
    assert np.array_equal(S.cpu().numpy(), S2.cpu().numpy())
    assert np.array_equal(bits(O), bits(O2))
    assert np.array_equal(bits(W), bits(W2)) and np.array_equal(bits(M), bits(M2))


@pytest.mark.parametrize("N,cols,k,norm,wd", [(512, 256, 64, 1, 0.0), (512, 256, 64, 2, 0.1),
                                              (200, 136, 24, 2, 0.0), (200, 136, 24, 1, 0.1),
                                              (200, 136, 35, 2, 0.0)])
def test_dion3_step_cols_matches_oracle(gns_mod, N, cols, k, norm, wd):
    """Column selection on a tall state, also with ragged tiles (N, k not multiples of
    64) and a k that is not a multiple of 8 (35): S and M bit-exact, O within 2e-2, W within O's tolerance (bit-exact on
    unselected columns when wd = 0)."""
    announce(f"dion3 column step {N}x{cols} k={k} norm={norm} wd={wd}")
    w, g, m = synth.dion3_state(n=N, m=cols, seed=32)
    lr = 0.02
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step_cols(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step_cols(w, m, g, k, lr, wd=wd, mu=0.95,
                                                        norm="l1" if norm == 1 else "l2")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    e = rel_fro(to_f64(O), O_ref)
    print(f"O rel err {e:.3e}")
    assert e <= 2e-2
    wg = bits(W)
    assert w_within_bound(wg, w_ref, lr, O_ref)
    if wd == 0.0:
        rest = np.setdiff1d(np.arange(cols), S_ref)
        assert np.array_equal(wg[:, rest], w_ref[:, rest])


@pytest.mark.timeout(900)
def test_dion3_step_cols_full_size_tall(gns_mod):
    """The 8192 x 28672 workload's transpose (a tall 28672 x 8192 state) with 2048
    columns (f = 1/4, l2): S and M bit-exact, unselected W columns untouched."""
    announce("dion3 column step 28672x8192 k=2048: generating inputs")
    w, g, m = synth.dion3_state(n=28672, m=8192, seed=33)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    announce("dion3 column step 28672x8192: GPU step")
    S = gns_mod.dion3_step_cols(W, M, G, 2048, 0.02, mu=0.95, score_norm=2).cpu().numpy()
    announce("dion3 column step 28672x8192: oracle accumulate and column scores")
    m1 = accumulate(m, g)
    S_ref = select_topk(row_scores(np.ascontiguousarray(m1.T), "l2"), 2048)
    assert np.array_equal(S, S_ref)
    announce("dion3 column step 28672x8192: comparing M and W")
    m_ref = np.ascontiguousarray(error_feedback(np.ascontiguousarray(m1.T), S_ref, 0.95).T)
    assert np.array_equal(bits(M), m_ref)
    rest = np.setdiff1d(np.arange(8192), S_ref)
    assert np.array_equal(bits(W)[:, rest], w[:, rest])


# ---- degenerate cases of the step ----

def test_dion3_step_all_rows_is_muon_step(gns_mod):
    """k = N (f = 1): every row is selected, so the step is Muon's on M + G."""
    announce("dion3 step k = N 256x1024")
    w, g, m = synth.dion3_state(n=256, m=1024, seed=34)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, 256, 0.01, weight_decay=0.0, mu=0.9, score_norm=1, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, 256, 0.01, wd=0.0, mu=0.9, norm="l1")
    assert np.array_equal(S.cpu().numpy(), np.arange(256))
    assert np.array_equal(bits(M), m_ref)
    assert rel_fro(to_f64(O), newton_schulz(bf16_to_f64(accumulate(m, g)))) <= 2e-2
    assert w_within_bound(bits(W), w_ref, 0.01, O_ref)


def test_dion3_step_tied_scores_pick_lower_rows(gns_mod):
    """Rows repeated three times tie exactly in score, and k = 40 splits one group of
    tied rows: the lower index wins, as in the oracle, and the whole step matches it."""
    announce("dion3 step with tied rows 256x512")
    w, g, m = synth.dion3_state(n=256, m=512, seed=35)
    m = np.ascontiguousarray(np.repeat(m[:86], 3, axis=0)[:256])     # rows 3i .. 3i+2 identical
    g = np.ascontiguousarray(np.repeat(g[:86], 3, axis=0)[:256])
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, 40, 0.02, weight_decay=0.0, mu=0.95, score_norm=2, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, 40, 0.02, wd=0.0, mu=0.95, norm="l2")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2


def test_dion3_step_zero_state(gns_mod):
    """M = G = 0: every score ties at zero, the first k rows are selected, X = 0 gives
    O = 0, so W keeps its bits (wd = 0) and M stays zero."""
    announce("dion3 step on a zero state 128x256")
    w, _, _ = synth.dion3_state(n=128, m=256, seed=36)
    z = np.zeros((128, 256), dtype=np.uint16)
    W, M, G = to_dev(w, "bf16"), to_dev(z, "bf16"), to_dev(z, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, 32, 0.02, weight_decay=0.0, mu=0.95, score_norm=1, return_O=True)
    assert np.array_equal(S.cpu().numpy(), np.arange(32))
    assert not np.any(bits(O) & 0x7fff)                   # +0 or -0 everywhere
    assert np.array_equal(bits(W), w)
    assert not np.any(bits(M) & 0x7fff)


@pytest.mark.parametrize("k", [1, 8])
def test_dion3_step_smallest_k(gns_mod, k):
    """k = 1 (a single row, padded to 8 inside the library) and k = 8."""
    announce(f"dion3 step k = {k} 512x1024")
    w, g, m = synth.dion3_state(n=512, m=1024, seed=37)
    W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
    S, O = gns_mod.dion3_step(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=1, return_O=True)
    w_ref, m_ref, S_ref, O_ref = oracle.dion3_step(w, m, g, k, 0.02, wd=0.1, mu=0.95, norm="l1")
    assert np.array_equal(S.cpu().numpy(), S_ref)
    assert np.array_equal(bits(M), m_ref)
    assert rel_fro(to_f64(O), O_ref) <= 2e-2
    assert w_within_bound(bits(W), w_ref, 0.02, O_ref)


# ---- the selected rows read in place (no gathered copy of M[S, :]) ----

def _step_bits(gns_mod, w, g, m, k, lr, wd, norm, compute, in_place, batched=False, S_rows=None, dev=False):
    import torch
    sched = gns_mod.default_schedule(rows_in_place=in_place)
    if batched:
        stack = lambda a: torch.stack([to_dev(x, "bf16") for x in a])
        W, M, G = stack(w), stack(m), stack(g)
        S, O = gns_mod.dion3_step_batched(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm,
                                          compute=compute, schedule=sched, return_O=True)
    else:
        W, M, G = to_dev(w, "bf16"), to_dev(m, "bf16"), to_dev(g, "bf16")
        if S_rows is not None:
            O = gns_mod.dion3_step_rows(W, M, G, _rows_tensor(S_rows), lr, weight_decay=wd, mu=0.95, compute=compute,
                                        schedule=sched, O=_bf16_empty(len(S_rows), w.shape[1]))
            S = _rows_tensor(S_rows)
        elif dev:
            sc = torch.tensor([lr, wd, 0.95], dtype=torch.float32, device="cuda")
            S, O = gns_mod.dion3_step_dev_scalars(W, M, G, k, sc, score_norm=norm, compute=compute, schedule=sched,
                                                  O=_bf16_empty(k, w.shape[1]))
        else:
            S, O = gns_mod.dion3_step(W, M, G, k, lr, weight_decay=wd, mu=0.95, score_norm=norm, compute=compute,
                                      schedule=sched, return_O=True)
    torch.cuda.synchronize()
    return S.cpu().numpy(), bits(O), bits(W), bits(M)


@pytest.mark.parametrize("case", ["small_wd", "k125_bf16", "long_k_split", "batched", "caller_rows", "dev_scalars",
                                  "k2047_half_copy"])
def test_dion3_rows_in_place_bitwise_equal(gns_mod, case):
    """rows_in_place = 1 (the Gram products read M[S, :] through the row list, the
    error feedback runs with the update) gives bitwise the step of the default path
    (rows gathered into a copy first): S, O, W and M."""
    announce(f"dion3 rows in place: {case}")
    kw = dict(k=128, lr=0.02, wd=0.1, norm=2, compute="f16")
    if case == "small_wd":
        w, g, m = synth.dion3_state(n=512, m=2048, seed=90)
    elif case == "k125_bf16":
        w, g, m = synth.dion3_state(n=1000, m=2048, seed=91)
        kw.update(k=125, wd=0.0, norm=1, compute="bf16")
    elif case == "long_k_split":
        w, g, m = synth.dion3_state(n=1024, m=16384, seed=92)
        kw.update(k=1024)
    elif case == "batched":
        sts = [synth.dion3_state(n=512, m=2048, seed=93 + b) for b in range(2)]
        w, g, m = ([st[i] for st in sts] for i in range(3))
    elif case == "k2047_half_copy":
        # 2048 padded rows: the gathered path also writes the fp16 copy that the restart
        # and final products read; reading the rows in place converts them on load
        w, g, m = synth.dion3_state(n=4096, m=4096, seed=98)
        kw.update(k=2047)
    elif case == "caller_rows":
        w, g, m = synth.dion3_state(n=256, m=1024, seed=95)
        rows = np.append(np.sort(np.random.default_rng(96).choice(256, size=23, replace=False)), 256)
        kw.update(k=24, S_rows=rows)
    else:
        w, g, m = synth.dion3_state(n=512, m=2048, seed=97)
        kw.update(dev=True)
    extra = {x: kw.pop(x) for x in ("S_rows", "dev") if x in kw}
    a = _step_bits(gns_mod, w, g, m, batched=case == "batched", in_place=False, **kw, **extra)
    b = _step_bits(gns_mod, w, g, m, batched=case == "batched", in_place=True, **kw, **extra)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
