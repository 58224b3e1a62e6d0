"""Out-of-bounds writes and resumable state.

Guard bands: every output of the library is placed inside a larger buffer whose other
bytes (a band before and after it, and the padding columns of rows longer than the
matrix) hold a sentinel pattern; after the call the sentinel bytes must be unchanged,
and so must every input the call only reads.  Shapes are ragged against the tiles
(edge tiles, partial diagonal tiles, padded Dion3 submatrices).

Resume: a stateful step sequence (Dion3, Muon) run as 3 steps equals 2 steps, a round
trip of the state through host memory (as a checkpoint would take it), and 1 more
step, bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import announce

pytestmark = pytest.mark.gpu

GUARD = 4096                       # elements of sentinel before and after each matrix


def raw(x):
    return x.detach().cpu().contiguous().view(torch.uint8).numpy().copy()


def guarded(rows, cols, ld, dtype, fill=None, seed=0):
    """A [rows, cols] view (row stride ld) into a flat buffer with GUARD sentinel
    elements on both sides; the padding columns hold the sentinel too.  fill: values
    for the matrix (float64 array) or None (left as sentinel)."""
    n_el = GUARD + rows * ld + GUARD
    flat = torch.empty(n_el, dtype=dtype, device="cuda")
    bits = flat.view(torch.int16 if dtype != torch.float32 else torch.int32)
    bits.fill_(-23131 if dtype != torch.float32 else -1515870811)        # 0xA5A5 / 0xA5A5A5A5
    view = flat[GUARD:GUARD + rows * ld].view(rows, ld)[:, :cols]
    if fill is not None:
        view.copy_(torch.from_numpy(np.asarray(fill, dtype=np.float64)).to(dtype))
    return flat, view


def sentinel_intact(flat, rows, cols, ld, before):
    """True when every byte of flat outside the [rows, cols] matrix equals `before`."""
    es = flat.element_size()
    now = raw(flat)
    mask = np.ones(flat.numel(), dtype=bool)
    idx = GUARD + (np.arange(rows)[:, None] * ld + np.arange(cols)[None, :]).ravel()
    mask[idx] = False
    mb = np.repeat(mask, es)
    return np.array_equal(now[mb], before[mb])


def rnd(rows, cols, seed, scale=0.02):
    return np.random.default_rng(seed).standard_normal((rows, cols)) * scale


@pytest.mark.parametrize("fn", ["orthogonalize", "newton_schulz"])
@pytest.mark.parametrize("n, m", [(200, 328), (328, 200), (64, 64)])
def test_orthogonalize_writes_only_its_output(gns_mod, fn, n, m):
    announce(f"guards {fn} {n}x{m}")
    ldx, ldo = m + 24, m + 40
    xf, X = guarded(n, m, ldx, torch.bfloat16, rnd(n, m, 1, 1.0))
    of, O = guarded(n, m, ldo, torch.bfloat16)
    x_before, o_before = raw(xf), raw(of)
    getattr(gns_mod, fn)(X, out=O)
    torch.cuda.synchronize()
    assert np.array_equal(raw(xf), x_before)                  # the input is only read
    assert sentinel_intact(of, n, m, ldo, o_before)
    assert torch.isfinite(O.float()).all()


@pytest.mark.parametrize("n, k", [(72, 200), (264, 136), (520, 64)])
def test_symm_gemm_writes_only_its_output(gns_mod, n, k):
    announce(f"guards symm_gemm n={n} k={k}")
    af, A = guarded(n, k, k + 8, torch.float16, rnd(n, k, 2, 0.1))
    bf, B = guarded(n, k, k + 16, torch.float16, rnd(n, k, 3, 0.1))
    cf, C = guarded(n, n, n + 8, torch.float16, rnd(n, n, 4, 0.1))
    df, D = guarded(n, n, n + 24, torch.float16)
    before = [raw(t) for t in (af, bf, cf, df)]
    gns_mod.symm_gemm(A, B, C=C, alpha=1.5, beta=-0.5, gamma=0.25, out=D)
    torch.cuda.synchronize()
    for t, b in zip((af, bf, cf), before[:3]):
        assert np.array_equal(raw(t), b)
    assert sentinel_intact(df, n, n, n + 24, before[3])


@pytest.mark.parametrize("n, k, m", [(72, 72, 200), (264, 264, 1032), (136, 136, 8)])
def test_rect_gemm_writes_only_its_output(gns_mod, n, k, m):
    announce(f"guards rect_gemm {n}x{k}x{m}")
    af, A = guarded(n, k, k + 8, torch.float16, rnd(n, k, 5, 0.1))
    bf, B = guarded(k, m, m + 8, torch.float16, rnd(k, m, 6, 0.1))
    cf, C = guarded(n, m, m + 16, torch.float16, rnd(n, m, 7, 0.1))
    df, D = guarded(n, m, m + 32, torch.float16)
    before = [raw(t) for t in (af, bf, cf, df)]
    gns_mod.rect_gemm(A, B, C=C, alpha=2.0, beta=0.5, out=D)
    torch.cuda.synchronize()
    for t, b in zip((af, bf, cf), before[:3]):
        assert np.array_equal(raw(t), b)
    assert sentinel_intact(df, n, m, m + 32, before[3])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N, m, k", [(200, 328, 37), (96, 64, 72)])
def test_dion3_step_writes_only_its_state_and_outputs(gns_mod, dt, N, m, k):
    announce(f"guards dion3_step {dt} N={N} m={m} k={k}")
    ld = m + 16
    wf, W = guarded(N, m, ld, dt, rnd(N, m, 8))
    mf, M = guarded(N, m, ld, dt, rnd(N, m, 9))
    gf, G = guarded(N, m, ld, dt, rnd(N, m, 10))
    of, O = guarded(k, m, m, dt)
    sflat = torch.full((GUARD + k + GUARD,), -7, dtype=torch.int32, device="cuda")
    S = sflat[GUARD:GUARD + k]
    before = [raw(t) for t in (wf, mf, gf, of, sflat)]
    gns_mod.dion3_step(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, S=S, O=O)
    torch.cuda.synchronize()
    assert np.array_equal(raw(gf), before[2])
    for t, rows, cols, ldd, b in ((wf, N, m, ld, before[0]), (mf, N, m, ld, before[1]), (of, k, m, m, before[3])):
        assert sentinel_intact(t, rows, cols, ldd, b)
    s_now = sflat.cpu().numpy()
    assert (s_now[:GUARD] == -7).all() and (s_now[GUARD + k:] == -7).all()
    s = s_now[GUARD:GUARD + k]
    assert (np.diff(s) > 0).all() and s[0] >= 0 and s[-1] < N


def test_dion3_step_cols_writes_only_its_state_and_outputs(gns_mod):
    announce("guards dion3_step_cols 264x200 k=37")
    N, m, k, ld = 264, 200, 37, 216
    wf, W = guarded(N, m, ld, torch.bfloat16, rnd(N, m, 11))
    mf, M = guarded(N, m, ld, torch.bfloat16, rnd(N, m, 12))
    gf, G = guarded(N, m, ld, torch.bfloat16, rnd(N, m, 13))
    of, O = guarded(k, N, N, torch.bfloat16)
    before = [raw(t) for t in (wf, mf, gf, of)]
    gns_mod.dion3_step_cols(W, M, G, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=2, O=O)
    torch.cuda.synchronize()
    assert np.array_equal(raw(gf), before[2])
    for t, rows, cols, ldd, b in ((wf, N, m, ld, before[0]), (mf, N, m, ld, before[1]), (of, k, N, N, before[3])):
        assert sentinel_intact(t, rows, cols, ldd, b)


def _roundtrip(*ts):
    """The state as a checkpoint takes it: copied to host memory, the device tensors
    dropped, and fresh device tensors made from the host copies."""
    host = [t.detach().cpu().clone() for t in ts]
    del ts
    torch.cuda.synchronize()
    return [h.to("cuda") for h in host]


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_dion3_resume_is_bitwise(gns_mod, dt):
    announce(f"resume dion3 {dt}")
    N, m, k = 256, 768, 64
    w0, m0 = (torch.from_numpy(rnd(N, m, s)).to(dt).cuda() for s in (20, 21))
    grads = [torch.from_numpy(rnd(N, m, 30 + i)).to(dt).cuda() for i in range(3)]
    W, M = w0.clone(), m0.clone()
    for g in grads:
        gns_mod.dion3_step(W, M, g, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=1)
    W2, M2 = w0.clone(), m0.clone()
    for g in grads[:2]:
        gns_mod.dion3_step(W2, M2, g, k, 0.02, weight_decay=0.1, mu=0.95, score_norm=1)
    W2, M2 = _roundtrip(W2, M2)
    gns_mod.dion3_step(W2, M2, grads[2], k, 0.02, weight_decay=0.1, mu=0.95, score_norm=1)
    assert np.array_equal(raw(W), raw(W2)) and np.array_equal(raw(M), raw(M2))


def test_muon_resume_is_bitwise(gns_mod):
    announce("resume muon")
    B, n, m = 2, 128, 384
    w0, m0 = (torch.from_numpy(np.stack([rnd(n, m, s + b) for b in range(B)])).to(torch.bfloat16).cuda()
              for s in (40, 50))
    grads = [torch.from_numpy(np.stack([rnd(n, m, 60 + 10 * i + b) for b in range(B)])).to(torch.bfloat16).cuda()
             for i in range(3)]
    W, M = w0.clone(), m0.clone()
    for g in grads:
        gns_mod.muon_step(W, M, g, 0.02, weight_decay=0.1)
    W2, M2 = w0.clone(), m0.clone()
    for g in grads[:2]:
        gns_mod.muon_step(W2, M2, g, 0.02, weight_decay=0.1)
    W2, M2 = _roundtrip(W2, M2)
    gns_mod.muon_step(W2, M2, grads[2], 0.02, weight_decay=0.1)
    assert np.array_equal(raw(W), raw(W2)) and np.array_equal(raw(M), raw(M2))
