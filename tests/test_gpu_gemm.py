"""GPU parity of the two MFMA GEMM kernels against the oracle's float64 definitions.

Shapes span several 128 x 128 output tiles and ragged tails (n, k, m not multiples
of the tile), every operand/output dtype combination the library accepts, the
alpha/beta/gamma epilogue, batching, and bitwise symmetry of the symmetric output.
Tolerances (relative Frobenius, and max-abs relative to max |ref|): the inputs are
exact in their stored dtype and products accumulate in fp32, so the error is the
final rounding to the output dtype plus fp32 accumulation:
  bf16 out 6e-3, f16 out 1e-3, f32 out 2e-5 (K <= 1024).
"""
import numpy as np
import pytest

import synth
from oracle import symm_gemm_ref, rect_gemm_ref
from gpu_helpers import to_dev, to_f64, rel_fro, announce

pytestmark = pytest.mark.gpu

TOL = {"bf16": 6e-3, "f16": 1e-3, "f32": 2e-5}


def stored(rng, shape, dt, scale=1.0):
    x = scale * rng.standard_normal(shape)
    st = synth.to_storage(x, dt)
    if dt == "bf16":
        return st, synth.bf16_bits_to_f32(st).astype(np.float64)
    return st, st.astype(np.float64)


def check(got, ref, tol):
    e = rel_fro(got, ref)
    mx = float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-300))
    assert e <= tol and mx <= 4 * tol, (e, mx)


@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "bf16"), ("bf16", "f16"), ("bf16", "f32"), ("f16", "f16"),
                                          ("f16", "f32"), ("f32", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("n,k", [(8, 8), (136, 72), (256, 512), (264, 200)])
def test_symm_gemm_parity(gns_mod, in_dt, out_dt, n, k):
    announce(f"symm_gemm {in_dt}->{out_dt} n={n} k={k}")
    rng = np.random.default_rng(n * 1000 + k)
    batch = 2
    a_st, a = stored(rng, (batch, n, k), in_dt)
    b_st, b = stored(rng, (batch, n, k), in_dt)
    c_st, c = stored(rng, (batch, n, n), out_dt)
    A, B, C = to_dev(a_st, in_dt), to_dev(b_st, in_dt), to_dev(c_st, out_dt)
    D = gns_mod.symm_gemm(A, B, C, alpha=0.75, beta=-0.5, gamma=1.25, out_dtype=out_dt)
    got = to_f64(D)
    ref = symm_gemm_ref(a, b, c, alpha=0.75, beta=-0.5, gamma=1.25)
    check(got, ref, TOL[out_dt])
    Dh = D.cpu()
    assert bool((Dh == Dh.transpose(1, 2)).all()), "output not bitwise symmetric"


@pytest.mark.parametrize("n,k,batch", [(2000, 200, 1), (2048, 136, 2)])
def test_symm_gemm_tri96_tiles(gns_mod, n, k, batch):
    """Lower-triangle products with n of about 2048 run on 96 x 96 tiles (ragged at
    n = 2000 and 2048: the last tile row holds 80 and 32 rows); the paired-size grid of
    two matrices takes two workgroups per CU."""
    announce(f"symm_gemm 96-tiles n={n} k={k} batch={batch}")
    rng = np.random.default_rng(n + k)
    a_st, a = stored(rng, (batch, n, k), "f16")
    b_st, b = stored(rng, (batch, n, k), "f16")
    c_st, c = stored(rng, (batch, n, n), "f16")
    A, B, C = to_dev(a_st, "f16"), to_dev(b_st, "f16"), to_dev(c_st, "f16")
    D = gns_mod.symm_gemm(A, B, C, alpha=0.75, beta=-0.5, gamma=1.25, out_dtype="f16")
    got = to_f64(D)
    ref = symm_gemm_ref(a, b, c, alpha=0.75, beta=-0.5, gamma=1.25)
    check(got, ref, TOL["f16"])
    Dh = D.cpu()
    assert bool((Dh == Dh.transpose(1, 2)).all()), "output not bitwise symmetric"


@pytest.mark.parametrize("in_dt", ["bf16", "f16", "f32"])
def test_syrk_same_operand(gns_mod, in_dt):
    announce(f"syrk {in_dt}")
    rng = np.random.default_rng(7)
    x_st, x = stored(rng, (3, 200, 776), in_dt, scale=0.05)
    X = to_dev(x_st, in_dt)
    D = gns_mod.symm_gemm(X, X, out_dtype="f32")
    check(to_f64(D), symm_gemm_ref(x, x), TOL["f32"])


@pytest.mark.parametrize("a_dt,b_dt,out_dt", [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"),
                                              ("f32", "f32", "f32"), ("f16", "bf16", "f32"),
                                              ("bf16", "f16", "bf16"), ("f16", "f16", "f32")])
@pytest.mark.parametrize("n,k,m", [(8, 8, 8), (136, 72, 200), (256, 256, 512), (120, 264, 1032)])
def test_rect_gemm_parity(gns_mod, a_dt, b_dt, out_dt, n, k, m):
    announce(f"rect_gemm {a_dt}x{b_dt}->{out_dt} n={n} k={k} m={m}")
    rng = np.random.default_rng(n + 7 * k + 13 * m)
    batch = 2
    a_st, a = stored(rng, (batch, n, k), a_dt)
    b_st, b = stored(rng, (batch, k, m), b_dt)
    c_st, c = stored(rng, (batch, n, m), out_dt)
    pre = 1.0 if a_dt == b_dt else 0.5
    D = gns_mod.rect_gemm(to_dev(a_st, a_dt), to_dev(b_st, b_dt), to_dev(c_st, out_dt), alpha=1.5, beta=0.25,
                          b_prescale=pre, out_dtype=out_dt)
    # with a dtype conversion the B operand is rounded to a_dt after the prescale
    if a_dt != b_dt:
        b = synth.to_storage(pre * b, a_dt)
        b = (synth.bf16_bits_to_f32(b) if a_dt == "bf16" else b).astype(np.float64)
    ref = rect_gemm_ref(a, b, c, alpha=1.5, beta=0.25)
    check(to_f64(D), ref, TOL[out_dt])


def test_frobenius_scale(gns_mod):
    announce("frobenius_scale")
    rng = np.random.default_rng(3)
    for dt in ("bf16", "f16", "f32"):
        x_st, x = stored(rng, (5, 40, 264), dt, scale=0.3)
        s = gns_mod.frobenius_scale(to_dev(x_st, dt), eps=1e-7).cpu().numpy()
        ref = 1.0 / (np.sqrt((x * x).sum(axis=(1, 2))) + 1e-7)
        assert np.allclose(s, ref, rtol=2e-6, atol=0)


# Large batches select the 256 x 256 and 128 x 128 tile configurations (the small
# shapes above run on 64 x 64 tiles); ragged sizes keep partial tiles in play.
@pytest.mark.parametrize("batch,n,k,expect", [(48, 776, 264, "256x256"), (12, 520, 136, "128x128")])
def test_symm_gemm_tile_configs(gns_mod, batch, n, k, expect):
    announce(f"symm_gemm batch={batch} n={n} k={k} ({expect})")
    rng = np.random.default_rng(batch + n)
    a_st, a = stored(rng, (batch, n, k), "f16")
    c_st, c = stored(rng, (batch, n, n), "f32")          # C is in the output dtype
    D = gns_mod.symm_gemm(to_dev(a_st, "f16"), to_dev(a_st, "f16"), to_dev(c_st, "f32"), alpha=0.5, beta=1.0,
                          gamma=-2.0, out_dtype="f32")
    for i in (0, batch // 2, batch - 1):
        check(to_f64(D[i]), symm_gemm_ref(a[i], a[i], c[i], alpha=0.5, beta=1.0, gamma=-2.0), TOL["f32"])
    Dh = D.cpu()
    assert bool((Dh == Dh.transpose(1, 2)).all())


@pytest.mark.parametrize("batch,n,k,m,expect", [(24, 776, 264, 1032, "256x256"), (8, 520, 136, 1032, "128x128")])
def test_rect_gemm_tile_configs(gns_mod, batch, n, k, m, expect):
    announce(f"rect_gemm batch={batch} n={n} k={k} m={m} ({expect})")
    rng = np.random.default_rng(batch + n + m)
    a_st, a = stored(rng, (batch, n, k), "f16")
    b_st, b = stored(rng, (batch, k, m), "bf16")
    D = gns_mod.rect_gemm(to_dev(a_st, "f16"), to_dev(b_st, "bf16"), alpha=2.0, b_prescale=0.25, out_dtype="f32")
    for i in (0, batch - 1):
        bc = synth.to_storage(0.25 * b[i], "f16").astype(np.float64)
        check(to_f64(D[i]), rect_gemm_ref(a[i], bc, alpha=2.0), TOL["f32"])


@pytest.mark.parametrize("out_dt", ["f16", "bf16"])
def test_epilogue_paths_agree_bitwise(gns_mod, out_dt):
    """The epilogue of the 64 x 64 tiles (C loaded before the k-loop, one fragment row
    per wave) and that of the 128 x 128 tiles (C loaded in the epilogue, two fragment
    rows) form the same values: the same matrices in a batch large enough for 128 x 128
    tiles give bitwise the same output, with C, beta and gamma (symmetric) and with C
    and beta (rectangular)."""
    import torch
    announce(f"epilogue paths {out_dt}")
    rng = np.random.default_rng(520)
    n, k, m = 520, 136, 1032
    a_st, a = stored(rng, (1, n, k), "f16")
    b_st, b = stored(rng, (1, n, k), "f16")
    c_st, c = stored(rng, (1, n, n), out_dt)
    r_st, r = stored(rng, (1, k, m), "f16")
    e_st, e = stored(rng, (1, n, m), out_dt)
    A, B, C = to_dev(a_st, "f16"), to_dev(b_st, "f16"), to_dev(c_st, out_dt)
    Rb, E = to_dev(r_st, "f16"), to_dev(e_st, out_dt)
    D = gns_mod.symm_gemm(A, B, C, alpha=0.75, beta=-0.5, gamma=1.25, out_dtype=out_dt)      # 45 tiles of 64
    check(to_f64(D[0]), symm_gemm_ref(a[0], b[0], c[0], alpha=0.75, beta=-0.5, gamma=1.25), TOL[out_dt])
    D18 = gns_mod.symm_gemm(A.repeat(18, 1, 1), B.repeat(18, 1, 1), C.repeat(18, 1, 1), alpha=0.75, beta=-0.5,
                            gamma=1.25, out_dtype=out_dt)                                    # 270 tiles of 128
    assert all(torch.equal(D18[i].view(torch.int16), D[0].view(torch.int16)) for i in (0, 17))
    Dh = D.cpu()
    assert bool((Dh == Dh.transpose(1, 2)).all())
    F = gns_mod.rect_gemm(A, Rb, E, alpha=1.5, beta=0.25, out_dtype=out_dt)                 # 9 x 17 tiles of 64
    check(to_f64(F[0]), rect_gemm_ref(a[0], r[0], e[0], alpha=1.5, beta=0.25), TOL[out_dt])
    F6 = gns_mod.rect_gemm(A.repeat(6, 1, 1), Rb.repeat(6, 1, 1), E.repeat(6, 1, 1), alpha=1.5, beta=0.25,
                           out_dtype=out_dt)                                                 # 6 x 45 tiles of 128
    assert all(torch.equal(F6[i].view(torch.int16), F[0].view(torch.int16)) for i in (0, 5))


def test_binding_rejects_operands_the_abi_cannot_check(gns_mod):
    """C in a dtype other than the output's (or a wrongly shaped output) is refused
    by the binding before any launch: the ABI only receives raw pointers."""
    import torch
    a = torch.zeros(2, 64, 64, dtype=torch.float16, device="cuda")
    c16 = torch.zeros(2, 64, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(TypeError):
        gns_mod.symm_gemm(a, a, C=c16, beta=1.0, out_dtype="f32")
    with pytest.raises(ValueError):
        gns_mod.symm_gemm(a, a, out=torch.empty(2, 64, 32, dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        gns_mod.rect_gemm(a, a, C=c16, beta=1.0, out_dtype="f32")


def test_symm_gemm_fp32_big_tiles(gns_mod):
    """fp32 operands on the 256 x 256 tile configuration (a batch with >= 256 such
    tiles), ragged n; the fp32 kernel shares the 8-wave tile layout."""
    announce("symm_gemm f32 batch=64 n=520 k=72 (256x256)")
    rng = np.random.default_rng(520)
    a_st, a = stored(rng, (64, 520, 72), "f32")
    c_st, c = stored(rng, (64, 520, 520), "f32")
    D = gns_mod.symm_gemm(to_dev(a_st, "f32"), to_dev(a_st, "f32"), to_dev(c_st, "f32"), alpha=1.5, beta=-1.0,
                          gamma=0.5, out_dtype="f32")
    for i in (0, 31, 63):
        check(to_f64(D[i]), symm_gemm_ref(a[i], a[i], c[i], alpha=1.5, beta=-1.0, gamma=0.5), TOL["f32"])
    Dh = D.cpu()
    assert bool((Dh == Dh.transpose(1, 2)).all())
