"""CPU-only checks of the boundary and host logic (no kernel is launched):

* libgns.so loads and exports every function include/gns.h declares;
* argument validation rejects bad calls before any launch (null pointers, short
  leading dimensions, misalignment, short workspace, bad schedule, unsupported dtype
  pairs);
* workspace-size queries;
* the FLOP formulas against the savings the Dion3 pages state (55% / 68% at T = 5,
  alpha = 4) and the restart cost 3 (alpha - 1) n^3.
"""
import ctypes
import json
import os

import pytest

import muon_gram_ns_amd as gns
from muon_gram_ns_amd import flops

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
L = gns.lib
BF16, F16, F32 = gns.GNS_BF16, gns.GNS_F16, gns.GNS_F32
OK, INVALID, UNSUP, WS = 0, -1, -2, -3

FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call here fails validation


def test_exports_every_declared_symbol():
    names = gns.header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    assert L.gns_status_string(0) == b"GNS_OK"
    assert L.gns_status_string(-3) == b"GNS_ERR_WORKSPACE"


def test_default_schedule_matches_pages():
    s = gns.default_schedule()
    a, b, c = GOLD["ns_coefficients"]["value"]
    assert s.steps == GOLD["ns_steps"]["value"]
    assert all(abs(s.a[t] - a) < 1e-6 and abs(s.b[t] - b) < 1e-6 and abs(s.c[t] - c) < 1e-6 for t in range(5))
    # restart before step 3 == after step 2
    assert s.restart_after_mask == 1 << (GOLD["restart_before_step"]["value"] - 1)
    assert abs(s.eps - GOLD["ns_eps"]["value"]) < 1e-12


def ortho(X=FAKE, xdt=BF16, ldx=256, sx=64 * 256, O=FAKE * 3, odt=BF16, ldo=256, so=64 * 256, B=1, n=64, m=256,
          cdt=F16, sched=None, ws=FAKE * 50, wsb=None, fn="gns_orthogonalize_batched"):
    if wsb is None:
        wsb = L.gns_workspace_size(B, n, m, cdt)
    return getattr(L, fn)(X, xdt, ldx, sx, O, odt, ldo, so, B, n, m, cdt,
                          ctypes.byref(sched) if sched else None, ws, wsb, None, None)


def test_validation_rejects_before_launch():
    # n > m is valid (the library runs on the transpose) but needs the larger workspace
    tall = L.gns_workspace_size(1, 512, 256, F16)
    assert tall > L.gns_workspace_size(1, 256, 512, F16)
    assert ortho(n=512, m=256, ldx=256, ldo=256, O=FAKE * 20, wsb=tall - 256) == WS
    assert ortho(n=512, m=256, ldx=128) == INVALID         # ld < m still checked
    assert ortho(X=None) == INVALID
    assert ortho(O=None) == INVALID
    assert ortho(ldx=128) == INVALID                       # ld < m
    assert ortho(n=60, m=256) == UNSUP                     # n not a multiple of 8
    assert ortho(X=FAKE + 2) == UNSUP                      # misaligned
    assert ortho(wsb=16) == WS
    assert ortho(ws=None) == WS
    assert ortho(xdt=F32, cdt=F16) == UNSUP                # fp32 input needs fp32 iterates
    assert ortho(xdt=BF16, cdt=F32) == UNSUP
    assert ortho(cdt=7) == INVALID
    assert ortho(O=FAKE) == INVALID                        # O aliases X
    bad = gns.default_schedule()
    bad.restart_after_mask = 1 << 5                        # restart after the last step
    assert ortho(sched=bad) == INVALID
    bad = gns.default_schedule()
    bad.steps = 0
    assert ortho(sched=bad) == INVALID
    for field in ("square_fallback", "rows_in_place"):   # flags are 0 or 1
        bad = gns.default_schedule()
        setattr(bad, field, 2)
        assert ortho(sched=bad) == INVALID
    assert ortho(fn="gns_newton_schulz_batched", n=512, m=256, ldx=128) == INVALID
    assert ortho(B=0) == OK                                # empty batch: nothing to do


def test_gemm_and_dion3_validation():
    # symm_gemm: k not a multiple of 8 for 16-bit operands
    assert L.symm_gemm(1, 64, 60, 1.0, FAKE, 64, 0, FAKE, 64, 0, 0.0, None, 64, 0, 0.0, FAKE * 2, 64, 0,
                       BF16, BF16, None) == UNSUP
    assert L.symm_gemm(1, 64, 64, 1.0, FAKE, 64, 0, None, 64, 0, 0.0, None, 64, 0, 0.0, FAKE * 2, 64, 0,
                       BF16, BF16, None) == INVALID
    # rect_gemm: unsupported dtype pair, prescale with equal dtypes
    assert L.rect_gemm(1, 64, 64, 64, 1.0, FAKE, 64, 0, F32, FAKE, 64, 0, BF16, 1.0, 0.0, None, 64, 0,
                       FAKE * 2, 64, 0, F32, None) == UNSUP
    assert L.rect_gemm(1, 64, 64, 64, 1.0, FAKE, 64, 0, BF16, FAKE, 64, 0, BF16, 2.0, 0.0, None, 64, 0,
                       FAKE * 2, 64, 0, BF16, None) == INVALID
    # dion3: k > N, bad norm, short workspace
    sched = gns.default_schedule()
    args = lambda k, norm=1, wsb=1 << 40, dt=BF16: (FAKE, FAKE * 2, FAKE * 3, dt, 64, 256, 256, k, 0.02, 0.0, 0.95,
                                                    norm, F16, ctypes.byref(sched), FAKE * 4, None, FAKE * 5, wsb,
                                                    None)
    assert L.dion3_step(*args(65)) == INVALID
    assert L.dion3_step(*args(16, norm=3)) == INVALID
    assert L.dion3_step(*args(16, wsb=8)) == WS
    # the state dtype: bf16, f16 and f32 reach the workspace check; any other value is
    # refused; an f32 state needs the larger workspace
    assert L.dion3_step(*args(16, wsb=8, dt=F16)) == WS
    assert L.dion3_step(*args(16, wsb=8, dt=F32)) == WS
    assert L.dion3_step(*args(16, dt=7)) == INVALID
    assert L.dion3_workspace_size(64, 256, 16, F32, F16) > L.dion3_workspace_size(64, 256, 16, BF16, F16)
    assert L.dion3_workspace_size(64, 256, 16, F16, F16) == L.dion3_workspace_size(64, 256, 16, BF16, F16)
    # with at least 2048 selected rows a bf16 state with fp16 iterates also holds the
    # fp16 copy of the selected rows
    assert (L.dion3_workspace_size(4096, 256, 2048, BF16, F16)
            == L.dion3_workspace_size(4096, 256, 2048, F16, F16) + 2048 * 256 * 2)
    assert L.dion3_workspace_size(4096, 256, 2047, BF16, F16) == L.dion3_workspace_size(4096, 256, 2047, F16, F16) \
        + 2048 * 256 * 2
    assert L.dion3_workspace_size(4096, 256, 2040, BF16, F16) == L.dion3_workspace_size(4096, 256, 2040, F16, F16)
    assert L.dion3_workspace_size(64, 256, 16, 7, F16) == 0
    # batched dion3: empty batch, short batch stride, aliased state, short workspace
    bargs = lambda B, stride, W=FAKE, M=FAKE * 8, G=FAKE * 16, wsb=1 << 40: (
        W, M, G, BF16, B, 64, 256, 256, stride, 16, 0.02, 0.0, 0.95, 1, F16, ctypes.byref(sched), FAKE * 30, None,
        FAKE * 40, wsb, None)
    assert L.dion3_step_batched(*bargs(0, 0)) == OK
    assert L.dion3_step_batched(*bargs(2, 64 * 256 - 8)) == INVALID
    assert L.dion3_step_batched(*bargs(2, 64 * 256, M=FAKE + 64 * 256 * 2)) == INVALID   # M overlaps W's 2nd entry
    assert L.dion3_step_batched(*bargs(2, 64 * 256, wsb=8)) == WS
    assert L.dion3_batched_workspace_size(2, 64, 256, 16, BF16, F16) > L.dion3_workspace_size(64, 256, 16, BF16,
                                                                                               F16)
    # dion3 on a caller-chosen row set: null S, k > N, short workspace, aliasing; any k is
    # accepted (the submatrix is padded to whole 8-row groups), so k = 12 reaches the
    # workspace check
    rargs = lambda S=FAKE * 30, k=16, W=FAKE, wsb=1 << 40: (W, FAKE * 8, FAKE * 16, BF16, 64, 256, 256, S, k, 0.02,
                                                           0.0, 0.95, F16, ctypes.byref(sched), None, FAKE * 40, wsb,
                                                           None)
    assert L.dion3_step_rows(*rargs(S=None)) == INVALID
    assert L.dion3_step_rows(*rargs(k=72)) == INVALID
    assert L.dion3_step_rows(*rargs(k=12, wsb=8)) == WS
    assert L.dion3_workspace_size(64, 256, 12, BF16, F16) == L.dion3_workspace_size(64, 256, 16, BF16, F16)
    assert L.dion3_step_rows(*rargs(wsb=8)) == WS
    assert L.dion3_step_rows(*rargs(W=FAKE * 8)) == INVALID                # W is M
    # dion3 with device scalars: null scalars, misaligned scalars, null S
    dargs = lambda sc=FAKE * 50, S=FAKE * 30: (FAKE, FAKE * 8, FAKE * 16, BF16, 64, 256, 256, 16, sc, 1, F16,
                                              ctypes.byref(sched), S, None, FAKE * 40, 1 << 40, None)
    assert L.dion3_step_dev_scalars(*dargs(sc=None)) == INVALID
    assert L.dion3_step_dev_scalars(*dargs(sc=FAKE * 50 + 2)) == UNSUP
    assert L.dion3_step_dev_scalars(*dargs(S=None)) == INVALID
    # dion3 on columns: k > m, N not a multiple of 8, short workspace
    cargs = lambda k=16, N=64, wsb=1 << 40: (FAKE, FAKE * 8, FAKE * 16, BF16, N, 256, 256, k, 0.02, 0.0, 0.95, 1,
                                            F16, ctypes.byref(sched), FAKE * 30, None, FAKE * 40, wsb, None)
    assert L.dion3_step_cols(*cargs(k=264)) == INVALID
    assert L.dion3_step_cols(*cargs(N=60)) == UNSUP
    assert L.dion3_step_cols(*cargs(wsb=8)) == WS
    assert L.dion3_cols_workspace_size(64, 256, 16, BF16, F16) > 2 * 16 * 64 * 2 + 2 * 256 * 8
    assert L.dion3_cols_workspace_size(64, 256, 16, F32, F16) > L.dion3_cols_workspace_size(64, 256, 16, BF16, F16)
    # O_out overlapping the workspace or the state is rejected before anything runs
    # (without a GPU, a launch would report GNS_ERR_HIP instead)
    oargs = lambda O: (FAKE, FAKE * 8, FAKE * 16, BF16, 64, 256, 256, 16, 0.02, 0.0, 0.95, 1, F16,
                       ctypes.byref(sched), FAKE * 30, O, FAKE * 40, 1 << 30, None)
    assert L.dion3_step(*oargs(FAKE * 40 + 4096)) == INVALID            # inside the workspace
    assert L.dion3_step(*oargs(FAKE * 8)) == INVALID                    # O is M
    coargs = lambda O: (FAKE, FAKE * 8, FAKE * 16, BF16, 64, 256, 256, 16, 0.02, 0.0, 0.95, 1, F16,
                        ctypes.byref(sched), FAKE * 30, O, FAKE * 40, 1 << 30, None)
    assert L.dion3_step_cols(*coargs(FAKE * 40 + 4096)) == INVALID
    assert L.dion3_step_cols(*coargs(FAKE)) == INVALID                  # O is W
    assert L.dion3_select_topk(FAKE, 10, 11, FAKE, None) == INVALID
    assert L.dion3_select_topk(FAKE, 10, 0, FAKE, None) == INVALID


def test_muon_validation():
    """The Muon step checks every argument before any launch: each rejected call
    below returns its error code.  On a machine without a GPU a well-formed call
    reaches the launch and reports GNS_ERR_HIP, which it could not before the checks
    had passed; with a GPU present those two calls are left out (their pointers are
    not real)."""
    sched = gns.default_schedule()
    HIP = -4

    def margs(B=2, n=64, m=256, ld=256, stride=64 * 256, W=FAKE, M=FAKE * 8, G=FAKE * 16, nest=1, lr=0.02,
              scale=0.0, compute=F16, O=None, ws=FAKE * 40, wsb=1 << 40, dt=BF16):
        return (W, M, G, dt, B, n, m, ld, stride, lr, 0.0, 0.95, nest, scale, compute, ctypes.byref(sched), O, ws,
                wsb, None)

    assert L.muon_step_batched(*margs(B=0)) == OK
    assert L.muon_step_batched(*margs(B=-1)) == INVALID
    assert L.muon_step_batched(*margs(W=None)) == INVALID
    assert L.muon_step_batched(*margs(ld=248)) == INVALID                # ld < m
    assert L.muon_step_batched(*margs(stride=64 * 256 - 8)) == INVALID   # entries overlap
    assert L.muon_step_batched(*margs(M=FAKE + 64 * 256 * 2)) == INVALID  # M overlaps W's 2nd entry
    assert L.muon_step_batched(*margs(nest=2)) == INVALID
    assert L.muon_step_batched(*margs(lr=float("nan"))) == INVALID
    assert L.muon_step_batched(*margs(scale=float("inf"))) == INVALID
    assert L.muon_step_batched(*margs(scale=-1.0)) == INVALID             # 0 = default; negative refused
    assert L.muon_step_batched(*margs(m=252, ld=256)) == UNSUP            # m not a multiple of 8
    assert L.muon_step_batched(*margs(n=60, stride=60 * 256)) == UNSUP    # n not a multiple of 8
    assert L.muon_step_batched(*margs(compute=F32)) == UNSUP
    assert L.muon_step_batched(*margs(W=FAKE + 2)) == UNSUP               # misaligned
    assert L.muon_step_batched(*margs(ws=None)) == WS
    assert L.muon_step_batched(*margs(wsb=8)) == WS
    assert L.muon_step_batched(*margs(O=FAKE * 40 + 4096)) == INVALID     # O inside the workspace
    assert L.muon_step_batched(*margs(O=FAKE * 8)) == INVALID             # O is M
    assert L.muon_step_batched(*margs(dt=7)) == INVALID                   # not a state type
    assert L.muon_step_batched(*margs(dt=F32, wsb=8)) == WS               # fp32 and f16 states accepted
    assert L.muon_step_batched(*margs(dt=F16, wsb=8)) == WS
    import torch
    if torch.cuda.device_count() == 0:
        assert L.muon_step_batched(*margs()) == HIP                       # valid: reaches the launch
        assert L.muon_step_batched(*margs(nest=0, B=1, n=512, m=64, ld=64, stride=0)) == HIP   # tall, no lookahead
    with_u = L.muon_workspace_size(2, 64, 256, BF16, F16, 1)
    assert with_u - L.muon_workspace_size(2, 64, 256, BF16, F16, 0) >= 2 * 64 * 256 * 2
    assert L.muon_workspace_size(2, 64, 256, BF16, F16, 2) == 0
    assert L.muon_workspace_size(2, 64, 256, F32, F16, 1) > with_u


def test_workspace_sizes_grow_with_problem():
    a = L.gns_workspace_size(1, 1024, 4096, F16)
    b = L.gns_workspace_size(2, 1024, 4096, F16)
    c = L.gns_workspace_size(1, 1024, 4096, F32)
    assert 0 < a < b and a < c
    # 5 n x n iterates + 2 X-shaped buffers in fp16, plus small scalars
    assert a >= (5 * 1024 * 1024 + 2 * 1024 * 4096) * 2
    assert L.dion3_workspace_size(8192, 28672, 2048, BF16, F16) > 2 * 2048 * 28672 * 2


def test_pages_flop_savings():
    g = GOLD["flop_savings_T5_alpha4"]
    gram = flops.pages_gram(5, 4)
    assert abs((1 - gram / flops.pages_standard_symmetric(5, 4)) - g["vs_standard_symmetric"]) < 0.01
    assert abs((1 - gram / flops.pages_standard_plain(5, 4)) - g["vs_standard_plain"]) < 0.01
    # equal cost at alpha = 1 without restart is NOT claimed; with one restart the schedule
    # costs pages_gram + restart_extra, which is what libgns runs
    n, m = 1024, 4096
    exact = flops.gram_schedule(n, m, 5, (2,))
    approx = (flops.pages_gram(5, 4) + flops.pages_restart_extra(4)) * n ** 3
    assert abs(exact / approx - 1) < 0.01
    assert flops.standard_ns_nominal(n, m) == flops.pages_standard_plain(5, 4) * n ** 3


@pytest.mark.parametrize("alpha", [1, 2, 4, 8, 14, 28])
def test_gram_cheaper_than_standard_for_alpha_above_one(alpha):
    n = 512
    g = flops.gram_schedule(n, alpha * n)
    s = flops.standard_schedule(n, alpha * n)
    if alpha == 1:
        assert g >= s * 0.99     # no saving (and the restart is not free) at alpha = 1
    else:
        assert g < s


def test_binding_rejects_mismatched_tensors_before_any_call():
    """The binding checks dtype/shape/device of every tensor it turns into a raw
    pointer (a C operand in the wrong dtype would make the kernel read past the
    allocation).  CPU tensors are rejected first, so this runs without a GPU."""
    import torch
    a = torch.zeros(2, 64, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        gns.symm_gemm(a, a)                       # not on the GPU
    with pytest.raises(ValueError):
        gns.rect_gemm(a, a)
    with pytest.raises(ValueError):
        gns.orthogonalize(a)


def test_missing_library_fails_loudly():
    """Without the built HIP library the package does not import: there is no CPU
    fallback to fall back on."""
    import glob
    import shutil
    import subprocess
    import sys
    import tempfile
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with tempfile.TemporaryDirectory() as tmp:
        pkg = os.path.join(tmp, "muon_gram_ns_amd")          # the package's Python files, no libgns.so
        os.makedirs(pkg)
        for f in glob.glob(os.path.join(root, "muon_gram_ns_amd", "*.py")):
            shutil.copy(f, pkg)
        env = dict(os.environ, PYTHONPATH=tmp)
        r = subprocess.run([sys.executable, "-c", "import muon_gram_ns_amd"], env=env, cwd=tmp, capture_output=True,
                           text=True, timeout=300)
    assert r.returncode != 0
    assert "is missing" in r.stderr


def test_binding_refuses_cpu_tensors():
    """Host tensors are refused before any pointer reaches the library."""
    import torch
    x = torch.zeros(64, 256, dtype=torch.bfloat16)
    calls = [lambda: gns.orthogonalize(x), lambda: gns.newton_schulz(x),
             lambda: gns.muon_step(x, x.clone(), x.clone(), 0.01),
             lambda: gns.dion3_step(x, x.clone(), x.clone(), 16, 0.01),
             lambda: gns.dion3_step_batched(x[None], x.clone()[None], x.clone()[None], 16, 0.01)]
    for call in calls:
        with pytest.raises(ValueError, match="no CPU path"):
            call()
