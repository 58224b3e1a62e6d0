"""The no-allocation entry point (gns_orthogonalize_batched_noalloc), called through
the C ABI, against the workspace entry point it is a variant of: the same kernels on
the library's static device scratch must give bitwise the same output.  Two calls in
a row, the second with a smaller input, so the second runs on scratch that still
holds the first call's data; a call larger than the scratch is refused."""
import ctypes

import numpy as np
import pytest

import synth
from gpu_helpers import to_dev, bits, announce

pytestmark = pytest.mark.gpu


def noalloc_call(gns_mod, X, out, compute):
    """One call of the C entry point with the binding's argument marshalling done by
    hand (pointers, sizes, strides, the current stream)."""
    import torch
    L = gns_mod.lib
    B, n, m = X.shape
    sched = gns_mod.default_schedule()
    code = {"f16": gns_mod.GNS_F16, "bf16": gns_mod.GNS_BF16}[compute]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    flops = ctypes.c_double(0.0)
    return L.gns_orthogonalize_batched_noalloc(X.data_ptr(), gns_mod.GNS_BF16, m, n * m, out.data_ptr(),
                                               gns_mod.GNS_BF16, m, n * m, B, n, m, code, ctypes.byref(sched),
                                               stream, ctypes.byref(flops)), flops.value


@pytest.mark.parametrize("compute", ["f16", "bf16"])
def test_noalloc_matches_workspace_entry_point(gns_mod, compute):
    import torch
    cases = [("gns_1024x4096_bf16", 1, 1024, 4096), ("gns_128x768x6144_bf16", 3, 256, 1024)]
    for name, B, n, m in cases:              # the second call is smaller than the first
        announce(f"noalloc {compute} {B}x{n}x{m}")
        st = synth.gns_batch(name, batch=B, n=n, m=m, seed=501)
        X = to_dev(st, "bf16")
        out = torch.full_like(X, float("nan"))
        status, fl = noalloc_call(gns_mod, X, out, compute)
        assert status == 0, gns_mod.lib.gns_last_error()
        torch.cuda.synchronize()
        ref, fl_ref = gns_mod.orthogonalize(X, compute=compute, return_flops=True)
        assert np.array_equal(bits(out), bits(ref))
        assert fl == fl_ref
        # the binding's wrapper of the same entry point
        assert np.array_equal(bits(gns_mod.orthogonalize_noalloc(X, compute=compute)), bits(ref))


def test_noalloc_refuses_a_call_larger_than_the_scratch(gns_mod):
    import torch
    announce("noalloc too large")
    B, n, m = 4, 1024, 4096
    assert gns_mod.workspace_size(B, n, m) > gns_mod._lib.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((B, n, m), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(X, 1.0)
    status, _ = noalloc_call(gns_mod, X, out, "f16")
    assert status == -3                                 # GNS_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert bool((out == 1.0).all())
    assert b"scratch" in gns_mod.lib.gns_last_error()
