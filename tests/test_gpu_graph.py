"""The ABI allocates nothing and issues only kernels on the caller's stream, so a call
can be captured in a HIP graph.  Each captured call is replayed several times, with
eager calls and synchronisations in between, and every replay must give the same bits
as the eager call."""
import numpy as np
import pytest

import synth
from gpu_helpers import to_dev, bits, announce

pytestmark = pytest.mark.gpu


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
