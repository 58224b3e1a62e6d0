"""HIP-graph replay of whole library calls on fixed buffers.

The library allocates nothing and only enqueues kernels on the caller's stream, so
one call can be captured in a HIP graph and replayed: the replay issues the same
kernels with the same arguments, without host-side launch work (the pages capture the
optimizer step in a CUDA graph at small scale: "Dion3: Full-Stack Orthogonal
Updates", paper.rainbus.top, 方法步骤详情 (4)).  This is for callers that capture a
larger step; measured on MI355X with ROCm 7, a replay of one Gram NS call is not
faster than its eager launches (the kernels, not the host, bound the call).  A
captured call reads and writes exactly the buffers it was captured with, so every
object here owns its output and workspace: nothing that a later call allocates or
frees can move them.  Inputs are read from the captured tensors, so refill them in
place (copy_) between replays.
"""
from __future__ import annotations

from . import _lib


class Graphed:
    """fn() captured once in a HIP graph on torch's capture stream; replay() reruns it
    and returns what the captured call returned."""

    def __init__(self, fn, warmup: int = 2):
        torch = _lib._torch()
        # lazy one-time work (kernel attributes, allocator growth) happens before the
        # capture, on a side stream at the default priority
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.result = fn()

    def replay(self):
        self.graph.replay()
        return self.result


def _owned_ns(method, X, out, compute, schedule):
    torch = _lib._torch()
    X3, B, n, m, _, _ = _lib._mat3(_lib._dev(X))
    if out is None:
        out = torch.empty_like(X)
    ws = torch.empty(max(_lib.workspace_size(B, n, m, compute), 256), dtype=torch.uint8, device=X.device)
    sched = schedule if schedule is not None else _lib.default_schedule()
    fn = (lambda: method(X, out=out, compute=compute, schedule=sched, workspace=ws))
    g = Graphed(fn)
    g.X, g.out, g.workspace, g.schedule = X, out, ws, sched
    return g


def graphed_orthogonalize(X, out=None, compute="f16", schedule=None) -> Graphed:
    """Gram NS of the tensor X into out (allocated if None), captured; replay()
    recomputes out from X's current contents."""
    return _owned_ns(_lib.orthogonalize, X, out, compute, schedule)


def graphed_newton_schulz(X, out=None, compute="f16", schedule=None) -> Graphed:
    """Standard NS on the same kernels, captured like graphed_orthogonalize."""
    return _owned_ns(_lib.newton_schulz, X, out, compute, schedule)


def graphed_dion3_step(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=1, compute="f16",
                       schedule=None, return_O=False, device_scalars=False) -> Graphed:
    """One Dion3 step on W, M (in place) and G, captured; each replay() runs one more
    step on the buffers' current contents and returns S (and O).

    device_scalars=True captures the step that reads lr, weight decay and mu from a
    device tensor the object owns (`scalars`); set_scalars() rewrites it between
    replays, so one capture follows a learning-rate schedule."""
    torch = _lib._torch()
    N, m, _ = _lib._rows(W)
    S = torch.empty(k, dtype=torch.int32, device=W.device)
    O = torch.empty((k, m), dtype=W.dtype, device=W.device) if return_O else None
    ws = torch.empty(max(int(_lib.lib.dion3_workspace_size(N, m, k, _lib.dtype_code(W), _lib.code_of(compute))),
                         256), dtype=torch.uint8, device=W.device)
    sched = schedule if schedule is not None else _lib.default_schedule()
    scalars = None
    if device_scalars:
        scalars = torch.tensor([lr, weight_decay, mu], dtype=torch.float32, device=W.device)
        fn = (lambda: _lib.dion3_step_dev_scalars(W, M, G, k, scalars, score_norm, compute, sched, S=S, O=O,
                                                  workspace=ws))
    else:
        fn = (lambda: _lib.dion3_step(W, M, G, k, lr, weight_decay, mu, score_norm, compute, sched, return_O,
                                      S=S, O=O, workspace=ws))
    # the warm-up calls run real steps (the capture itself executes nothing), so the
    # caller's W and M are saved before and restored after them
    saved = (W.clone(), M.clone())
    g = Graphed(fn)
    W.copy_(saved[0])
    M.copy_(saved[1])
    torch.cuda.synchronize()
    g.W, g.M, g.G, g.S, g.O, g.workspace, g.schedule, g.scalars = W, M, G, S, O, ws, sched, scalars

    def set_scalars(lr, weight_decay, mu):
        """Values the next replays read (device_scalars=True only)."""
        if g.scalars is None:
            raise ValueError("captured with host scalars: capture with device_scalars=True")
        g.scalars.copy_(torch.tensor([lr, weight_decay, mu], dtype=torch.float32))

    g.set_scalars = set_scalars
    return g


def graphed_muon_step(W, M, G, lr, weight_decay=0.0, mu=0.95, nesterov=True, scale=None, compute="f16",
                      schedule=None, return_O=False) -> Graphed:
    """One Muon step (muon_step) on W, M (in place) and G, each [n, m] or [B, n, m],
    captured; each replay() runs one more step on the buffers' current contents and
    returns O when return_O (else None)."""
    torch = _lib._torch()
    B, n, m = (1, *W.shape) if W.dim() == 2 else tuple(W.shape)
    O = torch.empty(W.shape, dtype=torch.bfloat16, device=W.device) if return_O else None
    ws = torch.empty(max(_lib.muon_workspace_size(B, n, m, compute, nesterov), 256), dtype=torch.uint8,
                     device=W.device)
    sched = schedule if schedule is not None else _lib.default_schedule()
    fn = (lambda: _lib.muon_step(W, M, G, lr, weight_decay, mu, nesterov, scale, compute, sched, O=O, workspace=ws))
    # the warm-up calls run real steps, so the caller's W and M are restored after them
    saved = (W.clone(), M.clone())
    g = Graphed(fn)
    W.copy_(saved[0])
    M.copy_(saved[1])
    torch.cuda.synchronize()
    g.W, g.M, g.G, g.O, g.workspace, g.schedule = W, M, G, O, ws, sched
    return g
