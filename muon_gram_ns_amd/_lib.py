"""ctypes binding of libgns.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module only turns
torch tensors into device pointers, sizes and the current HIP stream, allocates the
caller-owned workspace with torch (device memory plumbing) and raises on a non-zero
status.  If libgns.so is missing the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgns.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "gns.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python muon_gram_ns_amd/build.py` "
                      "(the HIP library is required; there is no CPU path)")
# Load torch (when installed) BEFORE libgns: PyTorch for ROCm ships its own HIP
# runtime, and the dynamic linker reuses it for libgns's libamdhip64.so.7 dependency
# only if it is already loaded.  Loading libgns first would bring in /opt/rocm's copy,
# after which torch loads a second runtime of its own; the two cannot share the GPU.
try:
    import torch as _torch_for_runtime  # noqa: F401
except ImportError:        # plain use without torch: libgns uses the system runtime
    pass
lib = ctypes.CDLL(LIB_PATH)

GNS_BF16, GNS_F32, GNS_F16 = 0, 1, 2
GNS_MAX_STEPS = 16
STATUS = {0: "GNS_OK", -1: "GNS_ERR_INVALID_ARG", -2: "GNS_ERR_UNSUPPORTED",
          -3: "GNS_ERR_WORKSPACE", -4: "GNS_ERR_HIP"}

F = ctypes.c_float
I = ctypes.c_int
LL = ctypes.c_longlong
P = ctypes.c_void_p
SZ = ctypes.c_size_t
DP = ctypes.POINTER(ctypes.c_double)


class Schedule(ctypes.Structure):
    _fields_ = [("steps", I), ("a", F * GNS_MAX_STEPS), ("b", F * GNS_MAX_STEPS),
                ("c", F * GNS_MAX_STEPS), ("restart_after_mask", ctypes.c_uint), ("eps", F),
                ("square_fallback", I), ("rows_in_place", I)]


def _sig(name, res, *args):
    f = getattr(lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_sig("gns_default_schedule", None, ctypes.POINTER(Schedule))
_sig("gns_status_string", ctypes.c_char_p, I)
_sig("gns_last_error", ctypes.c_char_p)
_sig("gns_frobenius_workspace_size", SZ, I, I, I)
_sig("gns_frobenius_scale", I, P, I, LL, LL, I, I, I, F, P, P, SZ, P)
_sig("gns_workspace_size", SZ, I, I, I, I)
_NS_ARGS = (P, I, LL, LL, P, I, LL, LL, I, I, I, I, ctypes.POINTER(Schedule), P, SZ, P, DP)
_sig("gns_orthogonalize_batched", I, *_NS_ARGS)
_sig("gns_newton_schulz_batched", I, *_NS_ARGS)
_sig("gns_orthogonalize_batched_noalloc", I, P, I, LL, LL, P, I, LL, LL, I, I, I, I, ctypes.POINTER(Schedule), P, DP)
NOALLOC_SCRATCH_BYTES = 64 << 20     # GNS_NOALLOC_SCRATCH_BYTES
_sig("symm_gemm", I, I, I, I, F, P, LL, LL, P, LL, LL, F, P, LL, LL, F, P, LL, LL, I, I, P)
_sig("rect_gemm", I, I, I, I, I, F, P, LL, LL, I, P, LL, LL, I, F, F, P, LL, LL, P, LL, LL, I, P)
_sig("dion3_accumulate_score", I, P, P, I, I, I, LL, I, P, P, P)
_sig("dion3_select_topk", I, P, I, I, P, P)
_sig("dion3_gather_feedback", I, P, I, I, I, LL, P, I, F, P, LL, P)
_sig("dion3_apply_update", I, P, I, I, I, LL, P, I, P, I, LL, F, F, P)
_sig("dion3_workspace_size", SZ, I, I, I, I, I)
_sig("dion3_step", I, P, P, P, I, I, I, LL, I, F, F, F, I, I, ctypes.POINTER(Schedule), P, P, P, SZ, P)
_sig("dion3_batched_workspace_size", SZ, I, I, I, I, I, I)
_sig("dion3_step_batched", I, P, P, P, I, I, I, I, LL, LL, I, F, F, F, I, I, ctypes.POINTER(Schedule), P, P, P, SZ,
     P)
_sig("dion3_step_rows", I, P, P, P, I, I, I, LL, P, I, F, F, F, I, ctypes.POINTER(Schedule), P, P, SZ, P)
_sig("dion3_step_dev_scalars", I, P, P, P, I, I, I, LL, I, P, I, I, ctypes.POINTER(Schedule), P, P, P, SZ, P)
_sig("dion3_cols_workspace_size", SZ, I, I, I, I, I)
_sig("dion3_step_cols", I, P, P, P, I, I, I, LL, I, F, F, F, I, I, ctypes.POINTER(Schedule), P, P, P, SZ, P)
_sig("muon_workspace_size", SZ, I, I, I, I, I, I)
_sig("muon_step_batched", I, P, P, P, I, I, I, I, LL, LL, F, F, F, I, F, I, ctypes.POINTER(Schedule), P, P, SZ, P)


def header_functions() -> list[str]:
    """Names of the functions include/gns.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


class GnsError(RuntimeError):
    pass


def check(status: int, what: str):
    if status != 0:
        detail = lib.gns_last_error().decode() if status == -4 else ""
        raise GnsError(f"{what} failed: {STATUS.get(status, status)} {detail}".rstrip())


def default_schedule(steps=5, abc=(3.4445, -4.7750, 2.0315), restart_after=(2,), eps=1e-7,
                     square_fallback=True, rows_in_place=False) -> Schedule:
    s = Schedule()
    lib.gns_default_schedule(ctypes.byref(s))
    s.steps = steps
    table = [abc] * steps if len(abc) == 3 and not hasattr(abc[0], "__len__") else list(abc)
    for t, (a, b, c) in enumerate(table):
        s.a[t], s.b[t], s.c[t] = a, b, c
    mask = 0
    for r in restart_after:
        mask |= 1 << r
    s.restart_after_mask = mask
    s.eps = eps
    s.square_fallback = 1 if square_fallback else 0
    s.rows_in_place = 1 if rows_in_place else 0
    return s


# ---- torch marshalling ---------------------------------------------------------------

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.bfloat16: GNS_BF16, torch.float16: GNS_F16, torch.float32: GNS_F32}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def torch_dtype(code: int):
    torch = _torch()
    return {GNS_BF16: torch.bfloat16, GNS_F16: torch.float16, GNS_F32: torch.float32}[code]


def code_of(name) -> int:
    if isinstance(name, int):
        return name
    return {"bf16": GNS_BF16, "f16": GNS_F16, "fp16": GNS_F16, "f32": GNS_F32, "fp32": GNS_F32}[name]


def _dev(t):
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU (the HIP library has no CPU path)")
    return t


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


_WS = {}


def workspace(nbytes: int, device):
    """Grow-only per-device workspace (torch-allocated device memory) for calls made
    without one.  Calls on one stream are ordered, so they share it safely; calls that
    run concurrently on different streams must each pass their own workspace.  The
    buffer is marked as used by the current stream, so when it grows, torch does not
    hand the old block to another stream before this stream's kernels are done."""
    torch = _torch()
    key = torch.device(device).index
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    if not torch.cuda.is_current_stream_capturing():
        buf.record_stream(torch.cuda.current_stream(buf.device))
    return buf


def _mat3(x):
    """(batch, n, m, ld, batch_stride) of a [B, n, m] or [n, m] tensor with unit column stride."""
    if x.dim() == 2:
        x = x.unsqueeze(0)
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("expected a [B, n, m] or [n, m] tensor with contiguous rows")
    B, n, m = x.shape
    return x, B, n, m, x.stride(1), (x.stride(0) if B > 1 else n * x.stride(1))


def _workspace_arg(ws, nbytes, device):
    """A caller-given workspace tensor (uint8 on the same device, >= nbytes), or the
    shared grow-only one."""
    torch = _torch()
    if ws is None:
        return workspace(nbytes, device)
    _expect(ws, "workspace", dtype=torch.uint8, device=torch.device(device))
    if not ws.is_contiguous() or ws.numel() < nbytes:
        raise ValueError(f"workspace needs {nbytes} contiguous bytes, got {ws.numel()}")
    return ws


def _ns(fn_name, X, out, compute, schedule, want_flops, ws=None):
    torch = _torch()
    _dev(X)
    squeeze = X.dim() == 2
    X3, B, n, m, ldx, sx = _mat3(X)
    if out is None:
        out = torch.empty((B, n, m), dtype=X.dtype, device=X.device)
    _expect(out, "out", device=X.device)
    O3, Bo, no, mo, ldo, so = _mat3(out)
    if (Bo, no, mo) != (B, n, m):
        raise ValueError("output shape mismatch")
    cdt = code_of(compute)
    sched = schedule if schedule is not None else default_schedule()
    ws_n = lib.gns_workspace_size(B, n, m, cdt)
    ws = _workspace_arg(ws, ws_n, X.device)
    flops = ctypes.c_double(0.0)
    st = getattr(lib, fn_name)(X3.data_ptr(), dtype_code(X3), ldx, sx, O3.data_ptr(), dtype_code(O3), ldo, so,
                               B, n, m, cdt, ctypes.byref(sched), ws.data_ptr(), ws.numel(),
                               _stream(X.device), ctypes.byref(flops))
    check(st, fn_name)
    res = out.squeeze(0) if (squeeze and out.dim() == 3) else out
    return (res, flops.value) if want_flops else res


def orthogonalize(X, out=None, compute="f16", schedule=None, return_flops=False, workspace=None):
    """Gram Newton-Schulz of X ([B, n, m] or [n, m]; a tall X runs on its transpose)
    -> same shape/dtype as X.
    workspace: optional uint8 device tensor of >= gns_workspace_size bytes."""
    return _ns("gns_orthogonalize_batched", X, out, compute, schedule, return_flops, workspace)


def orthogonalize_noalloc(X, out=None, compute="f16", schedule=None):
    """orthogonalize on the library's static device scratch (gns_orthogonalize_batched_noalloc):
    no workspace is allocated, for callers that cannot allocate.  Calls on one GPU
    share the scratch, so they must not overlap in time."""
    torch = _torch()
    _dev(X)
    squeeze = X.dim() == 2
    X3, B, n, m, ldx, sx = _mat3(X)
    if out is None:
        out = torch.empty((B, n, m), dtype=X.dtype, device=X.device)
    _expect(out, "out", device=X.device)
    O3, Bo, no, mo, ldo, so = _mat3(out)
    if (Bo, no, mo) != (B, n, m):
        raise ValueError("output shape mismatch")
    sched = schedule if schedule is not None else default_schedule()
    st = lib.gns_orthogonalize_batched_noalloc(X3.data_ptr(), dtype_code(X3), ldx, sx, O3.data_ptr(), dtype_code(O3),
                                               ldo, so, B, n, m, code_of(compute), ctypes.byref(sched),
                                               _stream(X.device), None)
    if st == -3:
        raise GnsError(f"gns_orthogonalize_batched_noalloc: {lib.gns_last_error().decode()}")
    check(st, "gns_orthogonalize_batched_noalloc")
    return out.squeeze(0) if (squeeze and out.dim() == 3) else out


def newton_schulz(X, out=None, compute="f16", schedule=None, return_flops=False, workspace=None):
    """Standard quintic Newton-Schulz on the same kernels."""
    return _ns("gns_newton_schulz_batched", X, out, compute, schedule, return_flops, workspace)


def workspace_size(batch, n, m, compute="f16") -> int:
    return int(lib.gns_workspace_size(batch, n, m, code_of(compute)))


def frobenius_scale(X, eps=1e-7):
    torch = _torch()
    _dev(X)
    X3, B, n, m, ldx, sx = _mat3(X)
    s = torch.empty(B, dtype=torch.float32, device=X.device)
    ws = workspace(lib.gns_frobenius_workspace_size(B, n, m), X.device)
    check(lib.gns_frobenius_scale(X3.data_ptr(), dtype_code(X3), ldx, sx, B, n, m, eps, s.data_ptr(),
                                  ws.data_ptr(), ws.numel(), _stream(X.device)), "gns_frobenius_scale")
    return s


def _expect(t, name, dtype=None, shape=None, device=None):
    """The C ABI receives raw pointers, so every tensor's dtype, shape and device are
    checked here: a mismatch would make a kernel read or write past an allocation."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    _dev(t)
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def symm_gemm(A, B=None, C=None, alpha=1.0, beta=0.0, gamma=0.0, out=None, out_dtype=None):
    """D = alpha A B^T + beta C + gamma I (lower tiles, mirrored) for [batch, n, k] A, B.
    C and the output are [batch, n, n] in the output dtype."""
    torch = _torch()
    _dev(A)
    squeeze = A.dim() == 2
    B = A if B is None else B
    A3, nb, n, k, lda, sa = _mat3(A)
    _expect(B, "B", dtype=A.dtype, shape=A.shape, device=A.device)
    B3, _, _, _, ldb, sb = _mat3(B)
    odt = dtype_code(A3) if out_dtype is None else code_of(out_dtype)
    tdt = torch_dtype(odt)
    if out is None:
        out = torch.empty((nb, n, n), dtype=tdt, device=A.device)
    _expect(out, "out", dtype=tdt, shape=(n, n) if (squeeze and out.dim() == 2) else (nb, n, n), device=A.device)
    D3, _, _, _, ldd, sd = _mat3(out)
    if C is not None:
        _expect(C, "C", dtype=tdt, shape=tuple(out.shape), device=A.device)
        C3, _, _, _, ldc, sc = _mat3(C)
        cptr = C3.data_ptr()
    else:
        cptr, ldc, sc = None, n, n * n
    check(lib.symm_gemm(nb, n, k, alpha, A3.data_ptr(), lda, sa, B3.data_ptr(), ldb, sb, beta, cptr, ldc, sc,
                        gamma, D3.data_ptr(), ldd, sd, dtype_code(A3), odt, _stream(A.device)),
          "symm_gemm")
    return out.squeeze(0) if (squeeze and out.dim() == 3) else out


def rect_gemm(A, Bm, C=None, alpha=1.0, beta=0.0, b_prescale=1.0, out=None, out_dtype=None):
    """D = alpha A B + beta C for A [batch, n, k], B [batch, k, m]; C and the output are
    [batch, n, m] in the output dtype."""
    torch = _torch()
    _dev(A)
    squeeze = A.dim() == 2
    A3, nb, n, k, lda, sa = _mat3(A)
    _expect(Bm, "B", device=A.device)
    if Bm.dim() != A.dim():
        raise ValueError("A and B must both be 2-D or both 3-D")
    B3, nb2, k2, m, ldb, sb = _mat3(Bm)
    if (nb2, k2) != (nb, k):
        raise ValueError("A and B shapes differ")
    odt = dtype_code(A3) if out_dtype is None else code_of(out_dtype)
    tdt = torch_dtype(odt)
    oshape = (n, m) if squeeze else (nb, n, m)
    if out is None:
        out = torch.empty(oshape, dtype=tdt, device=A.device)
    _expect(out, "out", dtype=tdt, shape=oshape, device=A.device)
    D3, _, _, _, ldd, sd = _mat3(out)
    if C is not None:
        _expect(C, "C", dtype=tdt, shape=oshape, device=A.device)
        C3, _, _, _, ldc, sc = _mat3(C)
        cptr = C3.data_ptr()
    else:
        cptr, ldc, sc = None, m, n * m
    check(lib.rect_gemm(nb, n, k, m, alpha, A3.data_ptr(), lda, sa, dtype_code(A3), B3.data_ptr(), ldb, sb,
                        dtype_code(B3), b_prescale, beta, cptr, ldc, sc, D3.data_ptr(), ldd, sd, odt,
                        _stream(A.device)), "rect_gemm")
    return out


# ---- Dion3 -------------------------------------------------------------------------

def _rows(x):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a [N, m] tensor with contiguous rows")
    return x.shape[0], x.shape[1], x.stride(0)


def _state_rows(x, name):
    """[N, m] rows of a Dion3 state tensor (bf16, fp16 or fp32) -> (N, m, ld, dtype code)."""
    torch = _torch()
    _dev(x)
    if x.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError(f"{name} must be bf16, fp16 or fp32")
    return (*_rows(x), dtype_code(x))


def _same_state(W, M, G):
    """W, M and G of one Dion3 state: same dtype, shape, device and row stride."""
    N, m, ld, dt = _state_rows(W, "W")
    for t, name in ((M, "M"), (G, "G")):
        _expect(t, name, dtype=W.dtype, shape=W.shape, device=W.device)
        if _rows(t)[2] != ld:
            raise ValueError("W, M, G must share the row stride")
    return N, m, ld, dt


def _index_vector(S, k_max, device):
    torch = _torch()
    _expect(S, "S", dtype=torch.int32, device=device)
    if S.dim() != 1 or not S.is_contiguous() or not (1 <= S.numel() <= k_max):
        raise ValueError("S must be a contiguous 1-D int32 tensor of 1..N indices")
    return S.numel()


def dion3_accumulate_score(M, G, score_norm=1):
    torch = _torch()
    N, m, ld, dt = _state_rows(M, "M")
    _expect(G, "G", dtype=M.dtype, shape=M.shape, device=M.device)
    if _rows(G)[2] != ld:
        raise ValueError("M and G must share the row stride")
    score = torch.empty(N, dtype=torch.float64, device=M.device)
    sumsq = torch.empty(N, dtype=torch.float64, device=M.device)
    check(lib.dion3_accumulate_score(M.data_ptr(), G.data_ptr(), dt, N, m, ld, score_norm, score.data_ptr(),
                                     sumsq.data_ptr(), _stream(M.device)), "dion3_accumulate_score")
    return score, sumsq


def dion3_select_topk(score, k):
    torch = _torch()
    _expect(score, "score", dtype=torch.float64)
    if score.dim() != 1 or not score.is_contiguous():
        raise ValueError("score must be a contiguous 1-D float64 tensor")
    S = torch.empty(k, dtype=torch.int32, device=score.device)
    check(lib.dion3_select_topk(_dev(score).data_ptr(), score.numel(), k, S.data_ptr(), _stream(score.device)),
          "dion3_select_topk")
    return S


def dion3_gather_feedback(M, S, mu):
    torch = _torch()
    N, m, ld, dt = _state_rows(M, "M")
    k = _index_vector(S, N, M.device)
    X = torch.empty((k, m), dtype=M.dtype, device=M.device)
    check(lib.dion3_gather_feedback(M.data_ptr(), dt, N, m, ld, S.data_ptr(), k, mu, X.data_ptr(), m,
                                    _stream(M.device)), "dion3_gather_feedback")
    return X


def dion3_apply_update(W, S, O, lr, wd):
    torch = _torch()
    N, m, ld, dt = _state_rows(W, "W")
    k = _index_vector(S, N, W.device)
    _expect(O, "O", device=W.device)
    if O.dtype not in (torch.bfloat16, torch.float16, torch.float32) or O.dim() != 2 or O.shape[0] != k \
            or O.shape[1] != m or O.stride(1) != 1:
        raise ValueError("O must be a [k, m] bf16, fp16 or fp32 tensor with contiguous rows")
    check(lib.dion3_apply_update(W.data_ptr(), dt, N, m, ld, S.data_ptr(), k, O.data_ptr(), dtype_code(O),
                                 O.stride(0), lr, wd, _stream(W.device)), "dion3_apply_update")
    return W


def dion3_step(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=1, compute="f16", schedule=None,
               return_O=False, S=None, O=None, workspace=None):
    """One Dion3 step in place on W and M (bf16, fp16 or fp32, one dtype for W, M, G);
    returns S (and O when return_O).  S ([k] int32), O ([k, m], the state's dtype) and
    workspace may be given (fixed buffers for graph replay)."""
    torch = _torch()
    N, m, ld, dt = _same_state(W, M, G)
    cdt = code_of(compute)
    if S is None:
        S = torch.empty(k, dtype=torch.int32, device=W.device)
    _expect(S, "S", dtype=torch.int32, shape=(k,), device=W.device)
    if return_O and O is None:
        O = torch.empty((k, m), dtype=W.dtype, device=W.device)
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=(k, m), device=W.device)
        if not O.is_contiguous():
            raise ValueError("O must be contiguous")
    if not S.is_contiguous():
        raise ValueError("S must be contiguous")
    sched = schedule if schedule is not None else default_schedule()
    ws = _workspace_arg(workspace, lib.dion3_workspace_size(N, m, k, dt, cdt), W.device)
    check(lib.dion3_step(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, N, m, ld, k, lr, weight_decay, mu,
                         score_norm, cdt, ctypes.byref(sched), S.data_ptr(),
                         O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                         _stream(W.device)), "dion3_step")
    return (S, O) if (return_O or O is not None) else S


def dion3_step_cols(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=1, compute="f16", schedule=None,
                    return_O=False, S=None, O=None, workspace=None):
    """One Dion3 step on the k columns of largest score of the [N, m] state (bf16, fp16
    or fp32; in place on W and M).  Returns S ([k] int32, ascending column indices)
    and, when return_O or O is given, O ([k, N] in the state's dtype: row j is the
    update of column S[j])."""
    torch = _torch()
    N, m, ld, dt = _same_state(W, M, G)
    if S is None:
        S = torch.empty(k, dtype=torch.int32, device=W.device)
    _expect(S, "S", dtype=torch.int32, shape=(k,), device=W.device)
    if return_O and O is None:
        O = torch.empty((k, N), dtype=W.dtype, device=W.device)
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=(k, N), device=W.device)
        if not O.is_contiguous():
            raise ValueError("O must be contiguous")
    if not S.is_contiguous():
        raise ValueError("S must be contiguous")
    cdt = code_of(compute)
    sched = schedule if schedule is not None else default_schedule()
    ws = _workspace_arg(workspace, lib.dion3_cols_workspace_size(N, m, k, dt, cdt), W.device)
    check(lib.dion3_step_cols(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, N, m, ld, k, lr, weight_decay, mu,
                              score_norm, cdt, ctypes.byref(sched), S.data_ptr(),
                              O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                              _stream(W.device)), "dion3_step_cols")
    return (S, O) if O is not None else S


def dion3_step_dev_scalars(W, M, G, k, scalars, score_norm=1, compute="f16", schedule=None, S=None, O=None,
                           workspace=None):
    """dion3_step with lr, weight decay and mu read on the device from `scalars`, a
    float32 device tensor [lr, weight_decay, mu] (for steps replayed from a HIP graph
    under a schedule).  Returns S (and O when O is given)."""
    torch = _torch()
    N, m, ld, dt = _same_state(W, M, G)
    _expect(scalars, "scalars", dtype=torch.float32, shape=(3,), device=W.device)
    if not scalars.is_contiguous():
        raise ValueError("scalars must be contiguous")
    if S is None:
        S = torch.empty(k, dtype=torch.int32, device=W.device)
    _expect(S, "S", dtype=torch.int32, shape=(k,), device=W.device)
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=(k, m), device=W.device)
        if not O.is_contiguous():
            raise ValueError("O must be contiguous")
    if not S.is_contiguous():
        raise ValueError("S must be contiguous")
    cdt = code_of(compute)
    sched = schedule if schedule is not None else default_schedule()
    ws = _workspace_arg(workspace, lib.dion3_workspace_size(N, m, k, dt, cdt), W.device)
    check(lib.dion3_step_dev_scalars(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, N, m, ld, k, scalars.data_ptr(),
                                     score_norm, cdt, ctypes.byref(sched), S.data_ptr(),
                                     O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                                     _stream(W.device)), "dion3_step_dev_scalars")
    return (S, O) if O is not None else S


def dion3_step_rows(W, M, G, S, lr, weight_decay=0.0, mu=0.95, compute="f16", schedule=None, O=None,
                    workspace=None):
    """One Dion3 step in place on W and M on the caller's row set S (a [k] int32 device
    tensor of distinct ascending row indices, e.g. drawn at random).  Returns O
    ([k, m] in the state's dtype) when O is given, else None."""
    torch = _torch()
    N, m, ld, dt = _same_state(W, M, G)
    _expect(S, "S", dtype=torch.int32, device=W.device)
    if S.dim() != 1 or not S.is_contiguous():
        raise ValueError("S must be a contiguous 1-D int32 tensor")
    k = S.shape[0]
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=(k, m), device=W.device)
        if not O.is_contiguous():
            raise ValueError("O must be contiguous")
    cdt = code_of(compute)
    sched = schedule if schedule is not None else default_schedule()
    ws = _workspace_arg(workspace, lib.dion3_workspace_size(N, m, k, dt, cdt), W.device)
    check(lib.dion3_step_rows(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, N, m, ld, S.data_ptr(), k, lr,
                              weight_decay, mu, cdt, ctypes.byref(sched),
                              O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                              _stream(W.device)), "dion3_step_rows")
    return O


def dion3_step_batched(W, M, G, k, lr, weight_decay=0.0, mu=0.95, score_norm=1, compute="f16", schedule=None,
                       return_O=False, S=None, O=None, workspace=None):
    """One Dion3 step on each of the [B, N, m] states W, M (bf16, fp16 or fp32; in place)
    with gradients G; the B selected k x m submatrices are orthogonalized by one batched
    Gram NS.  Returns S [B, k] int32 (and O [B, k, m] in the state's dtype when return_O
    or O is given)."""
    torch = _torch()
    _dev(W)
    if W.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError("W must be bf16, fp16 or fp32")
    dt = dtype_code(W)
    if W.dim() != 3 or W.stride(2) != 1:
        raise ValueError("W must be a [B, N, m] tensor with contiguous rows")
    B, N, m = W.shape
    ld, stride = W.stride(1), W.stride(0)
    for t, name in ((M, "M"), (G, "G")):
        _expect(t, name, dtype=W.dtype, shape=W.shape, device=W.device)
        if t.stride() != W.stride():
            raise ValueError("W, M, G must share their strides")
    cdt = code_of(compute)
    if S is None:
        S = torch.empty((B, k), dtype=torch.int32, device=W.device)
    _expect(S, "S", dtype=torch.int32, shape=(B, k), device=W.device)
    if return_O and O is None:
        O = torch.empty((B, k, m), dtype=W.dtype, device=W.device)
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=(B, k, m), device=W.device)
    if not S.is_contiguous() or (O is not None and not O.is_contiguous()):
        raise ValueError("S and O must be contiguous")
    sched = schedule if schedule is not None else default_schedule()
    ws = _workspace_arg(workspace, lib.dion3_batched_workspace_size(B, N, m, k, dt, cdt), W.device)
    check(lib.dion3_step_batched(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, B, N, m, ld, stride, k, lr,
                                 weight_decay, mu, score_norm, cdt, ctypes.byref(sched), S.data_ptr(),
                                 O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                                 _stream(W.device)), "dion3_step_batched")
    return (S, O) if O is not None else S


def muon_workspace_size(batch, n, m, compute="f16", nesterov=True, dtype="bf16") -> int:
    return int(lib.muon_workspace_size(batch, n, m, code_of(dtype), code_of(compute), 1 if nesterov else 0))


def muon_step(W, M, G, lr, weight_decay=0.0, mu=0.95, nesterov=True, scale=None, compute="f16", schedule=None,
              return_O=False, O=None, workspace=None):
    """One Muon step on the matrices W, M (updated in place) with gradients G, each
    [n, m] or [B, n, m] with contiguous rows and shared strides, all bf16, fp16 or fp32:
    M <- mu M + G; O = GramNS(G + mu M) (nesterov) or GramNS(M); W <- (1 - lr wd) W -
    lr scale O, scale = 0.2 sqrt(max(n, m)) unless given.  Returns O ([.., n, m], the
    state's dtype) when return_O or O is given, else None."""
    torch = _torch()
    _dev(W)
    if W.dtype not in (torch.bfloat16, torch.float16, torch.float32):
        raise ValueError("W must be bf16, fp16 or fp32")
    dt = dtype_code(W)
    if W.dim() not in (2, 3) or W.stride(-1) != 1:
        raise ValueError("W must be an [n, m] or [B, n, m] tensor with contiguous rows")
    W3 = W if W.dim() == 3 else W.unsqueeze(0)
    B, n, m = W3.shape
    ld, stride = W3.stride(1), W3.stride(0)
    for t, name in ((M, "M"), (G, "G")):
        _expect(t, name, dtype=W.dtype, shape=W.shape, device=W.device)
        if t.stride() != W.stride():
            raise ValueError("W, M, G must share their strides")
    cdt = code_of(compute)
    if return_O and O is None:
        O = torch.empty(W.shape, dtype=W.dtype, device=W.device)
    if O is not None:
        _expect(O, "O", dtype=W.dtype, shape=W.shape, device=W.device)
        if not O.is_contiguous():
            raise ValueError("O must be contiguous")
    if scale is not None and not float(scale) > 0.0:
        raise ValueError(f"scale must be positive (None selects 0.2 sqrt(max(n, m))), got {scale}")
    sched = schedule if schedule is not None else default_schedule()
    nest = 1 if nesterov else 0
    ws = _workspace_arg(workspace, lib.muon_workspace_size(B, n, m, dt, cdt, nest), W.device)
    check(lib.muon_step_batched(W.data_ptr(), M.data_ptr(), G.data_ptr(), dt, B, n, m, ld, stride, lr, weight_decay,
                                mu, nest, 0.0 if scale is None else float(scale), cdt, ctypes.byref(sched),
                                O.data_ptr() if O is not None else None, ws.data_ptr(), ws.numel(),
                                _stream(W.device)), "muon_step_batched")
    return O
