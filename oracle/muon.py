"""Muon optimizer step, written from the pages.  TEST INFRASTRUCTURE ONLY.

Source: "Muon: Orthogonalized Momentum and Why It Trains LLMs 2x Cheaper" (blog by
M. Chugh), the step listed after "Doing an SVD without an SVD" and the two practical
notes that follow it (decoupled weight decay, per-parameter update-scale matching):
  * heavy-ball momentum:   M <- mu M + G
  * Nesterov lookahead:    U = G + mu M   (with the updated M); plain: U = M
  * orthogonalise:         O = NS(U)       (quintic Newton-Schulz, the blog's iteration)
  * RMS matching:          scale = 0.2 sqrt(max(d_out, d_in))
  * decoupled decay first, then the update:  W <- (1 - lr wd) W - lr scale O
The Dion3 pages state that Dion3 with f = 1 is this step ("Dion3: Full-Stack
Orthogonal Updates", m.montaan.com; "Dion3：全栈正交更新", paper.rainbus.top,
核心方法), which pins the momentum recursion and the update below.

Storage model (the pages leave rounding open; this is the reading the GPU path
follows, the same as for the Dion3 step): W, M, G are stored in one format, the
caller's state dtype (bf16, f16 or f32), and every stored result is rounded once to
it (nearest, ties to even) from float32 arithmetic carried out op by op (numpy
float32, no fused multiply-add).  O is stored in the state format before the update
reads it.  The scale is fl32(fl32(0.2) * fl32(sqrt(max(n, m)))).

Storage modes: "bf16" (uint16 bit patterns), "f16" and "f32" (numpy float16 /
float32 arrays), all with the model above, and "f64" (no rounding anywhere, used to
pin the step against Dion3 with f = 1).

Parity status: momentum pinned by exact dyadic cases against its closed form and by
the f = 1 identity; muon_scale by the page's formula at shapes where it is exact;
muon_step by the f = 1 identity (float64), the zero-gradient decay closed form and
the Newton-Schulz oracle on U.
"""
from __future__ import annotations

import numpy as np

from .dion3 import _codec
from .newton_schulz import newton_schulz, JORDAN_ABC, EPS


def muon_scale(n: int, m: int) -> np.float32:
    """0.2 sqrt(max(n, m)) in float32: the update RMS matched to AdamW's."""
    return np.float32(np.float32(0.2) * np.sqrt(np.float32(max(n, m))))


def momentum(m, g, mu, nesterov=True, storage="bf16"):
    """M' = fl(fl32(fl32(mu) M) + G); U = fl(G + fl32(mu M')) with the lookahead, else
    U = M' (fl: one rounding to the state format).  Returns (M', U) as stored values."""
    dec, enc = _codec(storage)
    mu32 = np.float32(mu)
    m32 = dec(m).astype(np.float32)
    g32 = dec(g).astype(np.float32)
    m_new = enc(((mu32 * m32) + g32).astype(np.float64))
    if not nesterov:
        return m_new, m_new
    mn32 = dec(m_new).astype(np.float32)
    u = enc((g32 + (mu32 * mn32)).astype(np.float64))
    return m_new, u


def decay_and_update(w, o, lr, wd, scale, storage="bf16"):
    """W' = fl( fl32( fl32(d W) - fl32(fl32(lr scale) O) ) ), d = fl32(1 - fl32(lr wd));
    o: the update (float values as stored, e.g. in the state format)."""
    dec, enc = _codec(storage)
    lr32, wd32, sc32 = np.float32(lr), np.float32(wd), np.float32(scale)
    d = np.float32(np.float32(1.0) - lr32 * wd32)
    lre = np.float32(lr32 * sc32)
    w32 = dec(w).astype(np.float32)
    o32 = np.asarray(o, dtype=np.float64).astype(np.float32)
    return enc(((d * w32) - (lre * o32)).astype(np.float64))


def _arith(storage):
    """(number type, store) of a storage mode: "bf16", "f16" and "f32" round every
    stored value once to the format from float32 arithmetic; "f64" keeps float64
    values and rounds nothing."""
    if storage in ("bf16", "f16", "f32"):
        dec, enc = _codec(storage)
        return np.float32, lambda v: dec(enc(np.asarray(v, np.float64)))
    if storage == "f64":
        return np.float64, lambda v: np.asarray(v, np.float64)
    raise ValueError(storage)


def muon_step(w, m, g, lr, wd=0.0, mu=0.95, nesterov=True, scale=None, steps=5, abc=JORDAN_ABC, eps=EPS,
              storage="bf16", orthogonalize=None):
    """One Muon step on one matrix.  Returns (W', M', O) with O the orthogonalised
    update in float64.

    storage="bf16": w, m, g are uint16 bf16 bit patterns, results likewise;
    storage="f16" / "f32": numpy float16 / float32 arrays, results likewise;
    storage="f64":  w, m, g are float64 arrays and nothing is rounded.
    scale: None for 0.2 sqrt(max(n, m)).
    orthogonalize: function U -> O (default: standard Newton-Schulz).

    Both modes run the same sequence: the momentum recursion and its lookahead, the
    orthogonalised direction, then the decayed weights minus the scaled direction,
    each formed in the mode's number type and stored through the mode's rounding."""
    ortho = orthogonalize or (lambda x: newton_schulz(x, steps, abc, eps))
    num, store = _arith(storage)
    n, mm = np.asarray(m).shape
    if storage != "f64":
        dec, enc = _codec(storage)
        W, Mo, Gr = (dec(v).astype(num) for v in (w, m, g))
        sc = muon_scale(n, mm) if scale is None else num(scale)
    else:
        W, Mo, Gr = (np.asarray(v, np.float64) for v in (w, m, g))
        sc = 0.2 * np.sqrt(max(n, mm)) if scale is None else num(scale)
    mu_t, lr_t, wd_t = num(mu), num(lr), num(wd)
    m_new = store(mu_t * Mo + Gr).astype(num)
    direction = store(Gr + mu_t * m_new).astype(num) if nesterov else m_new
    O = ortho(np.asarray(direction, np.float64))
    o_stored = store(O).astype(num)
    keep = num(1) - lr_t * wd_t
    step = num(lr_t * num(sc))
    w_new = store(keep * W - step * o_stored)
    if storage != "f64":
        return enc(w_new), enc(m_new.astype(np.float64)), O
    return w_new, np.asarray(m_new, np.float64), O
