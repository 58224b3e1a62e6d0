"""CPU oracle for the Gram Newton-Schulz / Dion3 hot path.  TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import or
call anything in this package.  The product path (the HIP library and its Python
binding) never imports it, and this package never imports the product path: the two
share no code.  The only common dependency is the seeded input module `synth`,
which holds none of the method's arithmetic.

Everything here is plain, slow and written to be checked by eye against the pages:
numpy in float64, library matmul as the only "kernel", no blocking, fusion or
reordering beyond what the written algorithm states.

Sources (pages on the Dion3 / Muon method):
  * "Muon: Orthogonalized Momentum and Why It Trains LLMs 2x Cheaper" (blog by
    M. Chugh), section "Doing an SVD without an SVD": the quintic Newton-Schulz
    iteration, its coefficients, Frobenius normalisation with eps, transposition to
    the short side.
  * "Dion3：全栈正交更新 Dion3: Full-Stack Orthogonal Updates" (paper.rainbus.top
    summary), sections 核心方法 (core method: theorem 2, the scalar recursion behind
    Gram NS) and 方法步骤详情 (method steps: Algorithm 3 = stabilised Gram NS with a
    restart, Algorithm 4 = the Dion3 row-subsampled update with error feedback);
    section 前置知识 (prerequisites: polar factor, error feedback).
  * "Dion3: Full-Stack Orthogonal Updates" (m.montaan.com summary): f = 1 is Muon.
  * The Muon blog named first above: the Muon step listed after "Doing an SVD
    without an SVD" and its notes on decoupled weight decay and update-scale
    matching (oracle/muon.py).

Parity status of each function is stated in its docstring; "parity unpinned" marks
a function with no independent pin.
"""
from .bf16 import bf16_to_f64, f64_to_bf16_rne, f32_round  # noqa: F401
from .newton_schulz import (  # noqa: F401
    JORDAN_ABC, EPS, quintic, quintic_composed, normalize, newton_schulz,
    gram_newton_schulz, gram_newton_schulz_schedule,
)
from .gemm import symm_gemm_ref, rect_gemm_ref  # noqa: F401
from .dion3 import (  # noqa: F401
    k_from_fraction, accumulate, row_scores, select_topk, gather_rows, error_feedback, weight_update,
    dion3_step, dion3_step_rows, dion3_step_cols,
)
from .muon import muon_scale, momentum, decay_and_update, muon_step  # noqa: F401
