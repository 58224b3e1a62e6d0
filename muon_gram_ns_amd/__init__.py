"""MI355X-native Gram Newton-Schulz and Dion3 hot path.

The computation lives in libgns.so (hand-written HIP kernels for gfx950 behind a
C ABI declared in include/gns.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    lib, LIB_PATH, GnsError, Schedule, default_schedule, header_functions,
    GNS_BF16, GNS_F16, GNS_F32, orthogonalize, orthogonalize_noalloc, newton_schulz, frobenius_scale, symm_gemm,
    rect_gemm, dion3_accumulate_score, dion3_select_topk, dion3_gather_feedback,
    dion3_apply_update, dion3_step, dion3_step_batched, dion3_step_rows,
    dion3_step_dev_scalars, dion3_step_cols, muon_step, muon_workspace_size, workspace, workspace_size,
)
from . import flops  # noqa: F401
from .graphs import (  # noqa: F401
    Graphed, graphed_orthogonalize, graphed_newton_schulz, graphed_dion3_step, graphed_muon_step,
)
