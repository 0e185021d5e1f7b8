"""CPU oracle for the fused post-experts boundary -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  The product path
(``reduce_moe_finalize_amd``) never imports, calls or falls back to it, and the
two share no code: only the seeded input generators (``workloads``), which hold
none of the method's arithmetic, serve both.

The oracle is plain NumPy: float64 for the reference values (track A) and an
exact float32-operation emulation for the residual contract (track B).  See
:mod:`oracle.boundary` for the definition and its citations.
"""
from .boundary import (  # noqa: F401
    accumulate_f32,
    accumulate_f64,
    bf16_to_f64,
    evaluate,
    f64_to_bf16,
    moe_finalize_rmsnorm,
    reduce_rmsnorm,
    rms_norm_f64,
    run_case,
    run_case_split,
    shared_scale,
    split_evaluate,
)
