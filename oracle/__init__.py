"""Float64 CPU oracle for the CfC K-loop (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``cfc_recurrent_cell_amd``)
never imports it and fails loudly when its HIP library is missing.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    load_oracle,
    scratch_row_len,
    cfc_forward,
    cfc_backward,
    reduce_axis0,
    reduce_axis0_f32,
    cfc_step,
)
