"""Float64 CPU oracle for the fused linear cross-entropy engine.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` and by nothing else.  It shares no
code with the HIP library in ``lm_head_linear_flce_amd/``; neither imports the
other.  Every function follows the plain definition of the loss and its
gradients; see ``flce_ref`` for the passages each one follows.
"""
from .flce_ref import (  # noqa: F401
    targets, flce, forward_rows, dx_rows, dw_rows, round_bf16_f64,
    logits_bytes, cosine,
)
