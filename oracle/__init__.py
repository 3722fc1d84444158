"""Float64 CPU oracle for multi-scale retention (MSR).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares
no code with the HIP library and imports nothing from it.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, exact rational brute force, the pages' stated
equivalences between the three forms, and GroupNorm scale invariance.  No
function is "parity unpinned".
"""
from .retention import (  # noqa: F401
    rotary,
    decay_mask,
    retention_parallel,
    retention_recurrent,
    retention_chunkwise,
    retention_bruteforce,
    retention_parallel_normalized,
    recurrent_step,
    group_norm_heads,
    swish,
    msr_layer,
    msr_layer_decode_step,
    layer_norm,
    gelu,
    retnet_block,
    rotary_adjoint,
    retention_grad,
    log_sigmoid,
    rglru,
    max_rel_err,
    max_rel_err_per_head,
)
