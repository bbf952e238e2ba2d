"""CPU oracle for SAS gated block-sparse attention.

Test infrastructure only: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.  The training
path (gates, forward, backward) is in ``sas_oracle``; the sparse decode step
(per-group Top-K and attention over the gathered blocks) in
``sas_decode_oracle``.
"""

from .sas_oracle import (  # noqa: F401
    backward,
    backward_kv_block,
    dense_backward,
    dense_bias,
    dense_forward,
    default_scale,
    dscores,
    forward,
    gate_threshold,
    kth_largest_threshold,
)
