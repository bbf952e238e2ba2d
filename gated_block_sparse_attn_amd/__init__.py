"""MI355X (gfx950) gated block-sparse attention (SAS) -- HIP library + binding.

The computation lives in libsas.so (include/sas.h); this package only loads it
and marshals torch tensors to the C ABI.
"""

from .api import (  # noqa: F401
    Problem,
    SASAttention,
    SasError,
    abi_version,
    bwd_workspace_size,
    gate_threshold,
    gated_attn_bwd,
    gated_attn_fwd,
    sas_attention,
)
