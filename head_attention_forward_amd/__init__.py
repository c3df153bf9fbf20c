"""Multi-head scaled dot-product attention, forward, on AMD MI355X (gfx950).

The computation lives in ``libmha.so`` (HIP kernels behind a C ABI declared
in ``include/mha.h``); this package is its Python binding plus the seeded
synthetic workloads used by the tests and the bench.
"""

from ._binding import (  # noqa: F401
    LAYER_PARAMS,
    MHAError,
    add_layernorm_forward,
    embed_positional_forward,
    encoder_layer_forward,
    encoder_layer_workspace_bytes,
    ffn_forward,
    alloc_workspace,
    lib,
    mha_attend,
    mha_backward,
    mha_forward,
    mha_forward_train,
    mha_project_in,
    mha_project_out,
    sdpa_backward,
    sdpa_decode,
    sdpa_forward,
    sdpa_forward_lse,
    workspace_bytes,
    workspace_views,
)
from .workloads import (  # noqa: F401
    MASK_CAUSAL,
    MASK_CAUSAL_KEY_PADDING,
    MASK_KEY_PADDING,
    MASK_NONE,
    WORKLOADS,
    Workload,
    generate,
)
