"""MI355X (gfx950) DSpark draft attention (forward, backward), the MLA block
of a draft layer around it, and the draft's output head and loss.

The compute lives in libdspark_attn.so (hand-written HIP kernels behind the C
ABI of include/dspark_attn.h); this package is its Python binding.  Build the
library with ``python speculative_decoding_draft_amd/build.py``.
"""
from ._lib import (  # noqa: F401
    DSPARK_BF16,
    DSPARK_EANCHOR,
    DSPARK_ECAPACITY,
    DSPARK_EHIP,
    DSPARK_EINVAL,
    DSPARK_EUNSUPPORTED,
    DSPARK_EWORKSPACE,
    DSPARK_F32,
    DSPARK_OK,
    BoundFwd,
    EXPORTS,
    LIB_PATH,
    Desc,
    DSparkError,
    abi_version,
    attn_plan,
    attn_fwd,
    attn_bwd,
    bwd_plan,
    bwd_workspace_size,
    BWD_GRADS,
    LayerDesc,
    LAYER_WEIGHTS,
    make_layer_desc,
    layer_workspace_size,
    mla_layer_fwd,
    mla_layer_tune,
    LossDesc,
    LOSS_INPUTS,
    make_loss_desc,
    loss_workspace_size,
    loss_fwd,
    loss_tune,
    loss_read_status,
    build_index,
    last_error,
    make_desc,
    read_device_status,
    select_anchors_host,
    workspace_size,
)
