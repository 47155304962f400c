"""fp64 CPU oracle for the GLM-5.2 DSpark draft-attention forward and its
backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code with it; the two meet only in the seeded input
generator (``workloads``), which holds none of the method's arithmetic.

Every function cites the passage of the design page it follows ("GLM 5.2
DSpark 投机训练设计", the DSpark training-design page).  Parity status of each
function is listed in the module docstrings; the only unpinned part is the
numerical value of a real trained GLM-5.2 layer (no weights exist here).
"""
from .dspark_oracle import (  # noqa: F401
    bf16_to_f64,
    candidates,
    select_anchors,
    SplitMix64,
    positions,
    build_mask,
    mask_rows,
    rope_interleaved,
    rope_theta,
    expand_head,
    attend_dense,
    softmax_scale,
    attend_gathered,
    forward,
    forward_absorbed,
    block_index_records,
    row_index_sets,
    rope_interleaved_transpose,
    backward,
    loss,
    rmsnorm,
    layer_forward,
    LOSS_ALPHAS,
    eval_mask,
    draft_logits,
    teacher_logits,
    confidence_logit,
    step_terms,
    loss_head,
    ring_slot,
    decode_attention,
    softmax_t,
    acceptance,
    sample_inverse_cdf,
    spec_verify,
)
