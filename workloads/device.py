"""Copy a generated workload to GPU memory as torch tensors (plumbing only).

bf16 arrays are raw uint16 bit patterns on the host; they are reinterpreted
as torch.bfloat16 without any conversion.
"""
from __future__ import annotations

import numpy as np

LAYER_FIELDS = ("q_nope", "q_rope", "ckv_ctx", "kr_ctx", "ckv_blk", "kr_blk", "w_uk", "w_uv")


def to_torch(a: np.ndarray, dtype: str, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(device)


def upload_layer(wl, layer_idx: int = 0, device="cuda") -> dict:
    layer = wl.layers[layer_idx]
    return {f: to_torch(getattr(layer, f), wl.dtype, device) for f in LAYER_FIELDS}


def upload_anchors(anchors: np.ndarray, keep: np.ndarray, device="cuda"):
    import torch
    a = torch.from_numpy(np.ascontiguousarray(anchors, dtype=np.int32)).to(device)
    k = torch.from_numpy(np.ascontiguousarray(keep, dtype=np.uint8)).to(device)
    return a, k


def upload_loss(lh, loss_mask: np.ndarray, anchors: np.ndarray, keep: np.ndarray,
                device="cuda") -> dict:
    """The loss head's inputs as device tensors, keyed as the binding's
    LOSS_INPUTS."""
    import torch
    t = {k: to_torch(getattr(lh, k), lh.dtype, device)
         for k in ("h_final", "z", "w_lm", "w_m1", "w_m2", "w_conf")}
    t["input_ids"] = torch.from_numpy(np.ascontiguousarray(lh.input_ids, dtype=np.int32)).to(device)
    t["loss_mask"] = torch.from_numpy(np.ascontiguousarray(loss_mask, dtype=np.uint8)).to(device)
    t["anchors"], t["keep"] = upload_anchors(anchors, keep, device)
    return t
