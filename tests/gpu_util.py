"""Helpers for the GPU tests: run the HIP path through the C ABI and compare
with the oracle.  The oracle values are computed here on the host from the
same seeded inputs; nothing flows from the GPU into the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O
import workloads as wk
from workloads.device import upload_anchors, upload_layer

BF16_MAX_ABS = 2e-2     # tolerance fixed for bf16 inputs with fp32 accumulation
BF16_REL_L2 = 5e-3
# fp32 path: each output is a chain of fp32 dot products over <= 512 terms,
# a softmax and fp32 RoPE from an fp64-reduced angle; errors stay ~1e-6
# relative, so 1e-4 absolute / 2e-5 relative leave a wide margin.
F32_MAX_ABS = 1e-4
F32_REL_L2 = 2e-5


class HipEventPool:
    """Raw hipEvent_t handles from the HIP runtime torch loaded."""

    def __init__(self, n: int, timing: bool = True):
        import ctypes
        import torch  # noqa: F401  (loads the runtime)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0 if timing else 2) == 0
            self.handles.append(e.value)

    def close(self) -> None:
        for e in self.handles:
            self.hip.hipEventDestroy(e)
        self.handles = []


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def anchors_for(wl):
    """(GPU anchors, GPU keep, oracle anchors, oracle keep).  For sampler
    workloads each side runs its own sampler on the same mask and seed."""
    import speculative_decoding_draft_amd as sd
    if wl.anchor_source == "given":
        return wl.anchors, wl.keep, wl.anchors, wl.keep
    ga = np.zeros((wl.B, wl.N), np.int32)
    gk = np.zeros((wl.B, wl.N), np.uint8)
    oa = np.zeros((wl.B, wl.N), np.int32)
    ok = np.zeros((wl.B, wl.N), np.uint8)
    for b in range(wl.B):
        ga[b], gk[b] = sd.select_anchors_host(wl.loss_mask[b], wl.N, wl.sampler_seed + b)
        oa[b], ok[b] = O.select_anchors(wl.loss_mask[b], wl.N, wl.sampler_seed + b)
    return ga, gk, oa, ok


def desc_for(wl, softmax_scale=0.0):
    import speculative_decoding_draft_amd as sd
    return sd.make_desc(B=wl.B, S=wl.S, N=wl.N, window=wl.W, n_heads=wl.H, d_latent=wl.D,
                        d_nope=wl.d_c, d_rope=wl.d_r, d_v=wl.d_v, rope_base=wl.rope_base,
                        softmax_scale=softmax_scale, dtype=wl.dtype)


class ForwardRun:
    """Uploads one layer, owns out + workspace, runs the forward."""

    def __init__(self, wl, layer_idx=0, anchors=None, keep=None, guard=0, softmax_scale=0.0,
                 force_generic=False, chunk_blocks=0, one_launch=False):
        import torch
        import speculative_decoding_draft_amd as sd
        self.wl, self.sd, self.torch = wl, sd, torch
        self.desc = desc_for(wl, softmax_scale)
        self.t = upload_layer(wl, layer_idx)
        self.anchors, self.keep = upload_anchors(anchors, keep)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        n_out = wl.B * wl.q_len * wl.H * wl.d_v
        self.guard = guard
        # guard regions around `out` hold NaN canaries
        self.out_full = torch.full((n_out + 2 * guard,), float("nan"), dtype=tdt, device="cuda")
        self.out = self.out_full[guard:guard + n_out].view(wl.B, wl.q_len, wl.H, wl.d_v)
        ws = sd.workspace_size(self.desc)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")
        self.force_generic = force_generic
        self.chunk_blocks = chunk_blocks
        self.one_launch = one_launch

    def run(self, stream=None):
        t = self.t
        self.sd.attn_fwd(self.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"],
                         t["ckv_blk"], t["kr_blk"], t["w_uk"], t["w_uv"], self.anchors, self.keep,
                         self.out, self.ws, stream=stream, force_generic=self.force_generic,
                         chunk_blocks=self.chunk_blocks, one_launch=self.one_launch)
        return self

    def result(self) -> np.ndarray:
        self.torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype(np.float64)

    def guards_intact(self) -> bool:
        if self.guard == 0:
            return True
        g = self.guard
        head = self.out_full[:g].float().cpu().numpy()
        tail = self.out_full[-g:].float().cpu().numpy()
        return bool(np.all(np.isnan(head)) and np.all(np.isnan(tail)))


def compare(gpu: np.ndarray, ref: np.ndarray, keep: np.ndarray, max_abs: float, rel_l2: float,
            what: str = "") -> dict:
    """Rows of padding blocks must be exactly 0 on the GPU and are excluded;
    rows the reference did not compute (NaN) are skipped; the rest must match
    within max_abs and rel-L2."""
    B, L5 = gpu.shape[:2]
    kept_rows = np.repeat(keep.astype(bool), 5, axis=1)           # [B, 5N]
    pad = gpu[~kept_rows]
    assert np.all(pad == 0), f"{what}: padding rows are not zero"
    checked = kept_rows[:, :, None, None] & np.isfinite(ref)
    assert checked.any(), f"{what}: nothing compared"
    g, r = gpu[checked], ref[checked]
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output in kept rows"
    err = np.abs(g - r)
    stats = dict(max_abs=float(err.max()), rel_l2=float(np.linalg.norm(g - r) / np.linalg.norm(r)),
                 n=int(g.size))
    log(f"  {what}: max_abs={stats['max_abs']:.3e} rel_l2={stats['rel_l2']:.3e} n={stats['n']}")
    assert stats["max_abs"] <= max_abs, f"{what}: max_abs {stats['max_abs']} > {max_abs}"
    assert stats["rel_l2"] <= rel_l2, f"{what}: rel_l2 {stats['rel_l2']} > {rel_l2}"
    return stats


def sample_blocks(keep_row: np.ndarray, anchors_row: np.ndarray, W: int, n_random: int, seed: int):
    """Kept blocks to check at full size: every clamped-window block
    (A < W-1) plus n_random others."""
    kept = np.nonzero(keep_row)[0]
    clamped = [int(n) for n in kept if anchors_row[n] < W - 1]
    rest = [int(n) for n in kept if anchors_row[n] >= W - 1]
    rng = np.random.default_rng(seed)
    pick = rng.choice(rest, size=min(n_random, len(rest)), replace=False).tolist() if rest else []
    return sorted(set(clamped + pick + ([rest[0], rest[-1]] if rest else [])))


def context_of_two(seed):
    """The shortest context a block can have: S = 2, so A = 0 is the only valid
    anchor and every block sees only its own 5 keys.  Several kept blocks of a
    sample share that anchor (repeated anchors are valid input), with padding
    between them; odd N, B = 2, GLM dims (the MFMA path)."""
    wl = wk.make_workload("ctx2", B=2, S=2, N=5, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="sampler", seed=seed)
    wl.anchor_source = "given"
    wl.anchors = np.zeros((2, 5), np.int32)
    wl.keep = np.array([[1, 1, 0, 1, 1], [0, 1, 1, 0, 1]], np.uint8)
    wl.anchors[0, 2] = -9                   # padding slot: its anchor is never read
    wl.loss_mask[:, :] = 1
    return wl


def repeated_anchors(seed):
    """Kept anchors drawn with replacement (about a third of them repeat an
    earlier one), sorted, with a tenth of the slots padding and a few clamped
    windows: at S = 640 and N = 200 enough kept blocks for the attention's
    one-block-per-workgroup launch, and for runs of equal anchors in the
    backward's per-row sums over covering blocks."""
    wl = wk.make_workload("dup", B=1, S=640, N=200, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=seed)
    rng = np.random.default_rng(seed)
    a = np.sort(rng.integers(0, wl.S - 1, size=wl.N)).astype(np.int32)
    a[:4] = [0, 0, 5, 126]
    a = np.sort(a)
    keep = (rng.random(wl.N) >= 0.1).astype(np.uint8)
    a[keep == 0] = -1                        # padding: garbage anchors, never read
    wl.anchors, wl.keep = a[None, :], keep[None, :]
    wl.loss_mask[:, :] = 1
    return wl
