"""ctypes binding of libdspark_attn.so (argument marshalling only).

Every function mirrors an ``extern "C"`` entry point of
``include/dspark_attn.h``; tensors are torch tensors that live on the GPU
(torch supplies device memory and the current HIP stream), except where the
header says "host".  Nothing here computes any part of the forward or the
backward; if the
library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark_attn.so")

DSPARK_OK = 0
DSPARK_EINVAL = -1
DSPARK_EUNSUPPORTED = -2
DSPARK_EWORKSPACE = -3
DSPARK_EHIP = -4
DSPARK_EANCHOR = -5
DSPARK_ECAPACITY = -6
STATUS_NAMES = {0: "DSPARK_OK", -1: "DSPARK_EINVAL", -2: "DSPARK_EUNSUPPORTED",
                -3: "DSPARK_EWORKSPACE", -4: "DSPARK_EHIP", -5: "DSPARK_EANCHOR",
                -6: "DSPARK_ECAPACITY"}
DSPARK_F32 = 0
DSPARK_BF16 = 1

EXPORTS = ("dspark_attn_workspace_size", "dspark_attn_workspace_size_ex", "dspark_attn_fwd", "dspark_attn_fwd_ex", "dspark_attn_fwd_noalloc", "dspark_attn_plan",
           "dspark_attn_bwd_workspace_size", "dspark_attn_bwd", "dspark_attn_bwd_ex",
           "dspark_attn_bwd_plan", "dspark_mla_layer_workspace_size", "dspark_mla_layer_fwd",
           "dspark_mla_layer_fwd_ex", "dspark_mla_layer_tune", "dspark_mla_layer_read_status", "dspark_loss_workspace_size",
           "dspark_loss_fwd", "dspark_loss_fwd_ex", "dspark_loss_tune", "dspark_loss_read_status",
           "dspark_cache_append", "dspark_decode_workspace_size", "dspark_decode_attn",
           "dspark_verify_workspace_size", "dspark_spec_verify",
           "dspark_build_index",
           "dspark_select_anchors_host",
           "dspark_read_device_status", "dspark_last_error", "dspark_abi_version")


class DSparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("N", ctypes.c_int32),
                ("block", ctypes.c_int32), ("window", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("d_latent", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_double),
                ("dtype", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("attn", Desc), ("hidden", ctypes.c_int32), ("q_rank", ctypes.c_int32),
                ("rms_eps", ctypes.c_double), ("max_kept_blocks", ctypes.c_int32)]


class LossDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("N", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("markov_rank", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("max_kept_blocks", ctypes.c_int32), ("alpha_ce", ctypes.c_double),
                ("alpha_l1", ctypes.c_double), ("alpha_conf", ctypes.c_double),
                ("w_lm_ld", ctypes.c_int32), ("w_m2_ld", ctypes.c_int32),
                ("max_counted_steps", ctypes.c_int32)]


class DecodeDesc(ctypes.Structure):
    _fields_ = [("attn", Desc), ("cache_slots", ctypes.c_int32)]


class VerifyDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("K", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("temperature", ctypes.c_double)]


MAX_GEMMS = 8
BLAS_WORKSPACE_BYTES = 64 << 20


class GemmChoice(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("solution", ctypes.c_int32)]


class GemmChoices(ctypes.Structure):
    """dspark_gemm_choices: the rocBLAS kernel choice of each GEMM of one MLA
    block or loss call, filled by mla_layer_tune / loss_tune (caller-owned)."""
    _fields_ = [("n_gemms", ctypes.c_int32), ("gemm", GemmChoice * MAX_GEMMS)]

    def as_list(self):
        return [(g.m, g.n, g.k, g.solution) for g in self.gemm[:self.n_gemms]]


class Opts(ctypes.Structure):
    _fields_ = [("stage_events", ctypes.POINTER(ctypes.c_void_p)),
                ("n_stage_events", ctypes.c_int32), ("force_generic", ctypes.c_int32),
                ("chunk_blocks", ctypes.c_int32), ("aux_stream", ctypes.c_void_p),
                ("aux_events", ctypes.c_void_p * 2), ("reuse_forward", ctypes.c_int32),
                ("one_launch", ctypes.c_int32),
                ("gemm_choices", ctypes.POINTER(GemmChoices))]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python speculative_decoding_draft_amd/build.py`")
    # torch must bring in its HIP runtime (soname libamdhip64.so.7) first, so
    # that the library binds to that one instance: torch owns the device
    # memory and streams passed in, and a second runtime in the process would
    # not see the device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t
    pd = ctypes.POINTER(Desc)
    lib.dspark_attn_workspace_size.argtypes = [pd]
    lib.dspark_attn_workspace_size.restype = sz
    lib.dspark_attn_workspace_size_ex.argtypes = [pd, ctypes.POINTER(Opts)]
    lib.dspark_attn_workspace_size_ex.restype = sz
    fwd_args = [pd] + [vp] * 8 + [vp, vp, vp, vp, sz, vp]
    lib.dspark_attn_fwd.argtypes = fwd_args
    lib.dspark_attn_fwd.restype = i32
    lib.dspark_attn_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(Opts)]
    lib.dspark_attn_fwd_ex.restype = i32
    lib.dspark_attn_fwd_noalloc.argtypes = [pd] + [vp] * 8 + [vp, vp, vp, vp, vp]
    lib.dspark_attn_fwd_noalloc.restype = i32
    lib.dspark_attn_plan.argtypes = [pd, ctypes.POINTER(Opts)] + [ctypes.POINTER(i32)] * 3
    lib.dspark_attn_plan.restype = i32
    lib.dspark_attn_bwd_workspace_size.argtypes = [pd]
    lib.dspark_attn_bwd_workspace_size.restype = sz
    bwd_args = [pd] + [vp] * 8 + [vp, vp, vp] + [vp] * 8 + [vp, sz, vp]
    lib.dspark_attn_bwd.argtypes = bwd_args
    lib.dspark_attn_bwd.restype = i32
    lib.dspark_attn_bwd_ex.argtypes = bwd_args + [ctypes.POINTER(Opts)]
    lib.dspark_attn_bwd_ex.restype = i32
    lib.dspark_attn_bwd_plan.argtypes = [pd, ctypes.POINTER(Opts), ctypes.POINTER(i32)]
    lib.dspark_attn_bwd_plan.restype = i32
    pl = ctypes.POINTER(LayerDesc)
    lib.dspark_mla_layer_workspace_size.argtypes = [pl]
    lib.dspark_mla_layer_workspace_size.restype = sz
    layer_args = [pl] + [vp] * 11 + [vp, vp, vp, vp, sz, vp]
    lib.dspark_mla_layer_fwd.argtypes = layer_args
    lib.dspark_mla_layer_fwd.restype = i32
    lib.dspark_mla_layer_fwd_ex.argtypes = layer_args + [ctypes.POINTER(Opts)]
    lib.dspark_mla_layer_fwd_ex.restype = i32
    lib.dspark_mla_layer_tune.argtypes = layer_args + [ctypes.POINTER(GemmChoices)]
    lib.dspark_mla_layer_tune.restype = i32
    lib.dspark_mla_layer_read_status.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.dspark_mla_layer_read_status.restype = i32
    plo = ctypes.POINTER(LossDesc)
    lib.dspark_loss_workspace_size.argtypes = [plo]
    lib.dspark_loss_workspace_size.restype = sz
    loss_args = [plo] + [vp] * 10 + [vp, vp, vp, vp, sz, vp]
    lib.dspark_loss_fwd.argtypes = loss_args
    lib.dspark_loss_fwd.restype = i32
    lib.dspark_loss_fwd_ex.argtypes = loss_args + [ctypes.POINTER(Opts)]
    lib.dspark_loss_fwd_ex.restype = i32
    lib.dspark_loss_tune.argtypes = loss_args + [ctypes.POINTER(GemmChoices)]
    lib.dspark_loss_tune.restype = i32
    lib.dspark_loss_read_status.argtypes = [vp, vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                            ctypes.POINTER(i32)]
    lib.dspark_loss_read_status.restype = i32
    pdd = ctypes.POINTER(DecodeDesc)
    lib.dspark_cache_append.argtypes = [pdd, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.dspark_cache_append.restype = i32
    lib.dspark_decode_workspace_size.argtypes = [pdd]
    lib.dspark_decode_workspace_size.restype = sz
    lib.dspark_decode_attn.argtypes = [pdd] + [vp] * 11 + [vp, sz, vp]
    lib.dspark_decode_attn.restype = i32
    pvd = ctypes.POINTER(VerifyDesc)
    lib.dspark_verify_workspace_size.argtypes = [pvd]
    lib.dspark_verify_workspace_size.restype = sz
    lib.dspark_spec_verify.argtypes = [pvd] + [vp] * 8 + [vp, sz, vp]
    lib.dspark_spec_verify.restype = i32
    lib.dspark_build_index.argtypes = [pd, vp, vp, vp, vp, sz, vp]
    lib.dspark_build_index.restype = i32
    lib.dspark_select_anchors_host.argtypes = [vp, i32, i32, u64, vp, vp]
    lib.dspark_select_anchors_host.restype = i32
    lib.dspark_read_device_status.argtypes = [vp, vp, ctypes.POINTER(i32)]
    lib.dspark_read_device_status.restype = i32
    lib.dspark_last_error.argtypes = []
    lib.dspark_last_error.restype = ctypes.c_char_p
    lib.dspark_abi_version.argtypes = []
    lib.dspark_abi_version.restype = i32
    return lib


lib = _load()


def last_error() -> str:
    return lib.dspark_last_error().decode()


def abi_version() -> int:
    return int(lib.dspark_abi_version())


def _check(status: int) -> None:
    if status != DSPARK_OK:
        raise DSparkError(status, last_error())


def make_desc(*, B, S, N, window, n_heads, d_latent, d_nope, d_rope, d_v, rope_base=10000.0,
              softmax_scale=0.0, dtype="bf16", block=5) -> Desc:
    dt = {"bf16": DSPARK_BF16, "f32": DSPARK_F32}.get(dtype, dtype)
    return Desc(B, S, N, block, window, n_heads, d_latent, d_nope, d_rope, d_v,
                float(rope_base), float(softmax_scale), int(dt))


def workspace_size(desc: Desc) -> int:
    n = int(lib.dspark_attn_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


def workspace_size_ex(desc: Desc, force_generic: bool = False, chunk_blocks: int = 0,
                      one_launch: bool = False, for_backward: bool = False) -> int:
    """dspark_attn_workspace_size_ex: bytes for the path these options select."""
    opts, _ = _opts(None, force_generic, chunk_blocks, one_launch=one_launch)
    opts.reuse_forward = 1 if for_backward else 0
    n = int(lib.dspark_attn_workspace_size_ex(ctypes.byref(desc), ctypes.byref(opts)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _opts(stage_events=None, force_generic=False, chunk_blocks=0, aux_stream=None,
          aux_events=None, one_launch=False):
    opts = Opts()
    opts.one_launch = 1 if one_launch else 0
    if aux_stream is not None:
        opts.aux_stream = _stream(aux_stream)
        opts.aux_events[0], opts.aux_events[1] = aux_events
    keep = None
    if stage_events is not None:
        keep = (ctypes.c_void_p * len(stage_events))(*stage_events)
        opts.stage_events = ctypes.cast(keep, ctypes.POINTER(ctypes.c_void_p))
        opts.n_stage_events = len(stage_events)
    opts.force_generic = 1 if force_generic else 0
    opts.chunk_blocks = int(chunk_blocks)
    return opts, keep


def attn_plan(desc: Desc, force_generic: bool = False, chunk_blocks: int = 0,
              one_launch: bool = False):
    """dspark_attn_plan: (n_chunks, chunk_blocks, n_events)."""
    opts, _ = _opts(None, force_generic, chunk_blocks, one_launch=one_launch)
    nc, cb, ne = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.dspark_attn_plan(ctypes.byref(desc), ctypes.byref(opts), ctypes.byref(nc),
                                ctypes.byref(cb), ctypes.byref(ne)))
    return nc.value, cb.value, ne.value


def attn_fwd(desc: Desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
             anchors, keep, out, workspace, stream=None,
             stage_events: Optional[Sequence[int]] = None, force_generic: bool = False,
             chunk_blocks: int = 0, aux_stream=None,
             aux_events: Optional[Sequence[int]] = None,
             one_launch: bool = False, for_backward: bool = False) -> None:
    """dspark_attn_fwd / dspark_attn_fwd_ex; raises DSparkError on a non-OK
    status.  aux_stream / aux_events (two hipEvent_t handles) run odd rounds
    on a second stream; one_launch selects the one-launch forward;
    for_backward (opts.reuse_forward on a forward): workspace is a
    backward's, and the forward also leaves its softmax probabilities there
    for a backward with reuse_forward=2 (see dspark_attn_opts)."""
    args = [ctypes.byref(desc)] + [_ptr(t) for t in (q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk,
                                                     kr_blk, w_uk, w_uv, anchors, keep, out,
                                                     workspace)]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args += [ws_bytes, _stream(stream)]
    if (stage_events is None and not force_generic and not chunk_blocks and aux_stream is None
            and not one_launch and not for_backward):
        _check(lib.dspark_attn_fwd(*args))
        return
    opts, _arr = _opts(stage_events, force_generic, chunk_blocks, aux_stream, aux_events,
                       one_launch)
    opts.reuse_forward = 1 if for_backward else 0
    _check(lib.dspark_attn_fwd_ex(*args, ctypes.byref(opts)))


STATUS_BYTES = 64
NOALLOC_SCRATCH_BYTES = 64 << 20


def attn_fwd_noalloc(desc: Desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                     anchors, keep, out, status=None, stream=None) -> None:
    """dspark_attn_fwd_noalloc: the forward in the library's fixed per-device
    scratch array (no workspace).  status: None or a device tensor of at
    least STATUS_BYTES that receives the status words (read it with
    read_device_status)."""
    if status is not None:
        assert status.numel() * status.element_size() >= STATUS_BYTES
    args = [ctypes.byref(desc)] + [_ptr(t) for t in (q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk,
                                                     kr_blk, w_uk, w_uv, anchors, keep, out,
                                                     status)]
    _check(lib.dspark_attn_fwd_noalloc(*args, _stream(stream)))


class BoundFwd:
    """dspark_attn_fwd with its arguments marshalled once, for callers that
    issue the same call many times (a training loop, a benchmark).  The
    tensors must stay alive and in place while the object is used."""

    def __init__(self, desc: Desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                 anchors, keep, out, workspace, stream=None, chunk_blocks: int = 0,
                 n_stage_events: int = 0, aux_stream=None,
                 aux_events: Optional[Sequence[int]] = None, one_launch: bool = False):
        self._desc = desc
        ws_bytes = workspace.numel() * workspace.element_size()
        self._args = (ctypes.byref(desc),) + tuple(
            ctypes.c_void_p(_ptr(t)) for t in (q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk,
                                                w_uk, w_uv, anchors, keep, out, workspace)) + (
            ctypes.c_size_t(ws_bytes), ctypes.c_void_p(_stream(stream)))
        self._plain = lib.dspark_attn_fwd
        self._ex = lib.dspark_attn_fwd_ex
        self._opts, _ = _opts(None, False, chunk_blocks, aux_stream, aux_events,
                              one_launch)
        self._opts_ref = ctypes.byref(self._opts)
        self._events = (ctypes.c_void_p * max(1, n_stage_events))()
        self._opts_ev, _ = _opts(None, False, chunk_blocks, aux_stream, aux_events,
                                 one_launch)
        self._opts_ev.stage_events = ctypes.cast(self._events, ctypes.POINTER(ctypes.c_void_p))
        self._opts_ev.n_stage_events = n_stage_events
        self._opts_ev_ref = ctypes.byref(self._opts_ev)

    def __call__(self) -> None:
        st = self._ex(*self._args, self._opts_ref)
        if st != DSPARK_OK:
            _check(st)

    def with_events(self, events: Sequence[int]) -> None:
        """The same call, recording stage events (see dspark_attn_opts)."""
        for i, e in enumerate(events):
            self._events[i] = e
        st = self._ex(*self._args, self._opts_ev_ref)
        if st != DSPARK_OK:
            _check(st)


def bwd_workspace_size(desc: Desc) -> int:
    n = int(lib.dspark_attn_bwd_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


def bwd_plan(desc: Desc, force_generic: bool = False) -> int:
    """dspark_attn_bwd_plan: the number of stage events the call records."""
    opts, _ = _opts(None, force_generic, 0)
    ne = ctypes.c_int32()
    _check(lib.dspark_attn_bwd_plan(ctypes.byref(desc), ctypes.byref(opts), ctypes.byref(ne)))
    return ne.value


BWD_GRADS = ("dq_nope", "dq_rope", "dckv_ctx", "dkr_ctx", "dckv_blk", "dkr_blk", "dw_uk", "dw_uv")


def attn_bwd(desc: Desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
             anchors, keep, dout, grads, workspace, stream=None,
             stage_events: Optional[Sequence[int]] = None, force_generic: bool = False,
             reuse_forward: int = 0) -> None:
    """dspark_attn_bwd / dspark_attn_bwd_ex.  grads: a mapping with the
    output tensors named as in BWD_GRADS; raises DSparkError on a non-OK
    status.  reuse_forward: 0, 1 / True (the workspace holds the forward's
    index and q_abs) or 2 (and its softmax probabilities: a forward with
    for_backward); see dspark_attn_opts."""
    args = [ctypes.byref(desc)] + [_ptr(t) for t in (q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk,
                                                     kr_blk, w_uk, w_uv, anchors, keep, dout)]
    args += [_ptr(grads[k]) for k in BWD_GRADS]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args += [_ptr(workspace), ws_bytes, _stream(stream)]
    if stage_events is None and not force_generic and not reuse_forward:
        _check(lib.dspark_attn_bwd(*args))
        return
    opts, _arr = _opts(stage_events, force_generic, 0)
    opts.reuse_forward = int(reuse_forward)
    _check(lib.dspark_attn_bwd_ex(*args, ctypes.byref(opts)))


def make_layer_desc(attn: Desc, hidden: int, q_rank: int, rms_eps: float = 1e-6,
                    max_kept_blocks: int = 0) -> LayerDesc:
    return LayerDesc(attn, int(hidden), int(q_rank), float(rms_eps), int(max_kept_blocks))


def layer_read_status(workspace, stream=None):
    """Synchronises the stream; returns (status, first_bad_block, kept_blocks)."""
    fb, kb = ctypes.c_int32(-1), ctypes.c_int32(0)
    st = lib.dspark_mla_layer_read_status(_ptr(workspace), _stream(stream), ctypes.byref(fb),
                                          ctypes.byref(kb))
    return int(st), int(fb.value), int(kb.value)


def layer_workspace_size(desc: LayerDesc) -> int:
    n = int(lib.dspark_mla_layer_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


LAYER_WEIGHTS = ("g_in", "w_qa", "g_qa", "w_qb", "w_kva", "g_kva", "w_uk", "w_uv", "w_o")


def mla_layer_fwd(desc: LayerDesc, h_draft, h_ctx, weights, anchors, keep, out, workspace,
                  stream=None, stage_events: Optional[Sequence[int]] = None,
                  force_generic: bool = False, gemm_choices: Optional[GemmChoices] = None) -> None:
    """dspark_mla_layer_fwd / _ex; weights: a mapping named as in
    LAYER_WEIGHTS; gemm_choices: what mla_layer_tune returned (None: rocBLAS
    chooses)."""
    args = [ctypes.byref(desc), _ptr(h_draft), _ptr(h_ctx)]
    args += [_ptr(weights[k]) for k in LAYER_WEIGHTS]
    ws_bytes = workspace.numel() * workspace.element_size()
    args += [_ptr(anchors), _ptr(keep), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)]
    if stage_events is None and not force_generic and gemm_choices is None:
        _check(lib.dspark_mla_layer_fwd(*args))
        return
    opts, _arr = _opts(stage_events, force_generic, 0)
    if gemm_choices is not None:
        opts.gemm_choices = ctypes.pointer(gemm_choices)
    _check(lib.dspark_mla_layer_fwd_ex(*args, ctypes.byref(opts)))


def mla_layer_tune(desc: LayerDesc, h_draft, h_ctx, weights, anchors, keep, out, workspace,
                   stream=None) -> GemmChoices:
    """dspark_mla_layer_tune: one block call that also picks its GEMM kernels;
    returns them (pass to mla_layer_fwd as gemm_choices)."""
    args = [ctypes.byref(desc), _ptr(h_draft), _ptr(h_ctx)]
    args += [_ptr(weights[k]) for k in LAYER_WEIGHTS]
    ws_bytes = workspace.numel() * workspace.element_size()
    args += [_ptr(anchors), _ptr(keep), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)]
    choices = GemmChoices()
    _check(lib.dspark_mla_layer_tune(*args, ctypes.byref(choices)))
    return choices


def make_loss_desc(B: int, S: int, N: int, vocab: int, hidden: int, markov_rank: int,
                   dtype: str = "bf16", max_kept_blocks: int = 0, alpha_ce: float = 1.0,
                   alpha_l1: float = 0.9, alpha_conf: float = 1.0, w_lm_ld: int = 0,
                   w_m2_ld: int = 0, max_counted_steps: int = 0) -> LossDesc:
    dt = {"bf16": DSPARK_BF16, "f32": DSPARK_F32}[dtype]
    return LossDesc(int(B), int(S), int(N), int(vocab), int(hidden), int(markov_rank), dt,
                    int(max_kept_blocks), float(alpha_ce), float(alpha_l1), float(alpha_conf),
                    int(w_lm_ld), int(w_m2_ld), int(max_counted_steps))


def loss_workspace_size(desc: LossDesc) -> int:
    n = int(lib.dspark_loss_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


LOSS_INPUTS = ("input_ids", "loss_mask", "anchors", "keep", "h_final", "z", "w_lm", "w_m1", "w_m2",
               "w_conf")


def _loss_args(desc, t, terms, eval_mask, loss, workspace, stream):
    args = [ctypes.byref(desc)] + [_ptr(t[k]) for k in LOSS_INPUTS]
    ws_bytes = workspace.numel() * workspace.element_size()
    return args + [_ptr(terms), _ptr(eval_mask), _ptr(loss), _ptr(workspace), ws_bytes,
                   _stream(stream)]


def loss_fwd(desc: LossDesc, tensors, terms, eval_mask, loss, workspace, stream=None,
             stage_events: Optional[Sequence[int]] = None,
             gemm_choices: Optional[GemmChoices] = None) -> None:
    """dspark_loss_fwd / _ex; tensors: a mapping named as in LOSS_INPUTS;
    terms [4, B, N, 5] fp32, eval_mask [B, N, 5] uint8, loss [5] fp32;
    gemm_choices: what loss_tune returned (None: rocBLAS chooses)."""
    args = _loss_args(desc, tensors, terms, eval_mask, loss, workspace, stream)
    if stage_events is None and gemm_choices is None:
        _check(lib.dspark_loss_fwd(*args))
        return
    opts, _arr = _opts(stage_events, False, 0)
    if gemm_choices is not None:
        opts.gemm_choices = ctypes.pointer(gemm_choices)
    _check(lib.dspark_loss_fwd_ex(*args, ctypes.byref(opts)))


def loss_tune(desc: LossDesc, tensors, terms, eval_mask, loss, workspace,
              stream=None) -> GemmChoices:
    """dspark_loss_tune: one loss call that also picks its GEMM kernels;
    returns them (pass to loss_fwd as gemm_choices)."""
    choices = GemmChoices()
    _check(lib.dspark_loss_tune(*_loss_args(desc, tensors, terms, eval_mask, loss, workspace,
                                            stream), ctypes.byref(choices)))
    return choices


def loss_read_status(workspace, stream=None):
    """Synchronises the stream; returns (status, first_bad_block, kept_blocks,
    counted_steps)."""
    fb, kb, cs = ctypes.c_int32(-1), ctypes.c_int32(0), ctypes.c_int32(0)
    st = lib.dspark_loss_read_status(_ptr(workspace), _stream(stream), ctypes.byref(fb),
                                     ctypes.byref(kb), ctypes.byref(cs))
    return int(st), int(fb.value), int(kb.value), int(cs.value)


def make_decode_desc(attn: Desc, cache_slots: int) -> DecodeDesc:
    return DecodeDesc(attn, int(cache_slots))


def cache_append(desc: DecodeDesc, pos0, n_new, new_ckv, new_kr, cache_ckv, cache_kr,
                 stream=None) -> None:
    """dspark_cache_append; new_ckv [B, max_new, D] fixes max_new."""
    _check(lib.dspark_cache_append(ctypes.byref(desc), _ptr(pos0), _ptr(n_new),
                                   int(new_ckv.shape[1]), _ptr(new_ckv), _ptr(new_kr),
                                   _ptr(cache_ckv), _ptr(cache_kr), _stream(stream)))


def decode_workspace_size(desc: DecodeDesc) -> int:
    n = int(lib.dspark_decode_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


def decode_attn(desc: DecodeDesc, q_nope, q_rope, cache_ckv, cache_kr, ckv_blk, kr_blk, w_uk, w_uv,
                anchors, active, out, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dspark_decode_attn(ctypes.byref(desc), _ptr(q_nope), _ptr(q_rope), _ptr(cache_ckv),
                                  _ptr(cache_kr), _ptr(ckv_blk), _ptr(kr_blk), _ptr(w_uk),
                                  _ptr(w_uv), _ptr(anchors), _ptr(active), _ptr(out),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


VERIFY_MODES = {"rejection": 0, "target_only": 1}


def make_verify_desc(B: int, K: int, vocab: int, mode: str = "rejection",
                     temperature: float = 1.0) -> VerifyDesc:
    return VerifyDesc(int(B), int(K), int(vocab), VERIFY_MODES[mode], float(temperature))


def verify_workspace_size(desc: VerifyDesc) -> int:
    n = int(lib.dspark_verify_workspace_size(ctypes.byref(desc)))
    if n == 0:
        raise DSparkError(DSPARK_EINVAL, last_error())
    return n


def spec_verify(desc: VerifyDesc, draft_logits, target_logits, draft_tokens, uniforms, accept_prob,
                overlap, n_accept, next_token, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dspark_spec_verify(ctypes.byref(desc), _ptr(draft_logits), _ptr(target_logits),
                                  _ptr(draft_tokens), _ptr(uniforms), _ptr(accept_prob),
                                  _ptr(overlap), _ptr(n_accept), _ptr(next_token), _ptr(workspace),
                                  ws_bytes, _stream(stream)))


def build_index(desc: Desc, anchors, keep, index_out, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.dspark_build_index(ctypes.byref(desc), _ptr(anchors), _ptr(keep), _ptr(index_out),
                                  _ptr(workspace), ws_bytes, _stream(stream)))


def select_anchors_host(loss_mask: np.ndarray, num_anchors: int, seed: int):
    """Host sampler; returns (anchors int32 [num_anchors], keep uint8 [num_anchors])."""
    lm = np.ascontiguousarray(loss_mask, dtype=np.uint8)
    anchors = np.zeros(num_anchors, dtype=np.int32)
    keep = np.zeros(num_anchors, dtype=np.uint8)
    _check(lib.dspark_select_anchors_host(lm.ctypes.data, lm.shape[0], num_anchors,
                                          ctypes.c_uint64(seed & (2 ** 64 - 1)),
                                          anchors.ctypes.data, keep.ctypes.data))
    return anchors, keep


def read_device_status(workspace, stream=None):
    """Synchronises the stream; returns (status, first_bad_block)."""
    fb = ctypes.c_int32(-1)
    st = lib.dspark_read_device_status(_ptr(workspace), _stream(stream), ctypes.byref(fb))
    return int(st), int(fb.value)
