"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, validates its arguments before any
device work, and its host anchor sampler matches the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import workloads as wk
from conftest import ROOT

sd = pytest.importorskip("speculative_decoding_draft_amd")


def header_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    declared = header_functions()
    assert {"dspark_attn_fwd", "dspark_attn_workspace_size", "dspark_build_index",
            "dspark_select_anchors_host", "dspark_read_device_status", "dspark_last_error",
            "dspark_abi_version", "dspark_attn_fwd_ex", "dspark_attn_bwd",
            "dspark_attn_bwd_ex", "dspark_attn_bwd_workspace_size", "dspark_attn_bwd_plan"} <= declared
    lib = ctypes.CDLL(sd.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert set(sd.EXPORTS) == declared
    assert sd.abi_version() == 13


def glm_desc(**kw):
    d = dict(B=1, S=2048, N=64, window=128, n_heads=64, d_latent=512, d_nope=192, d_rope=64,
             d_v=256, dtype="bf16")
    d.update(kw)
    return sd.make_desc(**d)


def test_workspace_size_accounts_for_latent_buffers():
    d = glm_desc()
    n = sd.workspace_size(d)
    lat = 64 * 5 * 64 * 512 * 2
    assert n >= 2 * lat and n < 2 * lat + 4 * 2**20
    # a non-GLM shape takes the generic kernels: no latent buffers
    small = sd.workspace_size(glm_desc(n_heads=2, d_latent=32, d_nope=16, d_rope=8, d_v=16))
    assert small < 2**20
    # W > 128 also leaves the MFMA path
    assert sd.workspace_size(glm_desc(window=256)) < n


@pytest.mark.parametrize("field,value,status", [
    ("block", 4, sd.DSPARK_EUNSUPPORTED), ("window", 0, sd.DSPARK_EINVAL),
    ("S", 0, sd.DSPARK_EINVAL), ("d_rope", 7, sd.DSPARK_EINVAL),
    ("dtype", 9, sd.DSPARK_EINVAL), ("rope_base", -1.0, sd.DSPARK_EINVAL),
    ("n_heads", 0, sd.DSPARK_EINVAL), ("B", -1, sd.DSPARK_EINVAL)])
def test_bad_descriptor_is_rejected(field, value, status):
    d = glm_desc()
    setattr(d, field, value)
    assert sd._lib.lib.dspark_attn_workspace_size(ctypes.byref(d)) == 0
    st = sd._lib.lib.dspark_attn_fwd(ctypes.byref(d), *([None] * 12), 0, None)
    assert st == status
    assert sd.last_error() != ""


class FakePtr:
    """Stands in for a device tensor when only host-side validation runs."""

    def __init__(self, addr, nbytes=0):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def _call(d, ptrs, ws, ws_bytes):
    lib = sd._lib.lib
    return lib.dspark_attn_fwd(ctypes.byref(d), *ptrs, ws, ws_bytes, None)


def test_null_misaligned_and_workspace_errors_before_any_launch():
    d = glm_desc()
    good = [0x10000 * (i + 1) for i in range(11)]
    need = sd.workspace_size(d)
    ws = 0x7000000
    for i in range(11):
        p = list(good)
        p[i] = None
        assert _call(d, p, ws, need) == sd.DSPARK_EINVAL
        assert "NULL" in sd.last_error()
    p = list(good)
    p[0] += 4
    assert _call(d, p, ws, need) == sd.DSPARK_EINVAL
    assert "aligned" in sd.last_error()
    assert _call(d, good, ws, need - 1) == sd.DSPARK_EWORKSPACE
    assert "too small" in sd.last_error()
    assert _call(d, good, ws + 64, need) == sd.DSPARK_EWORKSPACE
    assert _call(d, good, None, need) == sd.DSPARK_EWORKSPACE


def test_empty_problem_is_a_no_op():
    d = glm_desc(N=0)
    assert sd._lib.lib.dspark_attn_fwd(ctypes.byref(d), *([None] * 12), 0, None) == sd.DSPARK_OK


def test_mfma_path_needs_32bit_offsets():
    """The MFMA path addresses q_nope and ckv_ctx with 32-bit byte offsets:
    beyond 4 GiB the generic path (no latent buffers) is planned instead."""
    fast = glm_desc(S=4096, N=64)
    assert sd.attn_plan(fast)[0] == 1
    big_ctx = glm_desc(S=4 * 2**20, N=64)          # ckv_ctx = 4 GiB
    assert sd.attn_plan(big_ctx) == (0, 0, 3)
    assert sd.workspace_size(big_ctx) < sd.workspace_size(glm_desc(S=4 * 2**20 - 8, N=64))
    big_q = glm_desc(B=2, S=256, N=20000)          # q_nope = 2 * 100000 rows * 24 KiB > 4 GiB
    assert sd.attn_plan(big_q) == (0, 0, 3)


def test_opts_struct_matches_header():
    """The binding's dspark_attn_opts has the header's layout (x86-64)."""
    assert ctypes.sizeof(sd._lib.Opts) == 8 + 4 * 3 + 4 + 8 + 16 + 8 + 8
    assert sd._lib.Opts.aux_stream.offset == 24 and sd._lib.Opts.aux_events.offset == 32
    assert sd._lib.Opts.reuse_forward.offset == 48 and sd._lib.Opts.one_launch.offset == 52
    assert sd._lib.Opts.gemm_choices.offset == 56


def test_aux_stream_is_validated():
    d = glm_desc(N=64)
    need = sd.workspace_size(d)
    p = [0x10000 * (i + 1) for i in range(11)]
    lib = sd._lib.lib
    opts = sd._lib.Opts()
    opts.chunk_blocks = 16
    opts.aux_stream = 0x1234
    st = lib.dspark_attn_fwd_ex(ctypes.byref(d), *p, 0x7000000, need, None, ctypes.byref(opts))
    assert st == sd.DSPARK_EINVAL and "aux_events" in sd.last_error()
    opts.aux_stream = None
    opts.aux_events[0] = opts.aux_events[1] = 0x10


def test_launch_plan():
    d = glm_desc(B=2, N=1000)
    assert sd.attn_plan(d) == (1, 2000, 6)
    assert sd.attn_plan(d, chunk_blocks=1) == (2000, 1, 2 + 4 * 2000)
    assert sd.attn_plan(d, chunk_blocks=300) == (7, 300, 30)
    assert sd.attn_plan(d, chunk_blocks=10**6) == (1, 2000, 6)    # capped at B*N
    assert sd.attn_plan(d, force_generic=True) == (0, 0, 3)
    assert sd.attn_plan(glm_desc(dtype="f32")) == (0, 0, 3)
    assert sd.attn_plan(glm_desc(N=0)) == (0, 0, 0)
    with pytest.raises(sd.DSparkError):
        sd.attn_plan(glm_desc(window=0))


def test_generic_lds_limit_is_reported():
    d = glm_desc(dtype="f32", window=4000, d_latent=2048)
    need = sd.workspace_size(d)
    p = [0x10000 * (i + 1) for i in range(11)]
    assert _call(d, p, 0x7000000, need) == sd.DSPARK_EUNSUPPORTED


# ---------------------------------------------------------------------------
# host sampler vs the oracle sampler (bit-exact)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S,N,p", [(48, 4, 0.9), (200, 10, 0.9), (64, 40, 0.5), (30, 30, 0.3),
                                   (2, 1, 1.0), (1, 3, 1.0), (5000, 512, 0.9)])
def test_sampler_matches_oracle(S, N, p):
    rng = np.random.default_rng(S * 31 + N)
    for trial in range(20):
        lm = (rng.random(S) < p).astype(np.uint8)
        seed = int(rng.integers(0, 2**63))
        a_c, k_c = sd.select_anchors_host(lm, N, seed)
        a_o, k_o = O.select_anchors(lm, N, seed)
        assert np.array_equal(a_c, a_o) and np.array_equal(k_c, k_o), (S, N, trial)


@pytest.mark.parametrize("k", [2, 5])
def test_sampler_matches_oracle_on_benchmark_masks(k):
    wl = wk.config(k, tensors=False)
    for b in range(wl.B):
        a_c, k_c = sd.select_anchors_host(wl.loss_mask[b], wl.N, wl.sampler_seed + b)
        a_o, k_o = O.select_anchors(wl.loss_mask[b], wl.N, wl.sampler_seed + b)
        assert np.array_equal(a_c, a_o) and np.array_equal(k_c, k_o)
        assert k_c.all()


# ---------------------------------------------------------------------------
# backward entry points: validation before any launch
# ---------------------------------------------------------------------------

def _bwd_call(d, ptrs, ws, ws_bytes, opts=None):
    lib = sd._lib.lib
    if opts is None:
        return lib.dspark_attn_bwd(ctypes.byref(d), *ptrs, ws, ws_bytes, None)
    return lib.dspark_attn_bwd_ex(ctypes.byref(d), *ptrs, ws, ws_bytes, None, ctypes.byref(opts))


def test_bwd_workspace_holds_forward_area_and_accumulators():
    d = glm_desc(B=1, S=2048, N=64)
    fwd, bwd = sd.workspace_size(d), sd.bwd_workspace_size(d)
    rows = 5 * 64
    acc = (2048 + rows) * (512 + 64) * 4
    lat = rows * 64 * 512 * 2
    pm = 64 * rows * 144 * 2
    part = 64 * 132 * (512 + 64) * 4
    assert bwd >= fwd + acc + 2 * lat + rows * 64 * 64 * 2 + 2 * pm + part
    g = glm_desc(dtype="f32", B=1, S=2048, N=64)
    wacc = 64 * (192 + 256) * 512 * 4
    assert sd.bwd_workspace_size(g) >= sd.workspace_size(g) + acc + wacc
    # the MFMA-path size also covers force_generic (weight accumulators)
    small = glm_desc(B=1, S=300, N=12)
    assert sd.bwd_workspace_size(small) >= (300 + 60) * (512 + 64) * 4 + wacc
    # a forward that leaves its probabilities for the backward needs the
    # backward's workspace on the MFMA path; the generic path leaves none
    assert fwd < sd.workspace_size_ex(d, for_backward=True) <= bwd
    assert sd.workspace_size_ex(d, for_backward=True) >= fwd + 2 * lat + 2 * pm
    assert (sd.workspace_size_ex(d, force_generic=True, for_backward=True)
            == sd.workspace_size_ex(d, force_generic=True))


def test_bwd_null_misaligned_and_workspace_errors_before_any_launch():
    d = glm_desc()
    good = [0x10000 * (i + 1) for i in range(19)]
    need = sd.bwd_workspace_size(d)
    ws = 0x7000000
    for i in range(19):
        p = list(good)
        p[i] = None
        assert _bwd_call(d, p, ws, need) == sd.DSPARK_EINVAL
        assert "NULL" in sd.last_error()
    p = list(good)
    p[12] += 8
    assert _bwd_call(d, p, ws, need) == sd.DSPARK_EINVAL and "aligned" in sd.last_error()
    assert _bwd_call(d, good, ws, need - 1) == sd.DSPARK_EWORKSPACE
    assert _bwd_call(d, good, ws + 64, need) == sd.DSPARK_EWORKSPACE
    # d_rope = 0: the six rope pointers may be NULL (generic path, no launch
    # happens here because the workspace is too small)
    z = glm_desc(d_rope=0)
    p = list(good)
    for i in (1, 3, 5, 12, 14, 16):
        p[i] = None
    assert _bwd_call(z, p, ws, 0) == sd.DSPARK_EWORKSPACE


def test_bwd_plan_and_event_count_check():
    d = glm_desc()
    assert sd.bwd_plan(d) == 11 and sd.bwd_plan(d, force_generic=True) == 5
    assert sd.bwd_plan(glm_desc(dtype="f32")) == 5 and sd.bwd_plan(glm_desc(N=0)) == 0
    opts = sd._lib.Opts()
    ev = (ctypes.c_void_p * 3)(0x10, 0x20, 0x30)
    opts.stage_events = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    opts.n_stage_events = 3
    good = [0x10000 * (i + 1) for i in range(19)]
    st = _bwd_call(d, good, 0x7000000, sd.bwd_workspace_size(d), opts)
    assert st == sd.DSPARK_EINVAL and "stage events" in sd.last_error()


def test_bwd_empty_problem_is_a_no_op():
    d = glm_desc(N=0)
    assert sd._lib.lib.dspark_attn_bwd(ctypes.byref(d), *([None] * 20), 0, None) == sd.DSPARK_OK


# ---------------------------------------------------------------------------
# MLA block entry point: validation before any launch
# ---------------------------------------------------------------------------

def layer_desc(**kw):
    return sd.make_layer_desc(glm_desc(**kw), hidden=6144, q_rank=2048)


def test_layer_desc_layout_and_workspace():
    assert ctypes.sizeof(sd.LayerDesc) == ctypes.sizeof(sd._lib.Desc) + 4 + 4 + 8 + 8
    d = layer_desc(S=2048, N=64)
    need = sd.layer_workspace_size(d)
    rows = 5 * 64
    inter = (rows * 6144 + rows * 2048 + rows * 64 * 256 + (2048 + rows) * 576 * 2
             + rows * 64 * 256) * 2
    assert need >= inter + sd.workspace_size(d.attn)
    bad = sd.make_layer_desc(glm_desc(), hidden=0, q_rank=2048)
    assert sd._lib.lib.dspark_mla_layer_workspace_size(ctypes.byref(bad)) == 0


def test_layer_null_misaligned_and_workspace_errors_before_any_launch():
    d = layer_desc()
    need = sd.layer_workspace_size(d)
    good = [0x10000 * (i + 1) for i in range(14)]
    lib = sd._lib.lib
    call = lambda p, ws, n: lib.dspark_mla_layer_fwd(ctypes.byref(d), *p, ws, n, None)
    for i in range(14):
        p = list(good)
        p[i] = None
        assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL and "NULL" in sd.last_error()
    p = list(good)
    p[0] += 2
    assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL and "aligned" in sd.last_error()
    assert call(good, 0x7000000, need - 1) == sd.DSPARK_EWORKSPACE
    assert call(good, 0x7000010, need) == sd.DSPARK_EWORKSPACE
    neg = sd.make_layer_desc(glm_desc(), hidden=6144, q_rank=2048, rms_eps=-1.0)
    assert lib.dspark_mla_layer_fwd(ctypes.byref(neg), *good, 0x7000000, need, None) == sd.DSPARK_EINVAL


def test_loss_desc_layout_and_workspace():
    assert ctypes.sizeof(sd.LossDesc) == 8 * 4 + 3 * 8 + 8 + 8
    d = sd.make_loss_desc(B=1, S=32768, N=1024, vocab=154880, hidden=6144, markov_rank=256)
    need = sd.loss_workspace_size(d)
    rows = 5 * 1024
    logits = 2 * rows * 154880 * 4
    gathered = 2 * rows * (6144 + 256) * 2
    stats = rows * 19 * (16 + 4)
    blas = sd.BLAS_WORKSPACE_BYTES            # rocBLAS works in the caller's workspace
    assert logits + gathered + stats + blas <= need < logits + gathered + stats + blas + 2**20
    # max_kept_blocks and max_counted_steps shrink every row-sized buffer
    d2 = sd.make_loss_desc(B=1, S=32768, N=1024, vocab=154880, hidden=6144, markov_rank=256,
                           max_kept_blocks=768)
    assert abs(sd.loss_workspace_size(d2) - blas - (need - blas) * 768 / 1024) < 2**20
    d3 = sd.make_loss_desc(B=1, S=32768, N=1024, vocab=154880, hidden=6144, markov_rank=256,
                           max_kept_blocks=768, max_counted_steps=2560)
    assert abs(sd.loss_workspace_size(d3) - blas - (need - blas) * 2560 / 5120) < 2**20
    for kw in (dict(vocab=0), dict(hidden=0), dict(markov_rank=0), dict(max_kept_blocks=-1),
               dict(S=0), dict(w_lm_ld=7), dict(w_m2_ld=3), dict(max_counted_steps=-1)):
        args = dict(B=1, S=64, N=4, vocab=100, hidden=8, markov_rank=4)
        args.update(kw)
        bad = sd.make_loss_desc(**args)
        assert sd._lib.lib.dspark_loss_workspace_size(ctypes.byref(bad)) == 0


def test_loss_null_misaligned_and_workspace_errors_before_any_launch():
    d = sd.make_loss_desc(B=1, S=64, N=4, vocab=100, hidden=8, markov_rank=8)
    need = sd.loss_workspace_size(d)
    good = [0x10000 * (i + 1) for i in range(13)]
    lib = sd._lib.lib
    call = lambda p, ws, n: lib.dspark_loss_fwd(ctypes.byref(d), *p, ws, n, None)
    for i in range(13):
        p = list(good)
        p[i] = None
        assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL and "NULL" in sd.last_error()
    for i in (4, 5, 6, 7, 8, 9):           # the dense tensors need 16-byte alignment
        p = list(good)
        p[i] += 4
        assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL and "aligned" in sd.last_error()
    p = list(good)
    p[0] += 2                              # input_ids: int32
    assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL
    assert call(good, 0x7000000, need - 1) == sd.DSPARK_EWORKSPACE
    assert call(good, 0x7000010, need) == sd.DSPARK_EWORKSPACE
    ev = (ctypes.c_void_p * 5)(*[0x100] * 5)
    opts = sd._lib.Opts()
    opts.stage_events = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p))
    opts.n_stage_events = 5
    assert lib.dspark_loss_fwd_ex(ctypes.byref(d), *good, 0x7000000, need, None,
                                  ctypes.byref(opts)) == sd.DSPARK_EINVAL


def test_decode_and_verify_validation_before_any_launch():
    lib = sd._lib.lib
    attn = glm_desc(B=4, S=0, N=1)
    d = sd.make_decode_desc(attn, 128)
    need = sd.decode_workspace_size(d)
    # the attention's workspace for 4 one-block problems of S' = W + 1 rows
    # comes first, then the gathered windows
    assert need >= sd.workspace_size(glm_desc(B=4, S=129, N=1)) + 4 * 129 * 576 * 2
    for bad in (sd.make_decode_desc(glm_desc(B=4, N=2), 128), sd.make_decode_desc(attn, 126)):
        assert lib.dspark_decode_workspace_size(ctypes.byref(bad)) == 0
    good = [0x10000 * (i + 1) for i in range(11)]
    call = lambda p, ws, n: lib.dspark_decode_attn(ctypes.byref(d), *p, ws, n, None)
    for i in (2, 3, 8, 9):                 # cache_ckv, cache_kr, anchors, active
        p = list(good)
        p[i] = None
        assert call(p, 0x7000000, need) == sd.DSPARK_EINVAL
    assert call(good, 0x7000000, need - 1) == sd.DSPARK_EWORKSPACE
    assert lib.dspark_cache_append(ctypes.byref(d), None, 0x1000, 3, 0x2000, 0x3000, 0x4000,
                                   0x5000, None) == sd.DSPARK_EINVAL
    assert lib.dspark_cache_append(ctypes.byref(d), 0x1000, 0x1000, -1, 0x2000, 0x3000, 0x4000,
                                   0x5000, None) == sd.DSPARK_EINVAL
    v = sd.make_verify_desc(B=8, K=5, vocab=154880)
    need = sd.verify_workspace_size(v)
    assert need >= 8 * 11 * 19 * 16 + 8 * 5 * 19 * 8
    for bad in (sd.make_verify_desc(8, 0, 100), sd.make_verify_desc(8, 65, 100),
                sd.make_verify_desc(8, 5, 0), sd.make_verify_desc(8, 5, 100, temperature=0.0)):
        assert lib.dspark_verify_workspace_size(ctypes.byref(bad)) == 0
    badmode = sd.make_verify_desc(8, 5, 100)
    badmode.mode = 7
    assert lib.dspark_verify_workspace_size(ctypes.byref(badmode)) == 0
    ptrs = [0x10000 * (i + 1) for i in range(8)]
    vcall = lambda p, ws, n: lib.dspark_spec_verify(ctypes.byref(v), *p, ws, n, None)
    for i in range(8):
        p = list(ptrs)
        p[i] = None
        assert vcall(p, 0x7000000, need) == sd.DSPARK_EINVAL
    assert vcall(ptrs, 0x7000000, need - 1) == sd.DSPARK_EWORKSPACE


@pytest.mark.parametrize("shape", [
    dict(N=2_000_000),                 # index alone (36 bytes a block) is over 64 MiB
    dict(S=300_000, window=256),       # generic path: RoPE table over 64 MiB
])
def test_noalloc_forward_rejects_shapes_beyond_its_scratch(shape):
    """The allocation-free forward refuses, before touching a device, any
    shape whose index and latent round (or RoPE table) exceed the fixed
    array; a shape that fits gets past that check (and then fails on the
    NULL tensors here)."""
    d = glm_desc(**shape)
    st = sd._lib.lib.dspark_attn_fwd_noalloc(ctypes.byref(d), *([None] * 12), None)
    assert st == sd.DSPARK_EUNSUPPORTED
    assert "scratch" in sd.last_error()
    assert sd.NOALLOC_SCRATCH_BYTES == 64 << 20 and sd.STATUS_BYTES == 64


def test_noalloc_forward_checks_status_alignment_and_empty_problems():
    d = glm_desc(N=0)
    assert sd._lib.lib.dspark_attn_fwd_noalloc(ctypes.byref(d), *([None] * 12), None) == 0
    d = glm_desc()
    st = sd._lib.lib.dspark_attn_fwd_noalloc(ctypes.byref(d), *([None] * 11), 0x1002, None)
    assert st == sd.DSPARK_EINVAL and "status" in sd.last_error()


def test_tune_calls_need_a_choices_table():
    """The *_tune calls write their GEMM choices into a caller-owned table and
    refuse a NULL one before any device work; the table's C layout is 4
    int32 per GEMM after the count."""
    lib = sd._lib.lib
    d = sd.make_layer_desc(glm_desc(), 6144, 2048)
    assert lib.dspark_mla_layer_tune(ctypes.byref(d), *([None] * 15), 0, None, None) == sd.DSPARK_EINVAL
    assert "choices" in sd.last_error()
    ld = sd.make_loss_desc(1, 2048, 64, 1000, 6144, 256)
    assert lib.dspark_loss_tune(ctypes.byref(ld), *([None] * 14), 0, None, None) == sd.DSPARK_EINVAL
    assert "choices" in sd.last_error()
    assert ctypes.sizeof(sd.GemmChoices) == 4 + 8 * 16
    assert sd.BLAS_WORKSPACE_BYTES == 64 << 20
