"""Parity of the HIP backward (dspark_attn_bwd through the C ABI) with the
fp64 oracle's backward, on the same seeded inputs and upstream gradient.

Tolerances (per gradient tensor, over every element):
  * fp32 generic path: rel-L2 <= 2e-5 and max|err| <= 1e-4 * max|ref|.
    Every value is a short chain of fp32 dot products (<= 512 terms), an
    fp32 softmax and an fp32 rotation; sums over blocks and heads are fp32
    atomics in any order.  Measured errors are ~1e-6 relative.
  * bf16 storage: every output is rounded to bf16 once (relative error
    <= 2^-9, RMS ~1.1e-3).  The MFMA path also rounds its intermediates to
    bf16 (q_abs, W_UV^T dout, P, dS', o_lat, dq_abs, rotated q^R: <= 4 such
    roundings on any chain), so its error is a few times that of one
    rounding; it is held to the forward's bar, rel-L2 <= 5e-3, with
    max|err| <= 1e-2 * max|ref| (measured: <= 4.0e-3 and 4.9e-3), as is
    the generic bf16 path (fp32 intermediates).  Two GPU paths compared
    with each other carry both errors: rel-L2 <= 1e-2, 3e-2 * max|ref|.
Rows that no kept block reaches must be exactly 0 (padding blocks' query
and key rows, context rows outside every window); outputs are pre-filled
with NaN so that an element the library does not write fails the check.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from gpu_util import anchors_for, context_of_two, desc_for, log, repeated_anchors, sample_blocks
from workloads.device import to_torch, upload_anchors, upload_layer

pytestmark = pytest.mark.gpu

GRADS = ("dq_nope", "dq_rope", "dckv_ctx", "dkr_ctx", "dckv_blk", "dkr_blk", "dw_uk", "dw_uv")
F32_TOL = (2e-5, 1e-4)
BF16_GENERIC_TOL = (5e-3, 2e-2)
BF16_MFMA_TOL = (5e-3, 1e-2)
GPU_PATHS_TOL = (1e-2, 3e-2)


class GpuBwd:
    """Uploads one layer and an upstream gradient, owns the gradient outputs
    (NaN-filled) and the workspace, runs dspark_attn_bwd."""

    def __init__(self, wl, dout, anchors, keep, force_generic=False):
        import torch
        import speculative_decoding_draft_amd as sd
        self.sd, self.torch, self.wl = sd, torch, wl
        self.desc = desc_for(wl)
        self.t = upload_layer(wl)
        self.dout = to_torch(dout, wl.dtype, "cuda")
        self.anchors, self.keep = upload_anchors(anchors, keep)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        B, S, L5, H = wl.B, wl.S, wl.q_len, wl.H
        shapes = {"dq_nope": (B, L5, H, wl.d_c), "dq_rope": (B, L5, H, wl.d_r),
                  "dckv_ctx": (B, S, wl.D), "dkr_ctx": (B, S, wl.d_r),
                  "dckv_blk": (B, L5, wl.D), "dkr_blk": (B, L5, wl.d_r),
                  "dw_uk": (H, wl.d_c, wl.D), "dw_uv": (H, wl.d_v, wl.D)}
        self.g = {k: torch.full(v, float("nan"), dtype=tdt, device="cuda")
                  for k, v in shapes.items()}
        self.ws = torch.empty(sd.bwd_workspace_size(self.desc), dtype=torch.uint8, device="cuda")
        self.force_generic = force_generic

    def run(self):
        t = self.t
        self.sd.attn_bwd(self.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"],
                         t["ckv_blk"], t["kr_blk"], t["w_uk"], t["w_uv"], self.anchors,
                         self.keep, self.dout, self.g, self.ws,
                         force_generic=self.force_generic)
        return self

    def result(self) -> dict:
        self.torch.cuda.synchronize()
        return {k: v.float().cpu().numpy().astype(np.float64) for k, v in self.g.items()}


def check(gpu: dict, ref: dict, tol, what: str, names=GRADS, rows=None) -> None:
    """rows: None, or {name: boolean mask over the leading dims} restricting
    the comparison (elements outside are not checked)."""
    rel_tol, abs_tol = tol
    for k in names:
        g, r = gpu[k], ref[k]
        if rows is not None and k in rows:
            g, r = g[rows[k]], r[rows[k]]
        assert np.all(np.isfinite(g)), f"{what} {k}: non-finite values"
        scale = np.abs(r).max()
        if scale == 0:
            assert np.all(g == 0), f"{what} {k}: expected all zero"
            continue
        err = np.abs(g - r)
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        mx = float(err.max() / scale)
        log(f"  {what} {k}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e} n={g.size}")
        assert rel <= rel_tol, f"{what} {k}: rel_l2 {rel} > {rel_tol}"
        assert mx <= abs_tol, f"{what} {k}: max_abs {mx} > {abs_tol} of max|ref|"


def unreached_rows_are_zero(gpu: dict, wl, anchors, keep) -> None:
    """Rows of padding blocks and context rows outside every window."""
    for b in range(wl.B):
        seen = np.zeros(wl.S, bool)
        for n in range(wl.N):
            if keep[b, n]:
                A = int(anchors[b, n])
                seen[max(0, A - wl.W + 1):A] = True
            else:
                r = slice(5 * n, 5 * n + 5)
                for k in ("dq_nope", "dq_rope", "dckv_blk", "dkr_blk"):
                    assert np.all(gpu[k][b, r] == 0), (k, b, n)
        assert np.all(gpu["dckv_ctx"][b][~seen] == 0) and np.all(gpu["dkr_ctx"][b][~seen] == 0)


def run_case(wl, force_generic=False, tol=None, form="dense"):
    ga, gk, oa, ok = anchors_for(wl)
    assert np.array_equal(ga, oa) and np.array_equal(gk, ok)
    dout = wk.make_dout(wl, seed=11)
    log(f"case {wl.name} generic={force_generic}")
    gpu = GpuBwd(wl, dout, ga, gk, force_generic=force_generic).run().result()
    ref = O.backward(wl, dout, anchors=oa, keep=ok, form=form)
    check(gpu, ref, tol, wl.name)
    unreached_rows_are_zero(gpu, wl, oa, ok)
    return gpu


def test_bwd_tiny_fp32_generic():
    run_case(wk.config(1), tol=F32_TOL)


@pytest.mark.parametrize("k,S,N", [(1, 90, 12), (4, 120, 16)])
def test_bwd_tiny_dims_fp32_recipes(k, S, N):
    wl = wk.scaled(k, S=S, N=N, dims=wk.TINY_DIMS, dtype="f32")
    run_case(wl, tol=F32_TOL)


def test_bwd_generic_bf16_glm_dims():
    wl = wk.scaled(4, S=300, N=12)
    run_case(wl, force_generic=True, tol=BF16_GENERIC_TOL, form="gathered")


@pytest.mark.parametrize("k,S,N", [(2, 512, 16), (3, 640, 16), (4, 1024, 40)])
def test_bwd_mfma_scaled(k, S, N):
    wl = wk.scaled(k, S=S, N=N)
    run_case(wl, tol=BF16_MFMA_TOL, form="gathered")


def test_bwd_context_of_two_positions():
    """S = 2: every kept block anchors at 0 (repeated within a sample), so the
    context gradients are all zero and every gradient comes from the blocks'
    own keys; MFMA path."""
    run_case(context_of_two(92), tol=BF16_MFMA_TOL, form="dense")


def test_bwd_repeated_kept_anchors():
    """Equal anchors in a sorted sample: the per-row sums over the covering
    blocks include runs of blocks with the same window."""
    run_case(repeated_anchors(94), tol=BF16_MFMA_TOL, form="gathered")


def test_bwd_mfma_matches_generic_path():
    """Both GPU paths on the same bf16 problem agree to the MFMA tolerance."""
    wl = wk.scaled(4, S=400, N=16)
    ga, gk, _, _ = anchors_for(wl)
    dout = wk.make_dout(wl, seed=12)
    fast = GpuBwd(wl, dout, ga, gk).run().result()
    gen = GpuBwd(wl, dout, ga, gk, force_generic=True).run().result()
    check(fast, gen, GPU_PATHS_TOL, "mfma vs generic")


def test_bwd_more_kept_blocks_than_one_row_table():
    """More than 1024 kept blocks: the weight-gradient kernel walks the rows
    in several LDS row tables.  The fp64 oracle would need about a minute
    for every block, so the MFMA path is held to the generic path here (that
    path is held to the oracle at the sizes it can reach)."""
    wl = wk.scaled(4, S=16384, N=1500)
    ga, gk, _, _ = anchors_for(wl)
    assert int(gk.sum()) > 1024
    dout = wk.make_dout(wl, seed=14)
    log(f"case {wl.name}: {int(gk.sum())} kept blocks, MFMA against generic")
    fast = GpuBwd(wl, dout, ga, gk).run().result()
    gen = GpuBwd(wl, dout, ga, gk, force_generic=True).run().result()
    check(fast, gen, GPU_PATHS_TOL, "mfma vs generic, several row tables")


def test_bwd_repeat_runs_agree():
    """A second call on the same workspace gives the same gradients (the
    accumulators are cleared by every call; atomics may reorder fp32 sums)."""
    wl = wk.scaled(2, S=512, N=16)
    ga, gk, _, _ = anchors_for(wl)
    run = GpuBwd(wl, wk.make_dout(wl, seed=13), ga, gk)
    a = run.run().result()
    b = run.run().result()
    for k in GRADS:
        if k in ("dckv_ctx", "dkr_ctx", "dckv_blk", "dkr_blk"):
            np.testing.assert_allclose(b[k], a[k], rtol=1e-2, atol=1e-2 * np.abs(a[k]).max())
        else:
            assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("generic", [False, True])
def test_bwd_bad_anchor_rows_are_nan(generic):
    """A kept block with an anchor outside [0, S-2]: its query-gradient rows
    are NaN, the status reports it, and every other gradient equals the
    oracle's with that block treated as padding."""
    import speculative_decoding_draft_amd as sd
    wl = wk.scaled(4, S=300, N=12)
    anchors, keep = wl.anchors.copy(), wl.keep.copy()
    bad = int(np.nonzero(keep[0])[0][3])
    anchors[0, bad] = wl.S + 3
    dout = wk.make_dout(wl, seed=14)
    run = GpuBwd(wl, dout, anchors, keep, force_generic=generic).run()
    gpu = run.result()
    st, first = sd.read_device_status(run.ws)
    assert st == sd.DSPARK_EANCHOR and first == bad
    r = slice(5 * bad, 5 * bad + 5)
    assert np.all(np.isnan(gpu["dq_nope"][0, r])) and np.all(np.isnan(gpu["dq_rope"][0, r]))
    gpu["dq_nope"][0, r] = 0
    gpu["dq_rope"][0, r] = 0
    keep_ref = keep.copy()
    keep_ref[0, bad] = 0
    ref = O.backward(wl, dout, anchors=anchors, keep=keep_ref, form="gathered")
    check(gpu, ref, BF16_GENERIC_TOL if generic else BF16_MFMA_TOL, f"bad anchor generic={generic}")


def test_bwd_headline_full_size_all_blocks():
    """Full headline size (B=1, S=32768, N=1024, 25 % padding) in the launch
    configuration the benchmark times, every gradient over every kept
    block.  The oracle runs in batches of kept blocks (the gradient is
    linear in dout, so the batches' sums are the whole gradient: pinned on
    the CPU); every row no kept block reaches must be 0."""
    wl = wk.config(4)
    dout = wk.make_dout(wl, seed=15)
    log("case headline full size")
    gpu = GpuBwd(wl, dout, wl.anchors, wl.keep).run().result()
    unreached_rows_are_zero(gpu, wl, wl.anchors, wl.keep)
    for k in GRADS:
        assert np.all(np.isfinite(gpu[k])), k
    kept = [int(n) for n in np.nonzero(wl.keep[0])[0]]
    ref = None
    for i in range(0, len(kept), 96):
        part = O.backward(wl, dout, form="gathered", blocks=[(0, n) for n in kept[i:i + 96]])
        ref = part if ref is None else {k: ref[k] + part[k] for k in ref}
    log(f"  oracle over {len(kept)} kept blocks")
    check(gpu, ref, BF16_MFMA_TOL, "headline all blocks")


def test_bwd_unsorted_anchors_take_the_atomic_path():
    """Kept anchors out of order within a sample: the MFMA path detects it
    and sums the c^KV / k^R shares with atomics; the result still matches."""
    wl = wk.scaled(3, S=640, N=16)
    anchors, keep = wl.anchors.copy(), wl.keep.copy()
    rng = np.random.default_rng(5)
    for b in range(wl.B):
        anchors[b] = anchors[b][rng.permutation(wl.N)]
    assert any(np.any(np.diff(anchors[b][keep[b] == 1]) < 0) for b in range(wl.B))
    dout = wk.make_dout(wl, seed=16)
    gpu = GpuBwd(wl, dout, anchors, keep).run().result()
    ref = O.backward(wl, dout, anchors=anchors, keep=keep, form="gathered")
    check(gpu, ref, BF16_MFMA_TOL, "unsorted anchors")
    unreached_rows_are_zero(gpu, wl, anchors, keep)


def test_bwd_sorted_path_is_deterministic():
    """Ascending anchors: every sum is taken in a fixed order, so two calls
    give identical bits."""
    wl = wk.scaled(4, S=1024, N=40)
    run = GpuBwd(wl, wk.make_dout(wl, seed=17), wl.anchors, wl.keep)
    a = run.run().result()
    b = run.run().result()
    for k in GRADS:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("generic", [False, True])
def test_bwd_reusing_the_forward_workspace_is_bit_identical(generic):
    """A training step: the forward on the backward's workspace, then the
    backward with reuse_forward (no index build, no q_abs recompute, the
    forward's o_lat for dW_UV) gives the same bits as a backward on its own,
    except dW_UV on the MFMA path (the forward's o_lat rows against the
    backward's own recomputation: bf16 rounding of o_lat at most) and the
    generic path (context sums by atomics: fp32 rounding only)."""
    import torch
    import speculative_decoding_draft_amd as sd
    wl = wk.config(1) if generic else wk.scaled(4, S=700, N=24)
    t = upload_layer(wl)
    a, k = upload_anchors(wl.anchors, wl.keep)
    desc = desc_for(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dout_np = wk.make_dout(wl, seed=11)
    dout = torch.from_numpy(dout_np)
    dout = (dout.view(torch.bfloat16) if wl.dtype == "bf16" else dout).cuda()
    B, S, L5, H = wl.B, wl.S, wl.q_len, wl.H
    shapes = {"dq_nope": (B, L5, H, wl.d_c), "dq_rope": (B, L5, H, wl.d_r),
              "dckv_ctx": (B, S, wl.D), "dkr_ctx": (B, S, wl.d_r),
              "dckv_blk": (B, L5, wl.D), "dkr_blk": (B, L5, wl.d_r),
              "dw_uk": (H, wl.d_c, wl.D), "dw_uv": (H, wl.d_v, wl.D)}
    ws = torch.empty(sd.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    ins = (t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"], t["kr_blk"],
           t["w_uk"], t["w_uv"], a, k)
    plain = {n: torch.full(v, float("nan"), dtype=tdt, device="cuda") for n, v in shapes.items()}
    sd.attn_bwd(desc, *ins, dout, plain, ws, force_generic=generic)
    ws.fill_(0x7f)                              # nothing left over from the plain call
    out = torch.empty((B, L5, H, wl.d_v), dtype=tdt, device="cuda")
    sd.attn_fwd(desc, *ins, out, ws, force_generic=generic)
    reuse = {n: torch.full(v, float("nan"), dtype=tdt, device="cuda") for n, v in shapes.items()}
    sd.attn_bwd(desc, *ins, dout, reuse, ws, force_generic=generic, reuse_forward=True)
    torch.cuda.synchronize()
    for n in shapes:
        x, y = plain[n].double(), reuse[n].double()
        if generic:
            assert float((x - y).norm() / y.norm()) < 1e-6, n
        elif n == "dw_uv":
            assert float((x - y).norm() / y.norm()) < 5e-3, n
        else:
            assert torch.equal(plain[n], reuse[n]), n
    # the forward also leaving its probabilities, the backward reading them
    # (reuse_forward 2) instead of recomputing the scores: the same P, so the
    # same bits as reuse_forward 1 (the generic path has no P to leave and
    # takes the same launches as with 1)
    ws.fill_(0x7f)
    sd.attn_fwd(desc, *ins, out, ws, force_generic=generic, for_backward=True)
    with_p = {n: torch.full(v, float("nan"), dtype=tdt, device="cuda") for n, v in shapes.items()}
    sd.attn_bwd(desc, *ins, dout, with_p, ws, force_generic=generic, reuse_forward=2)
    st, _ = sd.read_device_status(ws)
    assert st == sd.DSPARK_OK, sd.last_error()
    torch.cuda.synchronize()
    for n in shapes:
        if generic:
            x, y = with_p[n].double(), reuse[n].double()
            assert float((x - y).norm() / y.norm()) < 1e-6, n
        else:
            assert torch.equal(with_p[n], reuse[n]), n


def test_bwd_reuse_of_probabilities_needs_a_forward_that_left_them():
    """reuse_forward 2 after a forward without for_backward: reported
    (EINVAL, NaN gradients); a forward with for_backward then makes it work.
    A forward with for_backward needs a backward's workspace and the
    three-kernel path."""
    import torch
    import speculative_decoding_draft_amd as sd
    wl = wk.scaled(4, S=700, N=24)
    desc, ins, dout, g, out = _bwd_setup(wl)
    ws = torch.full((sd.bwd_workspace_size(desc),), 0x7f, dtype=torch.uint8, device="cuda")
    sd.attn_fwd(desc, *ins, out, ws)
    sd.attn_bwd(desc, *ins, dout, g, ws, reuse_forward=2)
    st, _ = sd.read_device_status(ws)
    assert st == sd.DSPARK_EINVAL and "reuse_forward" in sd.last_error()
    for n, v in g.items():
        assert bool(torch.isnan(v).all()), n
    sd.attn_fwd(desc, *ins, out, ws, for_backward=True)
    for v in g.values():
        v.fill_(float("nan"))
    sd.attn_bwd(desc, *ins, dout, g, ws, reuse_forward=2)
    st, _ = sd.read_device_status(ws)
    assert st == sd.DSPARK_OK, sd.last_error()
    for n, v in g.items():
        assert bool(torch.isfinite(v).all()), n
    # a forward-sized workspace is refused, and so is the one-launch forward
    small = torch.empty((sd.workspace_size(desc),), dtype=torch.uint8, device="cuda")
    assert small.numel() < ws.numel()
    with pytest.raises(sd.DSparkError) as e:
        sd.attn_fwd(desc, *ins, out, small, for_backward=True)
    assert e.value.status == sd.DSPARK_EWORKSPACE
    with pytest.raises(sd.DSparkError) as e:
        sd.attn_fwd(desc, *ins, out, ws, for_backward=True, one_launch=True)
    assert e.value.status == sd.DSPARK_EINVAL and "one-launch" in sd.last_error()


def _bwd_setup(wl):
    import torch
    import speculative_decoding_draft_amd as sd
    t = upload_layer(wl)
    a, k = upload_anchors(wl.anchors, wl.keep)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dout = to_torch(wk.make_dout(wl, seed=11), wl.dtype, "cuda")
    B, S, L5, H = wl.B, wl.S, wl.q_len, wl.H
    shapes = {"dq_nope": (B, L5, H, wl.d_c), "dq_rope": (B, L5, H, wl.d_r),
              "dckv_ctx": (B, S, wl.D), "dkr_ctx": (B, S, wl.d_r),
              "dckv_blk": (B, L5, wl.D), "dkr_blk": (B, L5, wl.d_r),
              "dw_uk": (H, wl.d_c, wl.D), "dw_uv": (H, wl.d_v, wl.D)}
    g = {n: torch.full(v, 3.0, dtype=tdt, device="cuda") for n, v in shapes.items()}
    ins = (t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"], t["kr_blk"],
           t["w_uk"], t["w_uv"], a, k)
    out = torch.empty((B, L5, H, wl.d_v), dtype=tdt, device="cuda")
    return desc_for(wl), ins, dout, g, out


@pytest.mark.parametrize("generic", [False, True])
def test_bwd_all_padding_gives_zero_gradients(generic):
    """No kept block: every gradient is exactly 0 and the status is OK."""
    import torch
    import speculative_decoding_draft_amd as sd
    wl = wk.make_workload("bwd-all-pad", B=2, S=256, N=12, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=84)
    wl.keep[:] = 0
    wl.anchors[:] = -4
    desc, ins, dout, g, _ = _bwd_setup(wl)
    ws = torch.empty(sd.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    sd.attn_bwd(desc, *ins, dout, g, ws, force_generic=generic)
    st, fb = sd.read_device_status(ws)
    assert st == sd.DSPARK_OK and fb == -1, sd.last_error()
    for n, v in g.items():
        assert bool((v == 0).all()), n


@pytest.mark.parametrize("case", ["fresh-workspace", "one-launch-forward", "generic-forward",
                                  "generic-backward", "other-shape"])
def test_bwd_reuse_forward_without_a_matching_forward_is_reported(case):
    """reuse_forward on a workspace whose last index build was not a forward
    of this descriptor on the backward's path: every gradient is NaN and the
    status is DSPARK_EINVAL; a matching forward afterwards makes the same
    call succeed again."""
    import torch
    import speculative_decoding_draft_amd as sd
    wl = wk.scaled(4, S=700, N=24)
    desc, ins, dout, g, out = _bwd_setup(wl)
    other = wk.scaled(4, S=700, N=32)
    desc2, ins2, _, _, out2 = _bwd_setup(other)
    n_ws = max(sd.bwd_workspace_size(desc), sd.workspace_size(desc),
               sd.bwd_workspace_size(desc2), sd.workspace_size(desc2))
    ws = torch.full((n_ws,), 0x7f, dtype=torch.uint8, device="cuda")
    generic_bwd = case == "generic-backward"
    log(f"reuse mismatch: {case}")
    if case == "one-launch-forward":
        sd.attn_fwd(desc, *ins, out, ws, one_launch=True)
    elif case == "generic-forward":
        sd.attn_fwd(desc, *ins, out, ws, force_generic=True)
    elif case == "generic-backward":
        sd.attn_fwd(desc, *ins, out, ws)
    elif case == "other-shape":
        sd.attn_fwd(desc2, *ins2, out2, ws)
    sd.attn_bwd(desc, *ins, dout, g, ws, force_generic=generic_bwd, reuse_forward=True)
    st, _ = sd.read_device_status(ws)
    assert st == sd.DSPARK_EINVAL, (st, sd.last_error())
    assert "reuse_forward" in sd.last_error()
    for n, v in g.items():
        assert bool(torch.isnan(v).all()), n
    # the matching forward, then the same backward: finite gradients, OK
    sd.attn_fwd(desc, *ins, out, ws, force_generic=generic_bwd)
    for v in g.values():
        v.fill_(float("nan"))
    sd.attn_bwd(desc, *ins, dout, g, ws, force_generic=generic_bwd, reuse_forward=True)
    st, _ = sd.read_device_status(ws)
    assert st == sd.DSPARK_OK, sd.last_error()
    for n, v in g.items():
        assert bool(torch.isfinite(v).all()), n
