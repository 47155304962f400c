"""Parity of the MLA block of a draft layer (dspark_mla_layer_fwd through the
C ABI) with the oracle's layer_forward, on the same seeded inputs.

Compared per kept row: the output out = H + o_proj(attention), and the delta
out - H (the block's contribution, smaller than H).  Rows of padding blocks
must equal H bit for bit (their attention rows are 0).

Tolerances: fp32 (generic attention, fp32 rocBLAS GEMMs): rel-L2 <= 2e-5 on
the delta.  bf16: every intermediate (normalised h, c^Q, q, [c^KV ; k^R],
the attention output) and the output are rounded to bf16.  The output is
held to rel-L2 <= 5e-3.  The delta carries the attention's error (rel-L2
~3e-3 on its bf16 output) and the projections' roundings, within 1e-2, plus
the rounding of out itself, whose RMS is 2^-9/sqrt(3) |out| ~ 1.13e-3 |H| and
so 1.13e-3 |H| / |delta| relative to the delta: the delta's bound is
1e-2 + 2 x 1.13e-3 |H| / |delta| (about 2.4e-2 where |delta| / |H| = 0.16).
"""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from gpu_util import anchors_for, desc_for, log
from workloads.device import to_torch, upload_anchors, upload_layer

pytestmark = pytest.mark.gpu

TINY = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)


def run_layer(wl, li, anchors, keep, force_generic=False, max_kept=0, want_status=False):
    import torch
    import speculative_decoding_draft_amd as sd
    t = upload_layer(wl)
    desc = sd.make_layer_desc(desc_for(wl), li.hidden, li.q_rank, li.rms_eps, max_kept)
    w = {k: to_torch(getattr(li, k), wl.dtype, "cuda") for k in ("g_in", "w_qa", "g_qa", "w_qb",
                                                                 "w_kva", "g_kva", "w_o")}
    w["w_uk"], w["w_uv"] = t["w_uk"], t["w_uv"]
    hd = to_torch(li.h_draft, wl.dtype, "cuda")
    hc = to_torch(li.h_ctx, wl.dtype, "cuda")
    a, k = upload_anchors(anchors, keep)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = torch.full(hd.shape, float("nan"), dtype=tdt, device="cuda")
    ws = torch.empty(sd.layer_workspace_size(desc), dtype=torch.uint8, device="cuda")
    sd.mla_layer_fwd(desc, hd, hc, w, a, k, out, ws, force_generic=force_generic)
    st = sd.layer_read_status(ws)
    torch.cuda.synchronize()
    if want_status:
        return out.float().cpu().numpy().astype(np.float64), ws, st
    assert st[0] == sd.DSPARK_OK, st
    return out.float().cpu().numpy().astype(np.float64), ws


def check(wl, li, gpu, ref, keep, tol_delta, tol_out, what):
    H = O.dspark_oracle._f64(li.h_draft, wl.dtype)
    kept = np.repeat(keep.astype(bool), 5, axis=1)
    assert np.array_equal(gpu[~kept], H[~kept]), f"{what}: padding rows are not H"
    g, r, h = gpu[kept], ref[kept], H[kept]
    assert np.all(np.isfinite(g))
    rel_out = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    rel_d = float(np.linalg.norm((g - h) - (r - h)) / np.linalg.norm(r - h))
    mx = float(np.abs(g - r).max())
    ratio = float(np.linalg.norm(r - h) / np.linalg.norm(h))
    if wl.dtype == "bf16":          # the output's own rounding, relative to the delta
        tol_delta = tol_delta + 2 * 2.0 ** -9 / np.sqrt(3.0) / ratio
    log(f"  {what}: out rel_l2={rel_out:.3e} delta rel_l2={rel_d:.3e} (bound {tol_delta:.2e}) "
        f"max_abs={mx:.3e} |delta|/|H|={ratio:.3f}")
    assert rel_d <= tol_delta and rel_out <= tol_out, (what, rel_d, rel_out)


def test_layer_tiny_fp32():
    wl = wk.make_workload("tiny-layer", B=1, S=40, N=6, dims=TINY, dtype="f32", recipe="headline",
                          seed=31, recipe_args=dict(low_frac=0.5))
    li = wk.make_layer_inputs(wl, hidden=24, q_rank=12, seed=32)
    gpu, _ = run_layer(wl, li, wl.anchors, wl.keep)
    ref = O.layer_forward(wl, li)
    check(wl, li, gpu, ref, wl.keep, 2e-5, 2e-5, "tiny fp32")


@pytest.mark.parametrize("k,S,N,B", [(2, 2048, 64, None), (4, 600, 24, None), (3, 400, 12, 2)])
def test_layer_glm_dims_bf16(k, S, N, B):
    wl = wk.scaled(k, S=S, N=N, B=B)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=33)
    ga, gk, oa, ok = anchors_for(wl)
    log(f"case {wl.name}")
    gpu, ws = run_layer(wl, li, ga, gk)
    ref = O.layer_forward(wl, li, anchors=oa, keep=ok)
    check(wl, li, gpu, ref, ok, 1e-2, 5e-3, wl.name)


def test_layer_generic_attention_matches():
    """force_generic runs the attention on the generic kernel; the block's
    output agrees with the MFMA path's within the bf16 tolerance."""
    wl = wk.scaled(4, S=300, N=12)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=34)
    a, _ = run_layer(wl, li, wl.anchors, wl.keep)
    b, _ = run_layer(wl, li, wl.anchors, wl.keep, force_generic=True)
    ref = O.layer_forward(wl, li)
    check(wl, li, b, ref, wl.keep, 1e-2, 5e-3, "generic attention")
    kept = np.repeat(wl.keep.astype(bool), 5, axis=1)
    assert np.linalg.norm(a[kept] - b[kept]) / np.linalg.norm(b[kept]) < 5e-3


def test_layer_repeat_runs_are_bit_identical():
    wl = wk.scaled(2, S=512, N=16)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=35)
    ga, gk, _, _ = anchors_for(wl)
    a, _ = run_layer(wl, li, ga, gk)
    b, _ = run_layer(wl, li, ga, gk)
    assert np.array_equal(a, b)


def test_layer_tune_then_forward():
    """dspark_mla_layer_tune returns the block's output like the plain call and
    writes its kernel choices into the caller's table (one per GEMM, with the
    GEMM's shape); later calls given the table give identical bits to each
    other and still match the oracle."""
    import torch
    import speculative_decoding_draft_amd as sd
    wl = wk.scaled(4, S=700, N=20)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=36)
    t = upload_layer(wl)
    desc = sd.make_layer_desc(desc_for(wl), li.hidden, li.q_rank, li.rms_eps)
    w = {k: to_torch(getattr(li, k), wl.dtype, "cuda") for k in ("g_in", "w_qa", "g_qa", "w_qb",
                                                                 "w_kva", "g_kva", "w_o")}
    w["w_uk"], w["w_uv"] = t["w_uk"], t["w_uv"]
    hd, hc = to_torch(li.h_draft, "bf16", "cuda"), to_torch(li.h_ctx, "bf16", "cuda")
    a, k = upload_anchors(wl.anchors, wl.keep)
    ws = torch.empty(sd.layer_workspace_size(desc), dtype=torch.uint8, device="cuda")
    outs = []
    choices = None
    for tune in (True, False, False):
        out = torch.full(hd.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        if tune:
            choices = sd.mla_layer_tune(desc, hd, hc, w, a, k, out, ws)
        else:
            sd.mla_layer_fwd(desc, hd, hc, w, a, k, out, ws, gemm_choices=choices)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy().astype(np.float64))
    table = choices.as_list()
    log(f"  layer GEMM choices {table}")
    assert len(table) == 5
    assert [g[:3] for g in table][:2] == [(5 * wl.B * wl.N, li.q_rank, li.hidden),
                                          (5 * wl.B * wl.N, wl.H * (wl.d_c + wl.d_r), li.q_rank)]
    ref = O.layer_forward(wl, li)
    for o in outs:
        check(wl, li, o, ref, wl.keep, 1e-2, 5e-3, "tuned")
    assert np.array_equal(outs[1], outs[2])


def test_layer_max_kept_blocks_exact_and_overflow():
    """max_kept_blocks = the kept count: the draft-row GEMMs run on the kept
    rows only and the result matches the oracle; one fewer: every row NaN and
    DSPARK_ECAPACITY."""
    import speculative_decoding_draft_amd as sd
    wl = wk.scaled(4, S=600, N=24)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=37)
    kept = int(wl.keep.sum())
    assert kept < wl.N
    gpu, _, st = run_layer(wl, li, wl.anchors, wl.keep, max_kept=kept, want_status=True)
    assert st[0] == sd.DSPARK_OK and st[2] == kept
    ref = O.layer_forward(wl, li)
    check(wl, li, gpu, ref, wl.keep, 1e-2, 5e-3, "max_kept_blocks = kept")
    full, _ = run_layer(wl, li, wl.anchors, wl.keep)
    kept_rows = np.repeat(wl.keep.astype(bool), 5, axis=1)
    assert np.array_equal(gpu[~kept_rows], full[~kept_rows])
    gpu, _, st = run_layer(wl, li, wl.anchors, wl.keep, max_kept=kept - 1, want_status=True)
    assert st[0] == sd.DSPARK_ECAPACITY and st[2] == kept
    assert np.all(np.isnan(gpu))


def test_layer_headline_size_sampled_blocks():
    """The configuration the benchmark times: S = 32768, N = 1024 (768 kept),
    d = 6144, q_lora_rank = 2048, bf16, max_kept_blocks = 768.  The oracle
    checks every row of 6 blocks (the clamped ones at anchors 0, 1 and 126
    among them); padding rows must be exactly H."""
    wl = wk.config(4)
    li = wk.make_layer_inputs(wl, hidden=6144, q_rank=2048, seed=5)
    kept = int(wl.keep.sum())
    gpu, _ = run_layer(wl, li, wl.anchors, wl.keep, max_kept=kept)
    ks = [n for n in range(wl.N) if wl.keep[0, n]]
    low = [n for n in ks if wl.anchors[0, n] in (0, 1, 126)]
    rng = np.random.default_rng(5)
    pick = sorted(set(low) | set(rng.choice([n for n in ks if n not in low], 6 - len(low),
                                             replace=False).tolist()))
    ref = O.layer_forward(wl, li, blocks=[(0, n) for n in pick])
    H = O.dspark_oracle._f64(li.h_draft, wl.dtype)
    pad = np.repeat(~wl.keep.astype(bool), 5, axis=1)
    assert np.array_equal(gpu[pad], H[pad]), "padding rows are not H"
    rows = np.zeros_like(pad)
    for n in pick:
        rows[0, 5 * n:5 * n + 5] = True
    g, r, h = gpu[rows], ref[rows], H[rows]
    assert np.all(np.isfinite(g))
    rel_out = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    rel_d = float(np.linalg.norm((g - h) - (r - h)) / np.linalg.norm(r - h))
    ratio = float(np.linalg.norm(r - h) / np.linalg.norm(h))
    bound = 1e-2 + 2 * 2.0 ** -9 / np.sqrt(3.0) / ratio
    log(f"  headline, {len(pick)} sampled blocks: out rel_l2={rel_out:.3e} "
        f"delta rel_l2={rel_d:.3e} (bound {bound:.2e})")
    assert rel_d <= bound and rel_out <= 5e-3
