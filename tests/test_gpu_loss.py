"""Parity of the output head and loss (dspark_loss_fwd through the C ABI)
with the oracle's loss_head, on the same seeded inputs.

Compared: the eval mask (bit for bit), the per-step terms ce, l1, the
confidence logit and bce on every counted step (0 elsewhere; NaN for a bad
anchor), the number of counted steps (exact) and the three means and the
total.

Tolerances.  Both sides start from the same stored values (bf16 or fp32).
The GPU forms the logits with fp32 accumulation over d + r products and
takes the softmax statistics, L1 and the confidence dot product in fp32; the
oracle does everything in fp64.  A logit's error is a few fp32 roundings of
partial sums of size ~|logit| (~1e-6 relative, up to ~1e-5 absolute for
|logit| ~ 10), and ce, l1 and bce inherit at most that, so 2e-4 absolute on
each term (and 1e-5 relative on the means) bounds them with a wide margin;
l1 carries in addition the fp32 sum of up to V terms (~1e-6 relative).
"""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from gpu_util import log
from workloads.device import upload_loss

pytestmark = pytest.mark.gpu

DIMS = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)
TERM_TOL = 2e-4
MEAN_REL = 1e-5


def run_loss(wl, lh, anchors, keep, max_kept=0, tune=False, loss_mask=None, ws=None,
             layout="dense", max_counted=0):
    """layout: "dense" weights, "fused" (lm_head and markov_w2 side by side in
    one [V, d + r] array: the one-GEMM path), "strided" (padded rows, apart)."""
    import torch
    import speculative_decoding_draft_amd as sd
    from workloads.device import to_torch
    lm = wl.loss_mask if loss_mask is None else loss_mask
    t = upload_loss(lh, lm, anchors, keep)
    d_, r_ = lh.hidden, lh.rank
    lds = (0, 0)
    if layout == "fused":
        buf = to_torch(np.concatenate([lh.w_lm, lh.w_m2], axis=1), lh.dtype, "cuda")
        t["w_lm"], t["w_m2"] = buf, buf[:, d_:]
        lds = (d_ + r_, d_ + r_)
    elif layout == "strided":
        pad = 8
        a = np.zeros((lh.vocab, d_ + pad), lh.w_lm.dtype)
        a[:, :d_] = lh.w_lm
        m = np.zeros((lh.vocab, r_ + pad), lh.w_m2.dtype)
        m[:, :r_] = lh.w_m2
        t["w_lm"], t["w_m2"] = to_torch(a, lh.dtype, "cuda"), to_torch(m, lh.dtype, "cuda")
        lds = (d_ + pad, r_ + pad)
    d = sd.make_loss_desc(wl.B, wl.S, wl.N, lh.vocab, lh.hidden, lh.rank, dtype=lh.dtype,
                          max_kept_blocks=max_kept, w_lm_ld=lds[0], w_m2_ld=lds[1],
                          max_counted_steps=max_counted)
    if ws is None:
        ws = torch.empty(sd.loss_workspace_size(d), dtype=torch.uint8, device="cuda")
    terms = torch.full((4, wl.B, wl.N, 5), 12345.0, dtype=torch.float32, device="cuda")
    em = torch.full((wl.B, wl.N, 5), 7, dtype=torch.uint8, device="cuda")
    loss = torch.full((5,), 12345.0, dtype=torch.float32, device="cuda")
    if tune:
        choices = sd.loss_tune(d, t, terms, em, loss, ws)
        assert 1 <= choices.n_gemms <= 3
        assert all(g[1] == lh.vocab for g in choices.as_list())
    else:
        sd.loss_fwd(d, t, terms, em, loss, ws)
    st = sd.loss_read_status(ws)
    torch.cuda.synchronize()
    return (terms.cpu().numpy().astype(np.float64), em.cpu().numpy(),
            loss.cpu().numpy().astype(np.float64), st, ws)


def check(name, gpu_terms, gpu_em, gpu_loss, ref, tol=TERM_TOL, means=True):
    np.testing.assert_array_equal(gpu_em, ref["eval_mask"])
    m = ref["eval_mask"] == 1
    worst = {}
    for i, k in enumerate(("ce", "l1", "conf", "bce")):
        g, r = gpu_terms[i], ref[k]
        assert np.all(g[~m] == 0), (name, k, "masked-off steps must be 0")
        err = np.abs(g[m] - r[m])
        worst[k] = float(err.max()) if err.size else 0.0
        assert worst[k] <= tol, (name, k, worst[k])
    log(f"  {name}: counted {int(m.sum())} steps; max |err| " +
        " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    if means:
        assert gpu_loss[4] == ref["count"]
        for j, k in ((0, "total"), (1, "mean_ce"), (2, "mean_l1"), (3, "mean_bce")):
            assert abs(gpu_loss[j] - ref[k]) <= MEAN_REL * max(1.0, abs(ref[k])) + 1e-6, (name, k)


def small(seed, B=2, S=64, N=6, V=300, d=24, r=8, dtype="f32", recipe="headline", low_frac=0.5):
    args = {"headline": dict(low_frac=low_frac)}.get(recipe, {})
    wl = wk.make_workload(f"loss-{seed}", B=B, S=S, N=N, dims=DIMS, dtype=dtype, recipe=recipe,
                          seed=seed, recipe_args=args, tensors=False)
    return wl, wk.make_loss_inputs(wl, V, d, r, seed=seed + 1)


@pytest.mark.parametrize("V,d,r", [(300, 24, 8), (301, 10, 3), (8192 + 20, 32, 8), (1, 12, 4)])
def test_loss_small_fp32(V, d, r):
    """fp32 storage; V not a multiple of 4 (scalar statistics loads), d and r
    whose rows are not 16-byte multiples (scalar gather), V spanning two
    statistics chunks with a ragged tail, and a one-token vocabulary (CE and
    L1 are 0, the confidence target 1)."""
    wl, lh = small(41, V=V, d=d, r=r)
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep)
    assert st[0] == 0, st
    check(f"fp32 V={V} d={d} r={r}", terms, em, loss, O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep))


@pytest.mark.parametrize("V", [20000, 8192 * 3])
def test_loss_glm_width_bf16(V):
    """GLM-5.2 widths (d = 6144, r = 256) in bf16, headline anchor recipe
    (padding slots, clamped windows), B = 2."""
    wl = wk.scaled(4, S=1024, N=24, B=2)
    lh = wk.make_loss_inputs(wl, V, 6144, 256, seed=43)
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep)
    assert st[0] == 0, st
    assert st[2] == int(wl.keep.sum())
    check(f"bf16 V={V}", terms, em, loss, O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep))


def test_loss_row_bounds_exact_and_overflow():
    """max_kept_blocks = the kept count, and max_counted_steps = the counted
    steps (read back from the status area): the oracle's result; one row
    fewer than the counted steps: every output NaN and DSPARK_ECAPACITY."""
    import speculative_decoding_draft_amd as sd
    wl, lh = small(45, B=2, N=8, S=96, dtype="bf16", V=1000, d=64, r=16)
    kept = int(wl.keep.sum())
    ref = O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep)
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep, max_kept=kept)
    assert st[0] == 0 and st[2] == kept and st[3] == ref["count"]
    check("max_kept_blocks = kept", terms, em, loss, ref)
    counted = st[3]
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep, max_counted=counted)
    assert st[0] == 0
    check("max_counted_steps = counted", terms, em, loss, ref)
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep, max_counted=counted - 1)
    assert st[0] == sd.DSPARK_ECAPACITY and st[3] == counted
    assert np.all(np.isnan(terms)) and np.all(np.isnan(loss[:4]))


def test_loss_bad_anchor_and_bad_token():
    import speculative_decoding_draft_amd as sd
    wl, lh = small(47, dtype="bf16", V=500, d=32, r=8)
    anchors = wl.anchors.copy()
    b, n = [(b, n) for b in range(wl.B) for n in range(wl.N) if wl.keep[b, n]][1]
    anchors[b, n] = wl.S - 1
    ref = O.loss_head(lh, wl.loss_mask, anchors, wl.keep)
    terms, em, loss, st, _ = run_loss(wl, lh, anchors, wl.keep)
    assert st[0] == sd.DSPARK_EANCHOR and st[1] == b * wl.N + n
    assert np.all(np.isnan(terms[:, b, n])) and np.all(np.isnan(loss[:4]))
    ok = np.ones_like(wl.keep, dtype=bool)
    ok[b, n] = False
    m = (ref["eval_mask"] == 1) & ok[..., None]
    for i, k in enumerate(("ce", "l1", "conf", "bce")):
        assert np.abs(terms[i][m] - ref[k][m]).max() <= TERM_TOL
    # a label id outside [0, V): status EINVAL, loss NaN
    bad = wk.LossInputs(**{**lh.__dict__, "input_ids": lh.input_ids.copy()})
    bb, nn, kk = [tuple(x) for x in np.argwhere(ref["eval_mask"] == 1)][0]
    bad.input_ids[bb, int(wl.anchors[bb, nn]) + kk + 1] = lh.vocab + 3
    terms, em, loss, st, _ = run_loss(wl, bad, wl.anchors, wl.keep)
    assert st[0] == sd.DSPARK_EINVAL and np.all(np.isnan(loss[:4]))


def test_loss_identical_draft_and_teacher_and_empty_mask():
    """H^(L) rows equal to z_{A+k} and no Markov bias: l1 = 0 and a = 1 on
    every counted step.  An all-zero loss mask counts nothing: loss 0."""
    wl, lh = small(49, dtype="bf16", V=2000, d=64, r=16)
    same = wk.LossInputs(**{**lh.__dict__, "h_final": lh.h_final.copy(),
                            "w_m2": np.zeros_like(lh.w_m2)})
    for b in range(wl.B):
        for n in range(wl.N):
            A = int(wl.anchors[b, n])
            if wl.keep[b, n] and 0 <= A <= wl.S - 2:
                for k in range(5):
                    same.h_final[b, 5 * n + k] = lh.z[b, min(A + k, wl.S - 1)]
    ref = O.loss_head(same, wl.loss_mask, wl.anchors, wl.keep)
    terms, em, loss, st, _ = run_loss(wl, same, wl.anchors, wl.keep)
    check("identical rows", terms, em, loss, ref)
    m = ref["eval_mask"] == 1
    assert np.abs(terms[1][m]).max() < 1e-5
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep,
                                      loss_mask=np.zeros_like(wl.loss_mask))
    assert st[0] == 0 and np.all(em == 0) and np.all(terms == 0) and np.all(loss == 0)


def test_loss_tune_then_repeat_is_bit_identical():
    wl, lh = small(51, B=1, S=512, N=16, dtype="bf16", V=5000, d=256, r=32, low_frac=0.25)
    a = run_loss(wl, lh, wl.anchors, wl.keep, tune=True)
    b = run_loss(wl, lh, wl.anchors, wl.keep, ws=a[4])
    c = run_loss(wl, lh, wl.anchors, wl.keep, ws=a[4])
    check("tuned", a[0], a[1], a[2], O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep))
    assert np.array_equal(b[0], c[0]) and np.array_equal(b[2], c[2])


def test_loss_headline_size_sampled_blocks():
    """The configuration the benchmark times: S = 32768, N = 1024 (768 kept),
    V = 154880, d = 6144, r = 256, bf16, max_kept_blocks = the kept count.
    The oracle checks every step of 8 blocks (the clamped ones at anchors 0,
    1 and 126 among them); the means are checked against the GPU's own terms
    and the exact count."""
    wl = wk.config(4, tensors=False)
    lh = wk.make_loss_inputs(wl, 154880, 6144, 256, seed=9)
    kept = int(wl.keep.sum())
    counted = int(O.eval_mask(wl.loss_mask, wl.anchors, wl.keep).sum())
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep, max_kept=kept,
                                      max_counted=counted)
    assert st[0] == 0 and st[2] == kept and st[3] == counted
    ks = [n for n in range(wl.N) if wl.keep[0, n]]
    low = [n for n in ks if wl.anchors[0, n] in (0, 1, 126)]
    rng = np.random.default_rng(3)
    pick = sorted(set(low) | set(rng.choice([n for n in ks if n not in low], 8 - len(low),
                                             replace=False).tolist()))
    ref = O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep, blocks=[(0, n) for n in pick])
    np.testing.assert_array_equal(em, ref["eval_mask"])
    sub = np.zeros_like(ref["eval_mask"])
    sub[0, pick] = ref["eval_mask"][0, pick]
    worst = 0.0
    for i, k in enumerate(("ce", "l1", "conf", "bce")):
        err = np.abs(terms[i][sub == 1] - ref[k][sub == 1])
        worst = max(worst, float(err.max()))
        assert err.max() <= TERM_TOL, k
    log(f"  headline: {int(sub.sum())} sampled steps, max |err| {worst:.2e}")
    m = ref["eval_mask"] == 1
    cnt = int(m.sum())
    assert loss[4] == cnt
    means = [terms[i][m].sum() / cnt for i in (0, 1, 3)]
    total = means[0] + 0.9 * means[1] + means[2]
    for got, want in zip(loss[:4], [total] + means):
        assert abs(got - want) <= 1e-5 * abs(want)


@pytest.mark.parametrize("layout,dtype", [("fused", "bf16"), ("strided", "bf16"), ("fused", "f32")])
def test_loss_weight_layouts(layout, dtype):
    """lm_head and markov_w2 side by side (one GEMM over [H | e ; z | 0]) and
    padded row strides (three GEMMs) give the oracle's terms."""
    if dtype == "bf16":
        wl = wk.scaled(4, S=1024, N=24)
        lh = wk.make_loss_inputs(wl, 20000, 6144, 256, seed=53)
    else:
        wl, lh = small(53, V=3000, d=32, r=8)
    kept = int(wl.keep.sum())
    terms, em, loss, st, _ = run_loss(wl, lh, wl.anchors, wl.keep, max_kept=kept, layout=layout)
    assert st[0] == 0, st
    check(f"{layout} {dtype}", terms, em, loss, O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep))
