"""Pins of the oracle's output head and loss (§5 "输出头", §6 "训练目标" of the
GLM 5.2 DSpark training-design page).

Each part is checked against something other than its own formula: torch's
cross_entropy / binary_cross_entropy_with_logits / linear / embedding, the
acceptance worked example of the explainer page, the total-variation
identity, closed forms (flat logits, identical draft and teacher), eval masks
worked out by hand from the §6 rule, and the page's Markov parameter count.
"""
import copy

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wk
from conftest import golden

DIMS = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)


def small(seed=3, B=2, S=64, N=6, V=300, d=24, r=8, recipe="headline"):
    args = {"headline": dict(low_frac=0.5)}.get(recipe, {})
    wl = wk.make_workload("s", B=B, S=S, N=N, dims=DIMS, dtype="f32", recipe=recipe, seed=seed,
                          recipe_args=args, tensors=False)
    return wl, wk.make_loss_inputs(wl, V, d, r, seed=seed + 1)


def test_eval_mask_hand_cases():
    # S = 12; loss_mask[3] = 0; loss_mask[11] is forced to 0 on read.
    lm = np.array([[1, 1, 1, 0, 1, 1, 1, 1, 1, 1, 1, 1]], np.uint8)
    anchors = np.array([[0, 3, 7, 9, 10, 2, -1, 4]], np.int32)
    keep = np.array([[1, 1, 1, 1, 1, 1, 0, 0]], np.uint8)
    want = np.array([[
        [1, 1, 0, 0, 0],   # A=0: x1, x2 counted; loss_mask[3] = 0 stops the block
        [1, 1, 1, 1, 1],   # A=3: labels x4..x8 all inside and unmasked
        [1, 1, 1, 0, 0],   # A=7: x8..x10; x11 is the last token (forced off)
        [1, 0, 0, 0, 0],   # A=9: x10, then x11 off
        [0, 0, 0, 0, 0],   # A=10: y_0 = x11 is off
        [0, 0, 0, 0, 0],   # A=2: y_0 = x3 is masked; the cumprod keeps the rest off
        [0, 0, 0, 0, 0],   # padding block (garbage anchor)
        [0, 0, 0, 0, 0],   # padding block (valid-looking anchor)
    ]], np.uint8)
    np.testing.assert_array_equal(O.eval_mask(lm, anchors, keep), want)
    # the caller's array is not modified
    assert lm[0, 11] == 1


def test_acceptance_worked_example():
    g = {r[0]: [float(x) for x in r[1:]] for r in golden("acceptance_worked_example.txt")}
    p, q = np.array(g["p"]), np.array(g["q"])
    # draft logits log q, teacher logits log p (any shift is immaterial)
    ce, l1, a, bce = O.step_terms(np.log(q)[None] + 3.0, np.log(p)[None] - 1.0, [1], [0.0])
    assert abs(np.minimum(p, q).sum() - g["acceptance"][0]) < 1e-15
    np.testing.assert_allclose(l1, [2 * (1 - g["acceptance"][0])], rtol=1e-12)
    np.testing.assert_allclose(a, [g["acceptance"][0]], rtol=1e-12)
    np.testing.assert_allclose(ce, [-np.log(0.35)], rtol=1e-12)
    np.testing.assert_allclose(bce, [np.log(2.0)], rtol=1e-12)   # c = 0: log 2 for any target


def test_acceptance_example_through_the_whole_head():
    """V = 3, d = 3, lm_head = I, Markov weights 0: draft row log q, teacher
    row log p -> l1 = 0.1, a = 0.95 on the one counted step.  The inputs are
    stored in fp32, so the logs carry a rounding of ~3e-8 relative."""
    g = {r[0]: [float(x) for x in r[1:]] for r in golden("acceptance_worked_example.txt")}
    p, q = np.array(g["p"]), np.array(g["q"])
    S, N = 8, 1
    lh = wk.LossInputs(vocab=3, hidden=3, rank=2, dtype="f32",
                       input_ids=np.array([[0, 1, 2, 0, 1, 2, 0, 1]], np.int32),
                       h_final=np.zeros((1, 5, 3), np.float32), z=np.zeros((1, S, 3), np.float32),
                       w_lm=np.eye(3, dtype=np.float32), w_m1=np.ones((3, 2), np.float32),
                       w_m2=np.zeros((3, 2), np.float32), w_conf=np.zeros(5, np.float32))
    lh.h_final[0, 0] = np.log(q)
    lh.z[0, 2] = np.log(p)
    lm = np.array([[1, 1, 1, 1, 0, 1, 1, 1]], np.uint8)       # only step 0 (label x3) counts
    r = O.loss_head(lh, lm, np.array([[2]], np.int32), np.array([[1]], np.uint8))
    assert r["eval_mask"].tolist() == [[[1, 0, 0, 0, 0]]]
    assert abs(r["l1"][0, 0, 0] - 0.1) < 1e-7 and abs(r["mean_l1"] - 0.1) < 1e-7
    assert abs(r["ce"][0, 0, 0] + np.log(q[0])) < 1e-7           # y_0 = x3 = token 0
    assert abs(r["bce"][0, 0, 0] - np.log(2.0)) < 1e-12
    assert abs(r["total"] - (-np.log(q[0]) + 0.9 * 0.1 + np.log(2.0))) < 1e-7


def test_l1_is_twice_the_total_variation():
    rng = np.random.default_rng(5)
    L, T = 3 * rng.standard_normal((7, 50)), 3 * rng.standard_normal((7, 50))
    _, l1, a, _ = O.step_terms(L, T, np.zeros(7, int), np.zeros(7))
    p, q = torch.softmax(torch.from_numpy(L), 1), torch.softmax(torch.from_numpy(T), 1)
    ov = torch.minimum(p, q).sum(1).numpy()
    np.testing.assert_allclose(l1, 2 * (1 - ov), rtol=1e-12)
    np.testing.assert_allclose(a, ov, rtol=1e-12)                # a = sum min(p, q)
    assert np.all((l1 > 0) & (l1 < 2))


def test_head_matches_a_torch_recomputation():
    """lm_head, Markov head, confidence head and the three terms recomputed
    with torch's fp64 linear / embedding / cross_entropy /
    binary_cross_entropy_with_logits, per counted step."""
    wl, lh = small(seed=11)
    r = O.loss_head(lh, wl.loss_mask, wl.anchors, wl.keep)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    F = torch.nn.functional
    m = r["eval_mask"]
    ce_s = l1_s = bce_s = 0.0
    for b, n, k in zip(*np.nonzero(m)):
        A = int(wl.anchors[b, n])
        prev = torch.tensor([int(lh.input_ids[b, A + k])])
        emb = F.embedding(prev, t(lh.w_m1))
        hrow = t(lh.h_final[b, 5 * n + k])[None]
        L = F.linear(hrow, t(lh.w_lm)) + F.linear(emb, t(lh.w_m2))
        T = F.linear(t(lh.z[b, A + k])[None], t(lh.w_lm))
        y = torch.tensor([int(lh.input_ids[b, A + k + 1])])
        ce = F.cross_entropy(L, y).item()
        l1 = (torch.softmax(L, 1) - torch.softmax(T, 1)).abs().sum().item()
        c = F.linear(torch.cat([hrow, emb], 1), t(lh.w_conf)[None]).item()
        a = min(max(1 - l1 / 2, 0.0), 1.0)
        bce = F.binary_cross_entropy_with_logits(torch.tensor([c], dtype=torch.float64),
                                                 torch.tensor([a], dtype=torch.float64)).item()
        for key, v in (("ce", ce), ("l1", l1), ("conf", c), ("bce", bce)):
            assert abs(r[key][b, n, k] - v) < 1e-10 * max(1, abs(v)), (key, b, n, k)
        ce_s, l1_s, bce_s = ce_s + ce, l1_s + l1, bce_s + bce
    cnt = int(m.sum())
    assert cnt == r["count"] and cnt > 10
    assert abs(r["total"] - (ce_s + 0.9 * l1_s + bce_s) / cnt) < 1e-10
    # steps the mask turns off carry 0
    for key in ("ce", "l1", "conf", "bce"):
        assert np.all(r[key][m == 0] == 0)


def test_closed_forms_flat_and_identical():
    wl, lh = small(seed=13)
    # lm_head = 0 and Markov bias 0: every distribution is uniform: ce = log V, l1 = 0
    flat = copy.copy(lh)
    flat.w_lm = np.zeros_like(lh.w_lm)
    flat.w_m2 = np.zeros_like(lh.w_m2)
    r = O.loss_head(flat, wl.loss_mask, wl.anchors, wl.keep)
    m = r["eval_mask"] == 1
    np.testing.assert_allclose(r["ce"][m], np.log(lh.vocab), rtol=1e-13)
    np.testing.assert_allclose(r["l1"][m], 0.0, atol=1e-15)
    # draft row = teacher row and no Markov bias: p = q, l1 = 0, a = 1, bce = log(1 + e^-c)
    same = copy.copy(lh)
    same.w_m2 = np.zeros_like(lh.w_m2)
    same.h_final = lh.h_final.copy()
    for b in range(wl.B):
        for n in range(wl.N):
            A = int(wl.anchors[b, n])
            if wl.keep[b, n] and 0 <= A <= wl.S - 2:
                for k in range(5):
                    if A + k < wl.S:
                        same.h_final[b, 5 * n + k] = lh.z[b, A + k]
    r = O.loss_head(same, wl.loss_mask, wl.anchors, wl.keep)
    m = r["eval_mask"] == 1
    np.testing.assert_allclose(r["l1"][m], 0.0, atol=1e-14)
    np.testing.assert_allclose(r["bce"][m], np.log1p(np.exp(-r["conf"][m])), rtol=1e-12)


def test_markov_bias_depends_only_on_prev():
    """B(prev) does not read H^(L); with H^(L) = 0 the draft logits are the
    Markov bias alone: markov_w1[prev] markov_w2^T."""
    rng = np.random.default_rng(2)
    w_lm, w1, w2 = rng.standard_normal((40, 6)), rng.standard_normal((40, 4)), rng.standard_normal((40, 4))
    prev = np.array([3, 3, 17])
    L0 = O.draft_logits(np.zeros((3, 6)), prev, w_lm, w1, w2)
    np.testing.assert_allclose(L0[0], L0[1])
    np.testing.assert_allclose(L0[2], w2 @ w1[17], rtol=1e-13)
    h = rng.standard_normal((3, 6))
    np.testing.assert_allclose(O.draft_logits(h, prev, w_lm, w1, w2) - L0, h @ w_lm.T, rtol=1e-12)


def test_markov_shapes_match_the_parameter_table():
    """markov_w1 and markov_w2 of [V, r] each: 2 V r = 79.3 M parameters, the
    page's 79 M; the confidence head's d + r weights are below 0.1 M."""
    g = {r[0]: float(r[1]) for r in golden("param_table.txt")}
    V, r, d = g["vocab"], g["markov_rank"], g["d"]
    assert round(2 * V * r / 1e6) == g["markov_M"]
    assert d + r < 0.1e6


def test_bad_anchor_poisons_its_block_and_the_means():
    wl, lh = small(seed=17)
    anchors = wl.anchors.copy()
    b, n = [(b, n) for b in range(wl.B) for n in range(wl.N) if wl.keep[b, n]][0]
    anchors[b, n] = wl.S - 1
    r = O.loss_head(lh, wl.loss_mask, anchors, wl.keep)
    assert np.all(np.isnan(r["ce"][b, n])) and r["eval_mask"][b, n].sum() == 0
    assert np.isnan(r["total"])
