"""Pins of the oracle's MLA block (§4 "MLA Projection": RMSNorms, low-rank
projections, attention, o_proj into the residual).

The projections are library matmuls and the attention is pinned on its own
(test_oracle_pins.py); these check the parts the block adds against a library
routine, closed forms and structural identities.
"""
import copy

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wk

DIMS = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)


def small(recipe="headline", seed=3, hidden=24, q_rank=12, B=1, S=40, N=6):
    args = {"headline": dict(low_frac=0.5), "uniform": dict(n_forced_low=1)}.get(recipe, {})
    wl = wk.make_workload("s", B=B, S=S, N=N, dims=DIMS, dtype="f32", recipe=recipe, seed=seed,
                          recipe_args=args)
    return wl, wk.make_layer_inputs(wl, hidden, q_rank, seed=seed + 1)


def test_rmsnorm_matches_torch_and_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33)) * 3.0
    g = 1.0 + 0.1 * rng.standard_normal(33)
    for eps in (0.0, 1e-6, 0.5):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g),
                                           eps=eps).numpy()
        np.testing.assert_allclose(O.rmsnorm(x, g, eps), ref, rtol=1e-13, atol=1e-13)
    # g = 1: mean(y^2) = m / (m + eps) with m = mean(x^2); eps = 0: scale invariant
    m = np.mean(x * x, axis=1)
    y = O.rmsnorm(x, np.ones(33), 0.5)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m / (m + 0.5), rtol=1e-13)
    np.testing.assert_allclose(O.rmsnorm(5.0 * x, g, 0.0), O.rmsnorm(x, g, 0.0), rtol=1e-13)


def test_zero_o_proj_is_the_identity_and_output_is_linear_in_w_o():
    wl, li = small()
    kept = np.repeat(wl.keep.astype(bool), 5, axis=1)
    base = O.layer_forward(wl, li)
    H = li.h_draft.astype(np.float64)
    z = copy.copy(li)
    z.w_o = np.zeros_like(li.w_o)
    np.testing.assert_array_equal(O.layer_forward(wl, z)[kept], H[kept])
    d = copy.copy(li)
    d.w_o = 2.0 * li.w_o
    np.testing.assert_allclose(O.layer_forward(wl, d)[kept] - H[kept], 2.0 * (base[kept] - H[kept]),
                               rtol=1e-12, atol=1e-12)
    assert np.all(np.isnan(base[~kept]))


def test_block_rows_depend_only_on_their_own_inputs():
    """A draft row's output uses its own block's hidden rows (queries and
    block keys) and the context; changing another block's draft rows leaves
    it unchanged (the projections are row-wise, the mask has no cross-block
    visibility)."""
    wl, li = small(seed=7)
    kept_n = [n for n in range(wl.N) if wl.keep[0, n]]
    n0, n1 = kept_n[0], kept_n[-1]
    base = O.layer_forward(wl, li)
    ch = copy.copy(li)
    ch.h_draft = li.h_draft.copy()
    ch.h_draft[0, 5 * n1:5 * n1 + 5] += 1.0
    out = O.layer_forward(wl, ch)
    np.testing.assert_array_equal(out[0, 5 * n0:5 * n0 + 5], base[0, 5 * n0:5 * n0 + 5])
    assert not np.allclose(out[0, 5 * n1:5 * n1 + 5], base[0, 5 * n1:5 * n1 + 5])


def test_library_torch_recomputation_of_the_projections():
    """The same block with torch's fp64 rms_norm / linear layers for every
    projection, feeding the pinned attention oracle, gives the same output."""
    wl, li = small(seed=11, recipe="uniform", N=4, S=48)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    lin = torch.nn.functional.linear
    rn = torch.nn.functional.rms_norm
    Hd, Hc = t(li.h_draft), t(li.h_ctx)
    h = rn(Hd, (li.hidden,), t(li.g_in), eps=li.rms_eps)
    cq = rn(lin(h, t(li.w_qa)), (li.q_rank,), t(li.g_qa), eps=li.rms_eps)
    q = lin(cq, t(li.w_qb)).reshape(wl.B, 5 * wl.N, wl.H, wl.d_c + wl.d_r).numpy()
    kv_c, kv_b = lin(Hc, t(li.w_kva)).numpy(), lin(h, t(li.w_kva)).numpy()
    D = wl.D
    sub = copy.copy(wl)
    sub.layers = [type(wl.layers[0])(
        q_nope=q[..., :wl.d_c], q_rope=q[..., wl.d_c:],
        ckv_ctx=rn(t(kv_c[..., :D]), (D,), t(li.g_kva), eps=li.rms_eps).numpy(),
        kr_ctx=kv_c[..., D:],
        ckv_blk=rn(t(kv_b[..., :D]), (D,), t(li.g_kva), eps=li.rms_eps).numpy(),
        kr_blk=kv_b[..., D:], w_uk=wl.layers[0].w_uk, w_uv=wl.layers[0].w_uv)]
    o = O.forward(sub, form="dense")
    ref = li.h_draft + lin(t(o.reshape(wl.B, 5 * wl.N, -1)), t(li.w_o)).numpy()
    got = O.layer_forward(wl, li)
    kept = np.repeat(wl.keep.astype(bool), 5, axis=1)
    np.testing.assert_allclose(got[kept], ref[kept], rtol=1e-11, atol=1e-11)


def test_block_restriction_matches_the_full_block():
    """layer_forward(blocks=...) projects only the sampled blocks' rows and
    their windows; their output rows equal the full computation's."""
    wl, li = small(seed=19, B=2, N=6, S=48)
    full = O.layer_forward(wl, li)
    kept = [(b, n) for b in range(wl.B) for n in range(wl.N) if wl.keep[b, n]]
    pick = kept[::2]
    part = O.layer_forward(wl, li, blocks=pick)
    for b, n in pick:
        np.testing.assert_allclose(part[b, 5 * n:5 * n + 5], full[b, 5 * n:5 * n + 5],
                                   rtol=1e-12, atol=1e-12)
    others = [(b, n) for b in range(wl.B) for n in range(wl.N) if (b, n) not in pick]
    assert all(np.all(np.isnan(part[b, 5 * n:5 * n + 5])) for b, n in others)
