"""Pins of the oracle's backward (gradients of the masked MLA attention).

The backward is written from the chain rule; none of these re-types it.  They
check it against central finite differences of the (separately pinned)
forward, closed forms the mathematics fixes, torch's autograd of its masked
SDPA in a special case, and the mask's visibility rules of the design page
(§3 "attention mask": no cross-block visibility, window [A-W+1, A), padding
blocks see nothing).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wk

SMALL = dict(H=2, D=8, d_c=4, d_r=4, d_v=4, W=6)
NAMES = ("q_nope", "q_rope", "ckv_ctx", "kr_ctx", "ckv_blk", "kr_blk", "w_uk", "w_uv")


def small(S=40, N=6, recipe="headline", seed=5, B=1, dims=None):
    d = dict(SMALL if dims is None else dims)
    # headline recipe: a quarter padding, half of the kept anchors < W - 1
    # (clamped windows, including A = 0)
    args = {"uniform": dict(n_forced_low=1), "headline": dict(low_frac=0.5)}.get(recipe, {})
    wl = wk.make_workload("s", B=B, S=S, N=N, dims=d, dtype="f32", recipe=recipe, seed=seed,
                          recipe_args=args)
    # fp64 storage so that finite differences resolve the gradient
    L = wl.layers[0]
    for nm in NAMES:
        setattr(L, nm, getattr(L, nm).astype(np.float64))
    return wl


def test_small_workload_has_padding_and_clamped_windows():
    wl = small()
    assert (wl.keep == 0).any() and (wl.keep == 1).any()
    kept_a = wl.anchors[wl.keep == 1]
    assert (kept_a < wl.W - 1).any() and (kept_a == 0).any() and (kept_a >= wl.W - 1).any()


@pytest.mark.parametrize("recipe,B", [("headline", 1), ("clustered", 2)])
def test_backward_matches_central_finite_differences(recipe, B):
    wl = small(recipe=recipe, B=B, S=44 if B == 1 else 80, N=6)
    dout = wk.make_dout(wl, seed=3).astype(np.float64)
    g = O.backward(wl, dout)
    rng = np.random.default_rng(0)
    L = wl.layers[0]
    eps = 1e-5
    worst = 0.0
    for nm in NAMES:
        x = getattr(L, nm)
        flat = x.reshape(-1)
        picks = rng.choice(flat.size, size=min(10, flat.size), replace=False)
        for i in picks:
            old = flat[i]
            flat[i] = old + eps
            lp = O.loss(wl, dout)
            flat[i] = old - eps
            lm = O.loss(wl, dout)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            an = g["d" + nm].reshape(-1)[i]
            err = abs(fd - an)
            worst = max(worst, err)
            assert err < 1e-7 + 1e-6 * abs(fd), (nm, int(i), fd, an)
    assert worst < 1e-6


def test_backward_dense_equals_gathered_and_is_linear_in_blocks():
    wl = small(S=44, N=6, seed=8)
    dout = wk.make_dout(wl, seed=4).astype(np.float64)
    full = O.backward(wl, dout)
    gath = O.backward(wl, dout, form="gathered")
    blocks_a = [(0, n) for n in range(0, 6, 2)]
    blocks_b = [(0, n) for n in range(1, 6, 2)]
    ga = O.backward(wl, dout, form="gathered", blocks=blocks_a)
    gb = O.backward(wl, dout, form="gathered", blocks=blocks_b)
    for k in full:
        np.testing.assert_allclose(gath[k], full[k], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ga[k] + gb[k], full[k], rtol=1e-12, atol=1e-13)


def test_equal_latents_closed_form():
    """All c^KV rows equal to c and k^R = 0: every score of a row is the same,
    so P is uniform over the v visible keys and no gradient flows through the
    scores (dq, dW_UK, dk^R vanish); out = W_UV c, so dW_UV[h] = sum_r G ⊗ c
    and d c^KV_k = sum over rows r that see k of (1/v_r) sum_h W_UV[h]^T G."""
    wl = small(S=44, N=6, seed=9)
    L = wl.layers[0]
    c = np.random.default_rng(2).standard_normal(wl.D)
    L.ckv_ctx[:] = c
    L.ckv_blk[:] = c
    L.kr_ctx[:] = 0
    L.kr_blk[:] = 0
    dout = wk.make_dout(wl, seed=5).astype(np.float64)
    g = O.backward(wl, dout)
    for k in ("dq_nope", "dq_rope", "dw_uk", "dkr_ctx", "dkr_blk"):
        assert np.max(np.abs(g[k])) < 1e-12, k
    kept_rows = np.repeat(wl.keep[0].astype(bool), 5)
    G = dout[0]
    for h in range(wl.H):
        want = np.einsum("rv,d->vd", G[kept_rows, h, :], c)
        np.testing.assert_allclose(g["dw_uv"][h], want, rtol=1e-12, atol=1e-12)
    want_ctx = np.zeros((wl.S, wl.D))
    want_blk = np.zeros((5 * wl.N, wl.D))
    for n in range(wl.N):
        if not wl.keep[0, n]:
            continue
        A = int(wl.anchors[0, n])
        ctx = list(range(max(0, A - wl.W + 1), A))
        v = len(ctx) + 5
        for j in range(5):
            r = 5 * n + j
            back = sum(L.w_uv[h].T @ G[r, h] for h in range(wl.H)) / v
            want_ctx[ctx] += back
            want_blk[5 * n:5 * n + 5] += back
    np.testing.assert_allclose(g["dckv_ctx"][0], want_ctx, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(g["dckv_blk"][0], want_blk, rtol=1e-11, atol=1e-12)


def test_library_sdpa_autograd_special_case():
    """k^R = q^R = 0 and D = d_c: the layer is masked SDPA with Q = q^C,
    K = c^KV W_UK^T, V = c^KV W_UV^T.  torch's autograd through its own
    scaled_dot_product_attention (fp64, CPU) gives dq^C, dc^KV, dW_UK, dW_UV."""
    dims = dict(H=2, D=8, d_c=8, d_r=4, d_v=6, W=6)
    wl = small(S=44, N=6, seed=12, dims=dims)
    L = wl.layers[0]
    L.q_rope[:] = 0
    L.kr_ctx[:] = 0
    L.kr_blk[:] = 0
    dout = wk.make_dout(wl, seed=6).astype(np.float64)
    g = O.backward(wl, dout)
    M = O.build_mask(wl.S, wl.N, wl.W, wl.anchors[0], wl.keep[0])
    live = M.any(axis=1)
    C = torch.tensor(np.concatenate([L.ckv_ctx[0], L.ckv_blk[0]]), requires_grad=True)
    wuk = torch.tensor(L.w_uk, requires_grad=True)
    wuv = torch.tensor(L.w_uv, requires_grad=True)
    q = torch.tensor(L.q_nope[0], requires_grad=True)
    total = 0
    for h in range(wl.H):
        K = C @ wuk[h].T
        V = C @ wuv[h].T
        o = torch.nn.functional.scaled_dot_product_attention(
            q[live, h, :][None], K[None], V[None], attn_mask=torch.from_numpy(M[live])[None],
            scale=1.0 / np.sqrt(dims["d_c"] + dims["d_r"]))[0]
        total = total + (o * torch.from_numpy(dout[0][live, h, :])).sum()
    total.backward()
    np.testing.assert_allclose(g["dq_nope"][0], q.grad.numpy(), rtol=1e-10, atol=1e-12)
    dC = C.grad.numpy()
    np.testing.assert_allclose(g["dckv_ctx"][0], dC[:wl.S], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dckv_blk"][0], dC[wl.S:], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dw_uk"], wuk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dw_uv"], wuv.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.max(np.abs(g["dq_rope"])) < 1e-13 and np.max(np.abs(g["dkr_ctx"])) < 1e-13


def test_gradient_respects_the_mask():
    """Gradient from one block's rows reaches only what those rows see:
    its context window [max(0, A-W+1), A), its own 5 draft keys and its own
    queries; a padding block's rows carry none even when dout is nonzero."""
    wl = small(S=44, N=6, seed=14)
    n_kept = [n for n in range(wl.N) if wl.keep[0, n]]
    n_pad = [n for n in range(wl.N) if not wl.keep[0, n]]
    assert n_pad
    for n in n_kept + n_pad[:1]:
        dout = wk.make_dout(wl, seed=7).astype(np.float64)
        only = np.zeros_like(dout)
        only[0, 5 * n:5 * n + 5] = dout[0, 5 * n:5 * n + 5]
        g = O.backward(wl, only)
        q_rows = np.zeros(5 * wl.N, bool)
        ctx_ok = np.zeros(wl.S, bool)
        if wl.keep[0, n]:
            A = int(wl.anchors[0, n])
            q_rows[5 * n:5 * n + 5] = True
            ctx_ok[max(0, A - wl.W + 1):A] = True
        for k, rows in (("dq_nope", q_rows), ("dq_rope", q_rows), ("dckv_blk", q_rows),
                        ("dkr_blk", q_rows), ("dckv_ctx", ctx_ok), ("dkr_ctx", ctx_ok)):
            outside = g[k][0][~rows]
            assert np.all(outside == 0), (k, n)
            if rows.any() and k != "dq_rope":
                assert np.all(np.any(g[k][0][rows] != 0, axis=tuple(range(1, g[k][0].ndim)))), (k, n)
        if not wl.keep[0, n]:
            assert np.all(g["dw_uk"] == 0) and np.all(g["dw_uv"] == 0)


def test_rope_transpose_is_the_inverse_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 8))
    pos = rng.integers(0, 10 ** 5, size=7)
    y = O.rope_interleaved(x, pos, 10000.0)
    np.testing.assert_allclose(O.rope_interleaved_transpose(y, pos, 10000.0), x,
                               rtol=1e-12, atol=1e-12)
    # adjoint: <R x, z> = <x, R^T z>
    z = rng.standard_normal((7, 8))
    assert abs(np.sum(y * z) - np.sum(x * O.rope_interleaved_transpose(z, pos, 10000.0))) < 1e-11
