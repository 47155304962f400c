"""Pins of the oracle's inference-time drafting: the decode attention over
the windowed draft cache (parameter summary "KV cache"; §3 mask; §4 MLA and
RoPE) and the rejection-sampling verification of the MTP / DSA explainer
page (acceptance sum_v min(p_v, q_v)).

The decode attention is checked against the pinned training forward on the
same latents; the verification against the page's worked example, the exact
acceptance probability and output distribution of rejection sampling
(enumerated over a fine grid of uniforms), and numpy's searchsorted."""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from conftest import golden

DIMS = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)


def decode_from_workload(wl, slots, shift=0):
    """The workload's N = 1 blocks seen through a ring cache of `slots`
    entries holding each sample's window (and positions shifted by `shift`)."""
    lay = wl.layers[0]
    f = lambda a: O.bf16_to_f64(a) if wl.dtype == "bf16" else np.asarray(a, np.float64)
    B = wl.B
    cc = np.zeros((B, slots, wl.D))
    ck = np.zeros((B, slots, wl.d_r))
    for b in range(B):
        A = int(wl.anchors[b, 0])
        for p in range(max(0, A - wl.W + 1), A):
            cc[b, (p + shift) % slots] = f(lay.ckv_ctx)[b, p]
            ck[b, (p + shift) % slots] = f(lay.kr_ctx)[b, p]
    return O.decode_attention(cc, ck, wl.anchors[:, 0] + shift, wl.keep[:, 0], f(lay.q_nope),
                              f(lay.q_rope), f(lay.ckv_blk), f(lay.kr_blk), f(lay.w_uk),
                              f(lay.w_uv), wl.W, wl.rope_base, "f64")


@pytest.mark.parametrize("slots", [64, 5, 7])
def test_decode_attention_equals_the_training_forward(slots):
    """One block per sample: the ring cache (linear when it is as long as
    the sequence, wrapping when it holds only W - 1 or W + 1 entries) gives
    the training forward's output."""
    # one workload with every window clamped at position 0, one with most
    # windows whole (anchor >= W - 1)
    for B, seed, args in ((3, 5, dict(n_forced_low=1)), (6, 7, {})):
        wl = wk.make_workload("dec", B=B, S=64, N=1, dims=DIMS, dtype="f32", recipe="uniform",
                              seed=seed, recipe_args=args)
        if not args:
            assert (wl.anchors[:, 0] >= wl.W).sum() >= 3
        ref = O.forward(wl, form="gathered")
        got = decode_from_workload(wl, slots)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_decode_attention_is_invariant_to_a_common_position_shift():
    """RoPE scores depend on relative positions only: moving every position
    by the same amount (the ring slots move with them) leaves the output of a
    block whose window is not clamped at position 0."""
    wl = wk.make_workload("dec", B=6, S=64, N=1, dims=DIMS, dtype="f32", recipe="uniform",
                          seed=7)
    full = wl.anchors[:, 0] >= wl.W - 1
    assert full.sum() >= 3
    a = decode_from_workload(wl, 6)
    b = decode_from_workload(wl, 6, shift=123457)
    np.testing.assert_allclose(a[full], b[full], rtol=1e-9, atol=1e-10)
    # an inactive sequence gives NaN rows
    f = lambda x: np.asarray(x, np.float64)
    lay = wl.layers[0]
    out = O.decode_attention(np.zeros((2, 6, wl.D)), np.zeros((2, 6, wl.d_r)), [3, 4], [1, 0],
                             f(lay.q_nope)[:2], f(lay.q_rope)[:2], f(lay.ckv_blk)[:2], f(lay.kr_blk)[:2],
                             f(lay.w_uk), f(lay.w_uv), wl.W, wl.rope_base, "f64")
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[0]))


def test_acceptance_worked_example():
    g = {r[0]: [float(x) for x in r[1:]] for r in golden("acceptance_worked_example.txt")}
    assert abs(O.acceptance(g["p"], g["q"]) - g["acceptance"][0]) < 1e-15
    # through the verification: overlap of the one step
    r = O.spec_verify(np.log(g["q"])[None], np.log([g["p"], g["p"]]), [1], [0.0, 0.5])
    assert abs(r["overlap"][0] - 0.95) < 1e-12
    assert abs(r["accept_prob"][0] - 0.30 / 0.35) < 1e-12
    assert r["n_accept"] == 1


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(1)
    for _ in range(200):
        w = rng.random(17) * (rng.random(17) < 0.7)
        w[rng.integers(17)] += 0.1
        u = rng.random()
        c = np.cumsum(w)
        assert O.sample_inverse_cdf(w, u) == int(np.searchsorted(c, u * c[-1], side="right"))


def test_inverse_cdf_at_breakpoints_never_returns_a_zero_weight():
    """The generalised inverse of a CDF F is min{i : F(i) > u}: with u = 0 it
    skips a prefix of zero weights, and at an exact breakpoint u = F(i) it
    returns the next index.  Weights are small integers with a power-of-two
    total, so every breakpoint u = c_i / total is exact; the expected index
    is the count of cumulative sums <= u * total."""
    assert O.sample_inverse_cdf([0.0, 0.0, 0.3, 0.7], 0.0) == 2
    assert O.sample_inverse_cdf([1.0, 1.0, 2.0], 0.25) == 1
    assert O.sample_inverse_cdf([1.0, 1.0, 2.0], 0.5) == 2
    rng = np.random.default_rng(3)
    for _ in range(50):
        w = rng.integers(0, 4, 12).astype(np.float64)
        w[0] = 0.0
        w[rng.integers(1, 12)] += 1.0
        w[-1] += 64.0 - w.sum()                   # total 64
        if w[-1] < 0:
            continue
        c = np.cumsum(w)
        for u in np.concatenate([[0.0], c[:-1] / c[-1]]):
            i = O.sample_inverse_cdf(w, float(u))
            assert w[i] > 0
            assert i == int(np.sum(c <= u * c[-1]))


def grid(n):
    return (np.arange(n) + 0.5) / n


def test_rejection_sampling_accepts_with_probability_sum_min_p_q():
    """For x drawn from q and u uniform, P(accept) = sum_x q(x) min(1, p/q) =
    sum_v min(p_v, q_v): enumerated over x and a grid of u."""
    rng = np.random.default_rng(2)
    for _ in range(5):
        lq, lp = rng.standard_normal(6) * 1.5, rng.standard_normal(6) * 1.5
        q, p = O.softmax_t(lq[None])[0], O.softmax_t(lp[None])[0]
        acc = 0.0
        for x in range(6):
            n_ok = sum(O.spec_verify(lq[None], np.stack([lp, lp]), [x], [u, 0.5])["n_accept"]
                       for u in grid(2000))
            acc += q[x] * n_ok / 2000
        assert abs(acc - O.acceptance(p, q)) < 1e-3


def test_rejection_sampling_output_is_distributed_as_the_target():
    """The token kept at position 0 -- the draft's x when accepted, else the
    residual sample -- is distributed exactly as p_0 (enumerated over x ~ q
    and grids of both uniforms)."""
    rng = np.random.default_rng(3)
    lq, lp, lb = rng.standard_normal(5) * 1.2, rng.standard_normal(5) * 1.2, rng.standard_normal(5)
    q, p = O.softmax_t(lq[None])[0], O.softmax_t(lp[None])[0]
    hist = np.zeros(5)
    n = 300
    for x in range(5):
        for u0 in grid(n):
            r = O.spec_verify(lq[None], np.stack([lp, lb]), [x], [u0, 0.0])
            if r["n_accept"] == 1:
                hist[x] += q[x] / n
            else:
                for u1 in grid(n):
                    r = O.spec_verify(lq[None], np.stack([lp, lb]), [x], [u0, u1])
                    hist[r["next_token"]] += q[x] / n / n
    np.testing.assert_allclose(hist, p, atol=6e-3)
    # when all are accepted the bonus token comes from p_K
    r = O.spec_verify(lq[None], np.stack([lp, lb]), [int(np.argmax(lp / q))], [0.0, 0.37])
    assert r["n_accept"] == 1
    assert r["next_token"] == O.sample_inverse_cdf(O.softmax_t(lb[None])[0], 0.37)


def test_target_only_accepts_the_target_argmax_only():
    rng = np.random.default_rng(4)
    lq = rng.standard_normal((3, 8))
    lp = rng.standard_normal((4, 8))
    top = lp.argmax(axis=1)
    r = O.spec_verify(lq, lp, top[:3], np.zeros(4), mode="target_only")
    assert r["n_accept"] == 3 and r["next_token"] == top[3]
    x = top[:3].copy()
    x[1] = (x[1] + 1) % 8
    r = O.spec_verify(lq, lp, x, np.zeros(4), mode="target_only")
    assert r["n_accept"] == 1 and r["next_token"] == top[1]


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((4, 30))
    r = O.spec_verify(l[:3], l, [3, 1, 4], np.full(4, 0.999999))
    assert r["n_accept"] == 3
    np.testing.assert_allclose(r["accept_prob"], 1.0)
    np.testing.assert_allclose(r["overlap"], 1.0)


def test_temperature_divides_the_logits():
    """softmax(x / T): closed forms.  Logits (0, ln 4) at T = 2 are (0, ln 2),
    probabilities (1/3, 2/3); (0, ln 9, 2 ln 9) at T = 2 give (1, 3, 9) / 13;
    at T = 1/2 the first pair gives (1, 16) / 17."""
    p = O.softmax_t(np.array([[0.0, np.log(4.0)]]), 2.0)[0]
    assert np.allclose(p, [1 / 3, 2 / 3], rtol=0, atol=1e-15)
    p = O.softmax_t(np.array([[0.0, np.log(9.0), 2 * np.log(9.0)]]), 2.0)[0]
    assert np.allclose(p, np.array([1.0, 3.0, 9.0]) / 13.0, rtol=0, atol=1e-15)
    p = O.softmax_t(np.array([[0.0, np.log(4.0)]]), 0.5)[0]
    assert np.allclose(p, [1 / 17, 16 / 17], rtol=0, atol=1e-15)


def test_temperature_flattens_and_verification_depends_on_logits_over_t():
    """A higher temperature never lowers the entropy, and the whole
    verification at temperature T equals the one at T = 1 on the logits
    divided by T (decisions, draws, acceptance and overlap)."""
    rng = np.random.default_rng(5)
    x = rng.normal(0.0, 3.0, size=(4, 50))
    ent = lambda p: -(p * np.log(p)).sum(axis=-1)
    e = [ent(O.softmax_t(x, t)) for t in (0.5, 1.0, 2.0, 4.0)]
    for lo, hi in zip(e, e[1:]):
        assert np.all(hi >= lo - 1e-12)
    K, V = 5, 40
    for T in (0.7, 1.3, 2.5):
        for s in range(20):
            r = np.random.default_rng(100 + s)
            dl = r.normal(0.0, 2.0, size=(K, V))
            tl = r.normal(0.0, 2.0, size=(K + 1, V))
            x_t = r.integers(0, V, size=K)
            u = r.random(K + 1)
            a = O.spec_verify(dl, tl, x_t, u, "rejection", temperature=T)
            b = O.spec_verify(dl / T, tl / T, x_t, u, "rejection", temperature=1.0)
            for k in ("n_accept", "next_token"):
                assert a[k] == b[k], (T, s, k)
            for k in ("accept_prob", "overlap"):
                assert np.allclose(a[k], b[k], rtol=1e-12, atol=1e-15), (T, s, k)
