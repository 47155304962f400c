"""Pins of the fp64 oracle against what the design page and mathematics fix.

None of these re-types the oracle's own formula: each checks a number printed
on the page, a closed form, an invariance the page states, a library routine
in a special case, or agreement of two independently written forms.
"""
import copy

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wk
from conftest import golden

TINY = dict(wk.TINY_DIMS)


def tiny(S=48, N=4, W=16, seed=7, recipe="uniform", B=1, dims=None, **kw):
    d = dict(TINY if dims is None else dims)
    d["W"] = W
    args = dict(n_forced_low=1) if recipe == "uniform" else {}
    args.update(kw)
    return wk.make_workload("t", B=B, S=S, N=N, dims=d, dtype="f32", recipe=recipe,
                            seed=seed, recipe_args=args)


# ---------------------------------------------------------------------------
# parameter summary: KV cache record and the parameter table
# ---------------------------------------------------------------------------

def test_kv_cache_record_numbers_from_page():
    g = {k: float(v) for k, v in golden("kv_cache_numbers.txt")}
    D, d_r = wk.GLM_DIMS["D"], wk.GLM_DIMS["d_r"]
    assert (D, d_r) == (g["per_layer_ckv_dims"], g["per_layer_kr_dims"])
    assert D + d_r == g["per_layer_numbers"]
    assert g["draft_layers"] * (D + d_r) == g["draft_numbers"]
    assert round(g["draft_numbers"] * 2 / 1024, 1) == g["draft_kib_bf16"]
    assert g["target_layers"] * (D + d_r) == g["target_numbers"]
    assert round(g["target_numbers"] * 2 / 1024, 1) == g["target_kib_bf16"]


def test_expanded_keys_depend_only_on_the_576_cached_numbers():
    """Perturbing one token's 512 + 64 cached numbers changes exactly that
    token's expanded key/value and nothing else (the cache record is the
    whole per-token state of the layer)."""
    rng = np.random.default_rng(0)
    H, D, d_c, d_r, d_v = 2, 512, 192, 64, 256
    L = 9
    ckv, kr = rng.standard_normal((L, D)), rng.standard_normal((L, d_r))
    w_uk, w_uv = rng.standard_normal((H, d_c, D)), rng.standard_normal((H, d_v, D))
    K0, V0 = O.expand_head(ckv, kr, w_uk, w_uv, 1)
    assert K0.shape == (L, d_c + d_r) and V0.shape == (L, d_v)
    assert ckv.shape[1] + kr.shape[1] == 576
    ckv2, kr2 = ckv.copy(), kr.copy()
    ckv2[4] += 1.0
    kr2[4] -= 0.5
    K1, V1 = O.expand_head(ckv2, kr2, w_uk, w_uv, 1)
    changed = np.nonzero(np.any(K1 != K0, axis=1) | np.any(V1 != V0, axis=1))[0]
    assert changed.tolist() == [4]


def test_parameter_table_fixes_the_up_projection_shapes():
    """The page's 165M per MLA layer is reproduced only when kv_b_proj holds
    n_h * (d_c + d_v) * kv_rank weights, i.e. W_UK [H, d_c, D] and
    W_UV [H, d_v, D] as the oracle and the generator lay them out."""
    g = {k: float(v) for k, v in golden("param_table.txt")}
    wl = wk.make_workload("shape", B=1, S=8, N=1, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=1)
    H, d_c, D = wl.layers[0].w_uk.shape
    H2, d_v, D2 = wl.layers[0].w_uv.shape
    assert (H, D) == (H2, D2) == (g["n_h"], g["kv_rank"])
    d, qr, d_r = g["d"], g["q_rank"], g["d_r"]
    kv_b = wl.layers[0].w_uk.size + wl.layers[0].w_uv.size
    q_a, q_b = d * qr, qr * H * (d_c + d_r)
    kv_a = d * (D + d_r)
    o_proj = H * d_v * d
    mla = q_a + q_b + kv_a + kv_b + o_proj + qr + D          # + the two inner RMSNorms
    assert round(mla / 1e6) == g["mla_per_layer_M"]
    assert kv_b == 512 * 64 * 448
    swiglu = 3 * d * g["ffn"]
    main_proj = g["aux_width"] * d + d
    markov = 2 * g["vocab"] * g["markov_rank"]
    assert round(swiglu / 1e6) == g["swiglu_per_layer_M"]
    assert round(main_proj / 1e6) == g["main_proj_and_norm_M"]
    assert round(markov / 1e6) == g["markov_M"]
    total = main_proj + 3 * mla + 3 * swiglu + markov
    assert round(total / 1e9, 2) == g["total_B"]
    # a plausible mis-reading (W_UV sized d_c, or a shared K/V head) misses the table
    assert round((q_a + q_b + kv_a + H * 2 * d_c * D + o_proj) / 1e6) != g["mla_per_layer_M"]


# ---------------------------------------------------------------------------
# anchors
# ---------------------------------------------------------------------------

def test_bf16_decoding_matches_torch_on_every_bit_pattern():
    """Every one of the 65,536 bf16 bit patterns decodes to the value torch's
    bfloat16 type gives it (a library routine): normals, subnormals, both
    zeros (sign kept), both infinities; NaN patterns decode to NaN."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                       # exponent all ones, fraction != 0
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoding_closed_forms():
    """bf16 = sign, 8-bit exponent (bias 127), 7-bit fraction: the value of a
    normal pattern is (-1)^s 2^(e-127) (1 + f/128), of a subnormal one
    (-1)^s 2^-126 f/128."""
    import math
    rng = np.random.default_rng(9)
    pats = np.concatenate([rng.integers(0, 1 << 16, 500),
                           [0x3F80, 0xC000, 0x0001, 0x007F, 0x0080, 0x7F7F, 0x8000, 0x3F81]])
    for p in pats.astype(np.int64).tolist():
        s, e, f = (p >> 15) & 1, (p >> 7) & 0xFF, p & 0x7F
        if e == 0xFF:
            continue
        v = math.ldexp(1.0 + f / 128.0, e - 127) if e else math.ldexp(f / 128.0, -126)
        v = -v if s else v
        got = float(O.bf16_to_f64(np.array([p], dtype=np.uint16))[0])
        assert got == v and math.copysign(1.0, got) == (-1.0 if s else 1.0), hex(p)
    named = O.bf16_to_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x7FC0],
                                   dtype=np.uint16))
    assert named[0] == 1.0 and named[1] == -2.0 and named[2] == 2.0 ** -133
    assert named[3] == np.inf and named[4] == -np.inf and np.isnan(named[5])


def test_splitmix64_published_vector():
    want = [int(r[0]) for r in golden("splitmix64_seed1234567.txt")]
    g = O.SplitMix64(1234567)
    assert [g.next() for _ in range(5)] == want


def test_candidates_exclude_last_position_and_need_two_ones():
    S = 12
    lm = np.ones(S, dtype=np.uint8)
    C = O.candidates(lm)
    # loss_mask[S-1] is reset to 0 on read, so A = S-2 can never be an anchor
    assert C.tolist() == list(range(S - 2))
    lm = np.array([1, 1, 0, 1, 1, 1, 0, 0, 1, 1, 1, 1], dtype=np.uint8)
    assert O.candidates(lm).tolist() == [0, 3, 4, 8, 9]
    assert O.candidates(np.zeros(S, np.uint8)).tolist() == []


def test_sampler_padding_when_few_candidates():
    lm = np.array([1, 1, 0, 1, 1, 0, 0, 0], dtype=np.uint8)
    a, k = O.select_anchors(lm, 4, seed=3)
    assert a.tolist() == [0, 3, 0, 0] and k.tolist() == [1, 1, 0, 0]


def test_sampler_properties_and_uniformity():
    rng = np.random.default_rng(5)
    lm = (rng.random(200) < 0.9).astype(np.uint8)
    C = set(O.candidates(lm).tolist())
    N = 10
    counts = {c: 0 for c in C}
    trials = 3000
    for s in range(trials):
        a, k = O.select_anchors(lm, N, seed=s * 7919 + 1)
        al = a.tolist()
        assert all(k == 1) and al == sorted(al) and len(set(al)) == N and set(al) <= C
        for x in al:
            counts[x] += 1
    # every candidate is drawn with probability N / |C|
    p = N / len(C)
    freq = np.array(list(counts.values())) / trials
    sd = np.sqrt(p * (1 - p) / trials)
    assert np.all(np.abs(freq - p) < 5 * sd)
    assert abs(freq.mean() - p) < 1e-12


# ---------------------------------------------------------------------------
# mask
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("W", [16, 128])
def test_mask_invariants(W):
    S = 3 * W + 7
    anchors = np.array([0, 1, W - 2, W - 1, W, S - 2, S // 2, 5], dtype=np.int32)
    keep = np.array([1, 1, 1, 1, 1, 1, 1, 0], dtype=np.uint8)
    anchors[7] = -12345                       # a padding block's anchor is garbage
    N = len(anchors)
    M = O.build_mask(S, N, W, anchors, keep)
    assert M.shape == (5 * N, S + 5 * N) and M.dtype == bool
    for n in range(N):
        rows = M[5 * n:5 * n + 5]
        if not keep[n]:
            assert not rows.any()             # padding rows see nothing
            continue
        A = int(anchors[n])
        for j in range(1, 5):
            assert np.array_equal(rows[j], rows[0])   # window does not shift with j
        ctx = np.nonzero(rows[0, :S])[0]
        assert len(ctx) == min(A, W - 1) <= W - 1
        assert not rows[:, A].any()           # A itself is excluded
        if len(ctx):
            assert ctx[-1] == A - 1 and ctx[0] == max(0, A - W + 1)
            assert np.all(np.diff(ctx) == 1)
        draft = np.nonzero(rows[0, S:])[0]
        assert draft.tolist() == [5 * n + j for j in range(5)]   # own block only
    assert M[0:5].sum(axis=1).tolist() == [5] * 5              # A = 0: block keys only


def test_mask_brute_force_against_window_list():
    """Tiny shapes: every (q, kv) pair against an explicit window list."""
    S, W = 20, 6
    anchors = np.array([3, 0, 17, 9], dtype=np.int32)
    keep = np.array([1, 1, 1, 0], dtype=np.uint8)
    N = len(anchors)
    M = O.build_mask(S, N, W, anchors, keep)
    for q in range(5 * N):
        n = q // 5
        if keep[n]:
            A = anchors[n]
            visible = {A - t for t in range(1, W)} | {S + 5 * n + j for j in range(5)}
        else:
            visible = set()
        for kv in range(S + 5 * N):
            assert M[q, kv] == (kv in visible), (q, kv)


def test_index_records_match_mask():
    S, W = 300, 128
    anchors = np.array([0, 7, 126, 127, 128, 250, -1], dtype=np.int32)
    keep = np.array([1, 1, 1, 1, 1, 1, 0], dtype=np.uint8)
    recs = O.block_index_records(S, len(anchors), W, anchors, keep)
    assert recs.tolist() == [[0, 0, 0, 1], [0, 7, 7, 1], [0, 126, 126, 1], [0, 127, 127, 1],
                             [1, 127, 128, 1], [123, 127, 250, 1], [0, 0, 0, 0]]


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_softmax_scale_reading():
    """§4 fixes the scale at (d_c + d_r)^(-1/2): 1/16 for the GLM head dims,
    not the generic sqrt(d) of the appendix equation (d = 6144)."""
    assert O.softmax_scale(192, 64) == 1.0 / 16
    assert O.softmax_scale(16, 8) == pytest.approx(24 ** -0.5, rel=1e-15)


def test_rope_identity_norm_and_complex_form():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 8))
    assert np.array_equal(O.rope_interleaved(x, np.zeros(7), 10000.0), x)
    pos = rng.integers(0, 200000, size=7)
    y = O.rope_interleaved(x, pos, 10000.0)
    assert np.allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(x[:, 0::2], x[:, 1::2]),
                       rtol=1e-13, atol=0)
    # closed form: pair i is the complex number x_{2i} + i x_{2i+1} times
    # exp(i p theta_i), theta_i = base^(-2i/d_r)  (interleaved adjacent pairs)
    theta = 10000.0 ** (-np.arange(4) * 2 / 8)
    assert np.allclose(O.rope_theta(8, 10000.0), theta, rtol=1e-15)
    assert O.rope_theta(8, 10000.0)[2] == pytest.approx(1e-2)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * theta[None, :])
    assert np.allclose(y[:, 0::2], z.real, atol=1e-12) and np.allclose(y[:, 1::2], z.imag, atol=1e-12)


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((5, 64)), rng.standard_normal((9, 64))
    pq, pk = rng.integers(0, 1000, 5), rng.integers(0, 1000, 9)
    s0 = O.rope_interleaved(q, pq, 1e4) @ O.rope_interleaved(k, pk, 1e4).T
    s1 = O.rope_interleaved(q, pq + 123457, 1e4) @ O.rope_interleaved(k, pk + 123457, 1e4).T
    assert np.allclose(s0, s1, rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# forward: independent forms, closed forms, invariances, library special case
# ---------------------------------------------------------------------------

def _rel(a, b):
    m = np.isfinite(b)
    return np.linalg.norm(a[m] - b[m]) / np.linalg.norm(b[m])


@pytest.mark.parametrize("recipe,S,N,W,B", [("uniform", 48, 4, 16, 1),
                                             ("headline", 60, 8, 16, 1),
                                             ("clustered", 90, 6, 16, 2)])
def test_dense_gathered_absorbed_agree(recipe, S, N, W, B):
    wl = tiny(S=S, N=N, W=W, recipe=recipe, B=B, seed=11)
    dense = O.forward(wl, form="dense")
    gath = O.forward(wl, form="gathered")
    absd = O.forward_absorbed(wl)
    kept = np.repeat(wl.keep.astype(bool), 5, axis=1)
    assert np.all(np.isfinite(dense[kept])) and np.all(np.isnan(dense[~kept]))
    assert np.array_equal(np.isnan(dense), np.isnan(gath))
    assert np.array_equal(np.isnan(dense), np.isnan(absd))
    assert _rel(gath, dense) < 1e-12 and _rel(absd, dense) < 1e-12
    # sampled-block mode equals the full computation on those rows
    pick = [(b, n) for b in range(B) for n in range(N) if (b + n) % 2 == 0]
    part = O.forward(wl, form="gathered", blocks=pick)
    for b, n in pick:
        r = slice(5 * n, 5 * n + 5)
        np.testing.assert_allclose(part[b, r], dense[b, r], rtol=1e-12, atol=1e-12)


def test_equal_latents_give_w_uv_times_c():
    wl = tiny(seed=3)
    L = wl.layers[0]
    c = np.random.default_rng(4).standard_normal(wl.D).astype(np.float32)
    L.ckv_ctx[:] = c
    L.ckv_blk[:] = c
    out = O.forward(wl)
    for h in range(wl.H):
        want = L.w_uv[h].astype(np.float64) @ c.astype(np.float64)
        np.testing.assert_allclose(out[0, :, h, :], np.broadcast_to(want, out[0, :, h, :].shape),
                                   rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    wl = tiny(seed=5)
    L = wl.layers[0]
    L.q_nope[:] = 0
    L.q_rope[:] = 0
    out = O.forward(wl)
    S, W = wl.S, wl.W
    for n, A in enumerate(wl.anchors[0]):
        ctx = list(range(max(0, A - W + 1), A))
        lat = np.concatenate([L.ckv_ctx[0][ctx], L.ckv_blk[0][5 * n:5 * n + 5]]).astype(np.float64)
        mean_c = lat.mean(axis=0)
        for h in range(wl.H):
            want = L.w_uv[h].astype(np.float64) @ mean_c
            for j in range(5):
                np.testing.assert_allclose(out[0, 5 * n + j, h], want, rtol=1e-12, atol=1e-12)


def test_library_sdpa_special_case():
    """k^R = q^R = 0, D = d_c, W_UK = W_UV = I: the layer is plain masked
    scaled-dot-product attention with Q = q^C, K = V = c^KV."""
    dims = dict(H=2, D=16, d_c=16, d_r=8, d_v=16, W=16)
    wl = tiny(seed=9, dims=dims, recipe="headline", S=70, N=8)
    L = wl.layers[0]
    L.q_rope[:] = 0
    L.kr_ctx[:] = 0
    L.kr_blk[:] = 0
    L.w_uk[:] = np.eye(16, dtype=np.float32)
    L.w_uv[:] = np.eye(16, dtype=np.float32)
    out = O.forward(wl)
    M = O.build_mask(wl.S, wl.N, wl.W, wl.anchors[0], wl.keep[0])
    kv = torch.from_numpy(np.concatenate([L.ckv_ctx[0], L.ckv_blk[0]]).astype(np.float64))
    live = M.any(axis=1)
    for h in range(wl.H):
        q = torch.from_numpy(L.q_nope[0][:, h, :].astype(np.float64))[live]
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None], kv[None], kv[None], attn_mask=torch.from_numpy(M[live])[None],
            scale=1.0 / np.sqrt(16 + 8))[0].numpy()
        np.testing.assert_allclose(out[0][live, h, :], ref, rtol=1e-11, atol=1e-12)
    assert np.all(np.isnan(out[0][~live]))


def test_window_edges_and_cross_block_invariance():
    """Changing latents just outside a block's window (position A and A-W)
    or another block's draft keys leaves that block's rows unchanged; changing
    A-1 or A-W+1 changes them.  A = 0 rows ignore the whole context."""
    wl = tiny(S=64, N=4, W=16, seed=21)
    wl.anchors[0] = np.array([0, 20, 40, 45], dtype=np.int32)
    for a in wl.anchors[0]:
        wl.loss_mask[0, a] = wl.loss_mask[0, a + 1] = 1
    base = O.forward(wl)

    def perturbed(ctx_pos=None, blk_rows=None):
        w2 = copy.deepcopy(wl)
        if ctx_pos is not None:
            w2.layers[0].ckv_ctx[0, ctx_pos] += 3.0
            w2.layers[0].kr_ctx[0, ctx_pos] -= 2.0
        if blk_rows is not None:
            w2.layers[0].ckv_blk[0, blk_rows] += 3.0
        return O.forward(w2)

    r1 = slice(5, 10)                        # block 1, A = 20, window [5, 20)
    for p, changes in [(20, False), (4, False), (19, True), (5, True)]:
        out = perturbed(ctx_pos=p)
        assert (not np.allclose(out[0, r1], base[0, r1], rtol=0, atol=0)) == changes, p
    out = perturbed(blk_rows=slice(15, 20))  # block 3's own keys
    assert np.array_equal(out[0, 0:15], base[0, 0:15])
    out = perturbed(ctx_pos=slice(0, 64))    # the whole context
    assert np.array_equal(out[0, 0:5], base[0, 0:5])   # A = 0 block untouched


def test_block_order_does_not_matter():
    wl = tiny(S=64, N=4, W=16, seed=31)
    base = O.forward(wl)
    perm = np.array([2, 0, 3, 1])
    w2 = copy.deepcopy(wl)
    rows = np.concatenate([np.arange(5 * p, 5 * p + 5) for p in perm])
    w2.anchors[0] = wl.anchors[0][perm]
    w2.keep[0] = wl.keep[0][perm]
    for name in ("q_nope", "q_rope", "ckv_blk", "kr_blk"):
        getattr(w2.layers[0], name)[0] = getattr(wl.layers[0], name)[0][rows]
    out = O.forward(w2)
    np.testing.assert_allclose(out[0], base[0][rows], rtol=1e-12, atol=1e-12)
