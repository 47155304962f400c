"""Parity of inference-time drafting with the oracle: the draft cache
(dspark_cache_append), the decode attention over it (dspark_decode_attn)
and the verification of drafted tokens (dspark_spec_verify).

Tolerances.  Cache contents: bit for bit.  Decode attention: the training
attention's (bf16 MFMA path: max-abs 2e-2, rel-L2 5e-3; fp32 generic path
1e-4 / 2e-5) -- it is that attention on a re-based window.  Verification:
acceptance probabilities and overlaps are fp32 expressions of fp32
log-sum-exps (errors ~1e-6), held to 2e-5.  The accept/reject decisions
and the drawn token are integers decided in floating point: they must equal
the oracle's unless the uniform lies within 1e-4 of the threshold (then
either decision is valid); a differing draw must still satisfy the inverse
CDF's bracket within 1e-5 of the total weight.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from gpu_util import BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, log
from workloads.device import to_torch

pytestmark = pytest.mark.gpu

TINY = dict(H=2, D=16, d_c=8, d_r=4, d_v=8, W=6)


def run_decode(dims, dtype, C, anchors, active, split=20, seed=13):
    import torch
    import speculative_decoding_draft_amd as sd
    B = len(anchors)
    W = dims["W"]
    n_ctx = C + 40
    di = wk.make_decode_inputs(B, dims, dtype, n_ctx, seed=seed)
    dev = lambda a: to_torch(a, dtype, "cuda")
    attn = sd.make_desc(B=B, S=0, N=1, window=W, n_heads=dims["H"], d_latent=dims["D"],
                        d_nope=dims["d_c"], d_rope=dims["d_r"], d_v=dims["d_v"], dtype=dtype)
    d = sd.make_decode_desc(attn, C)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache_ckv = torch.full((B, C, dims["D"]), 7.0, dtype=tdt, device="cuda")
    cache_kr = torch.full((B, C, dims["d_r"]), 7.0, dtype=tdt, device="cuda")
    # host ring built by the oracle's slot rule from the same rows, in the
    # storage type (bf16 bit patterns or fp32); unwritten slots hold 7.0
    f = (lambda a: O.bf16_to_f64(a)) if dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    seven = wk.f32_to_bf16_bits(np.float32([7.0]))[0] if dtype == "bf16" else np.float32(7.0)
    ring_ckv = np.full((B, C, dims["D"]), seven, dtype=di.ctx_ckv.dtype)
    ring_kr = np.full((B, C, dims["d_r"]), seven, dtype=di.ctx_kr.dtype)
    p0 = np.array([max(0, a - n_ctx) for a in anchors], np.int64)
    n_b = np.array([max(0, a - p) for a, p in zip(anchors, p0)], np.int64)
    first = np.minimum(n_b, split + C)                # the first call may hold more than C rows
    rows_ckv, rows_kr = di.ctx_ckv, di.ctx_kr
    for b in range(B):
        for t in range(int(n_b[b])):
            s = int(O.ring_slot(p0[b] + t, C))
            ring_ckv[b, s] = rows_ckv[b, t]
            ring_kr[b, s] = rows_kr[b, t]
    for lo, cnt in ((np.zeros(B, np.int64), first), (first, n_b - first)):
        mx = int(cnt.max()) if B else 0
        if mx == 0:
            continue
        sl_ckv = np.zeros((B, mx, dims["D"]), di.ctx_ckv.dtype)
        sl_kr = np.zeros((B, mx, dims["d_r"]), di.ctx_kr.dtype)
        for b in range(B):
            sl_ckv[b, :cnt[b]] = di.ctx_ckv[b, lo[b]:lo[b] + cnt[b]]
            sl_kr[b, :cnt[b]] = di.ctx_kr[b, lo[b]:lo[b] + cnt[b]]
        pos = torch.tensor((p0 + lo).astype(np.int32), device="cuda")
        n = torch.tensor(cnt.astype(np.int32), device="cuda")
        sd.cache_append(d, pos, n, dev(sl_ckv), dev(sl_kr), cache_ckv, cache_kr)
    a_dev = torch.tensor(np.asarray(anchors, np.int32), device="cuda")
    act = torch.tensor(np.asarray(active, np.uint8), device="cuda")
    out = torch.full((B, 5, dims["H"], dims["d_v"]), float("nan"), dtype=tdt, device="cuda")
    ws = torch.empty(sd.decode_workspace_size(d), dtype=torch.uint8, device="cuda")
    sd.decode_attn(d, dev(di.q_nope), dev(di.q_rope), cache_ckv, cache_kr, dev(di.ckv_blk),
                   dev(di.kr_blk), dev(di.w_uk), dev(di.w_uv), a_dev, act, out, ws)
    st, fb = sd.read_device_status(ws)
    torch.cuda.synchronize()
    got_ring = (cache_ckv.float().cpu().numpy().astype(np.float64),
                cache_kr.float().cpu().numpy().astype(np.float64))
    ref = O.decode_attention(ring_ckv, ring_kr, anchors, active, di.q_nope, di.q_rope, di.ckv_blk,
                             di.kr_blk, di.w_uk, di.w_uv, W, 10000.0, dtype)
    return out.float().cpu().numpy().astype(np.float64), ref, got_ring, (f(ring_ckv), f(ring_kr)), st


def check_decode(name, gpu, ref, active, tol):
    act = np.asarray(active, bool)
    assert np.all(gpu[~act] == 0), name
    g, r = gpu[act], ref[act]
    mx = float(np.abs(g - r).max())
    rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
    log(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e}")
    assert mx <= tol[0] and rel <= tol[1], (name, mx, rel)


def test_decode_bench_shape():
    """The decode bench's shape: 64 sequences at GLM dims, W = C = 128,
    anchors drawn as the bench draws them."""
    anchors = np.random.default_rng(31).integers(128, 10**6, size=64).tolist()
    active = [1] * 64
    gpu, ref, ring, ring_ref, st = run_decode(dict(wk.GLM_DIMS), "bf16", 128, anchors, active)
    assert st == 0
    check_decode("decode bench shape", gpu, ref, active, (BF16_MAX_ABS, BF16_REL_L2))


@pytest.mark.parametrize("C", [127, 128, 200])
def test_decode_glm_bf16(C):
    """GLM dims, bf16; C = 127 = W - 1 is the smallest ring the window fits:
    the window of the longest sequences then fills every slot."""
    dims = dict(wk.GLM_DIMS)
    anchors = [0, 3, 126, 127, 1_000_003, 5000, 131]
    active = [1, 1, 1, 1, 1, 0, 1]
    gpu, ref, ring, ring_ref, st = run_decode(dims, "bf16", C, anchors, active)
    assert st == 0
    for g, r in zip(ring, ring_ref):
        np.testing.assert_array_equal(g, r)       # every slot, written or not
    check_decode(f"decode bf16 C={C}", gpu, ref, active, (BF16_MAX_ABS, BF16_REL_L2))


@pytest.mark.parametrize("C", [5, 6, 9])
def test_decode_tiny_fp32(C):
    anchors = [0, 1, 4, 5, 6, 37, 123457]
    active = [1, 1, 1, 0, 1, 1, 1]
    gpu, ref, ring, ring_ref, st = run_decode(TINY, "f32", C, anchors, active, split=3)
    assert st == 0
    for g, r in zip(ring, ring_ref):
        np.testing.assert_array_equal(g, r)
    check_decode(f"decode fp32 C={C}", gpu, ref, active, (F32_MAX_ABS, F32_REL_L2))


def test_decode_negative_anchor_is_reported():
    import speculative_decoding_draft_amd as sd
    gpu, ref, _, _, st = run_decode(TINY, "f32", 6, [4, -3, 9], [1, 1, 1])
    assert st == sd.DSPARK_EANCHOR
    assert np.all(np.isnan(gpu[1]))
    check_decode("decode with a bad anchor", gpu[[0, 2]], ref[[0, 2]], [1, 1], (F32_MAX_ABS, F32_REL_L2))


def run_verify(B, K, V, mode, T=1.0, seed=17, bad_token=False):
    import torch
    import speculative_decoding_draft_amd as sd
    dl, tl, u, ud = wk.make_verify_inputs(B, K, V, seed=seed)
    q = O.softmax_t(dl.reshape(B * K, V), T).reshape(B, K, V)
    tok = np.array([[O.sample_inverse_cdf(q[b, k], float(ud[b, k])) for k in range(K)]
                    for b in range(B)], np.int32)
    if bad_token:
        tok[1, 2] = V + 5
    d = sd.make_verify_desc(B, K, V, mode, T)
    ws = torch.empty(sd.verify_workspace_size(d), dtype=torch.uint8, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    ap = torch.full((B, K), -1.0, device="cuda")
    ov = torch.full((B, K), -1.0, device="cuda")
    na = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sd.spec_verify(d, t(dl), t(tl), t(tok), t(u), ap, ov, na, nt, ws)
    torch.cuda.synchronize()
    return (dl, tl, tok, u), (ap.cpu().numpy(), ov.cpu().numpy(), na.cpu().numpy(), nt.cpu().numpy())


def check_verify(name, inputs, got, mode, T=1.0, skip=()):
    dl, tl, tok, u = inputs
    ap, ov, na, nt = got
    B, K, V = dl.shape
    n_same_draw = 0
    for b in range(B):
        if b in skip:
            continue
        r = O.spec_verify(dl[b], tl[b], tok[b], u[b].astype(np.float64), mode, T)
        assert np.abs(ap[b] - r["accept_prob"]).max() <= 2e-5, (name, b)
        assert np.abs(ov[b] - r["overlap"]).max() <= 2e-5, (name, b)
        if na[b] != r["n_accept"]:
            k = min(int(na[b]), r["n_accept"])
            assert mode == "rejection" and abs(u[b, k] - r["accept_prob"][k]) < 1e-4, (name, b)
            continue
        j = r["n_accept"]
        if nt[b] == r["next_token"]:
            n_same_draw += 1
            continue
        assert mode == "rejection", (name, b, nt[b], r["next_token"])
        p = O.softmax_t(tl[b], T)
        qq = O.softmax_t(dl[b], T)
        w = np.maximum(0.0, p[j] - qq[j]) if j < K else p[K]
        if w.sum() == 0:
            w = p[j]
        c = np.cumsum(w) / w.sum()
        x = int(nt[b])
        lo = c[x - 1] if x > 0 else 0.0
        assert lo <= u[b, K] + 1e-5 and c[x] >= u[b, K] - 1e-5, (name, b, x, r["next_token"])
    log(f"  {name}: {B - len(skip)} sequences, {n_same_draw} draws identical to the oracle's; "
        f"n_accept {na.tolist()}")


@pytest.mark.parametrize("V,mode,T", [(1000, "rejection", 1.0), (20000, "rejection", 0.7),
                                      (8192 * 2 + 3, "target_only", 1.0), (777, "target_only", 1.3),
                                      (1, "rejection", 1.0), (1, "target_only", 1.0)])
def test_verify_matches_oracle(V, mode, T):
    inputs, got = run_verify(16, 5, V, mode, T)
    check_verify(f"verify V={V} {mode} T={T}", inputs, got, mode, T)


def test_verify_full_vocabulary_and_a_bad_token():
    inputs, got = run_verify(8, 5, 154880, "rejection", bad_token=True, seed=19)
    assert got[2][1] == -1 and got[3][1] == -1
    check_verify("verify V=154880", inputs, got, "rejection", skip=(1,))


def test_verify_identical_distributions_accept_everything():
    import torch
    import speculative_decoding_draft_amd as sd
    B, K, V = 4, 5, 3000
    dl, tl, u, ud = wk.make_verify_inputs(B, K, V, seed=23)
    tl[:, :K] = dl
    tok = np.zeros((B, K), np.int32) + 17
    d = sd.make_verify_desc(B, K, V)
    ws = torch.empty(sd.verify_workspace_size(d), dtype=torch.uint8, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    ap, ov = torch.empty((B, K), device="cuda"), torch.empty((B, K), device="cuda")
    na, nt = torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda")
    sd.spec_verify(d, t(dl), t(tl), t(tok), t(u), ap, ov, na, nt, ws)
    torch.cuda.synchronize()
    assert np.all(na.cpu().numpy() == K)
    assert np.abs(ap.cpu().numpy() - 1).max() < 1e-6 and np.abs(ov.cpu().numpy() - 1).max() < 1e-5


def test_verify_target_only_accepts_argmax_prefixes():
    """Drafted tokens equal to the target's top choice for the first m_b
    positions (m_b = b mod 6), then another token: n_accept = m_b and the
    next token is the top choice of row m_b."""
    import torch
    import speculative_decoding_draft_amd as sd
    B, K, V = 12, 5, 9000
    dl, tl, u, _ = wk.make_verify_inputs(B, K, V, seed=29)
    top = tl.argmax(axis=2)
    tok = np.zeros((B, K), np.int32)
    for b in range(B):
        m = b % (K + 1)
        tok[b] = top[b, :K]
        if m < K:
            tok[b, m] = (top[b, m] + 1) % V
    d = sd.make_verify_desc(B, K, V, "target_only")
    ws = torch.empty(sd.verify_workspace_size(d), dtype=torch.uint8, device="cuda")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    ap, ov = torch.empty((B, K), device="cuda"), torch.empty((B, K), device="cuda")
    na, nt = torch.empty(B, dtype=torch.int32, device="cuda"), torch.empty(B, dtype=torch.int32, device="cuda")
    sd.spec_verify(d, t(dl), t(tl), t(tok), t(u), ap, ov, na, nt, ws)
    torch.cuda.synchronize()
    check_verify("target-only prefixes", (dl, tl, tok, u),
                 (ap.cpu().numpy(), ov.cpu().numpy(), na.cpu().numpy(), nt.cpu().numpy()),
                 "target_only")
    assert na.cpu().numpy().tolist() == [b % (K + 1) for b in range(B)]
