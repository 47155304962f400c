"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Index records must match bit for bit; outputs within the
stated tolerances; padding rows must be exactly zero."""
import numpy as np
import pytest

import oracle as O
import workloads as wk
from gpu_util import (BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, ForwardRun, HipEventPool,
                      anchors_for, compare, desc_for, log, sample_blocks, context_of_two,
                      repeated_anchors)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_draft_amd as sd
    return sd


def check_full(wl, form="dense", layer=0, force_generic=False, tol=None, guard=0,
               chunk_blocks=0, one_launch=False):
    ga, gk, oa, ok = anchors_for(wl)
    assert np.array_equal(ga, oa) and np.array_equal(gk, ok), "anchor selection differs"
    run = ForwardRun(wl, layer, ga, gk, guard=guard, force_generic=force_generic,
                     chunk_blocks=chunk_blocks, one_launch=one_launch).run()
    gpu = run.result()
    st, _ = run.sd.read_device_status(run.ws)
    assert st == run.sd.DSPARK_OK, run.sd.last_error()
    ref = O.forward(wl, layer, oa, ok, form=form)
    if tol is None:
        tol = (F32_MAX_ABS, F32_REL_L2) if wl.dtype == "f32" else (BF16_MAX_ABS, BF16_REL_L2)
    stats = compare(gpu, ref, ok, *tol, what=wl.name)
    assert run.guards_intact(), "write outside `out`"
    return run, gpu, stats


# ---------------------------------------------------------------------------
# index builder: bit-exact against the oracle's mask
# ---------------------------------------------------------------------------

def gpu_index(sd, wl, anchors, keep):
    import torch
    desc = desc_for(wl)
    ws = torch.empty(sd.workspace_size(desc), dtype=torch.uint8, device="cuda")
    a = torch.from_numpy(np.ascontiguousarray(anchors, np.int32)).cuda()
    k = torch.from_numpy(np.ascontiguousarray(keep, np.uint8)).cuda()
    out = torch.full((wl.B, wl.N, 4), -7, dtype=torch.int32, device="cuda")
    sd.build_index(desc, a, k, out, ws)
    st, first_bad = sd.read_device_status(ws)
    return out.cpu().numpy(), st, first_bad


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_index_records_bit_exact(sd, k):
    wl = wk.config(k, tensors=False)
    ga, gk, oa, ok = anchors_for(wl)
    assert np.array_equal(ga, oa) and np.array_equal(gk, ok)
    rec, st, first_bad = gpu_index(sd, wl, ga, gk)
    assert st == sd.DSPARK_OK and first_bad == -1
    # slots are the ranks of the kept blocks in (b, n) order
    rank = np.cumsum(ok.ravel().astype(np.int64)) - 1
    assert np.array_equal(rec[..., 3].ravel(), np.where(ok.ravel() == 1, rank, -1))
    for b in range(wl.B):
        want = O.block_index_records(wl.S, wl.N, wl.W, oa[b], ok[b])
        for n in range(wl.N):
            if ok[b, n]:
                assert rec[b, n, :3].tolist() == want[n, :3].tolist(), (b, n)
            else:
                assert rec[b, n].tolist() == [0, 0, 0, -1], (b, n)
    log(f"  cfg{k}: {int(ok.sum())} kept blocks, records identical")


def test_index_sets_equal_mask_rows(sd):
    """Column sets implied by the GPU records equal the nonzeros of the
    oracle's materialised mask, row by row (headline recipe, small S)."""
    wl = wk.make_workload("idx", B=2, S=700, N=64, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="headline", seed=5, tensors=False)
    rec, st, _ = gpu_index(sd, wl, wl.anchors, wl.keep)
    assert st == sd.DSPARK_OK
    for b in range(wl.B):
        M = O.build_mask(wl.S, wl.N, wl.W, wl.anchors[b], wl.keep[b])
        sets = O.row_index_sets(M, wl.S)
        for n in range(wl.N):
            lo, ln, pos0, slot = rec[b, n]
            for j in range(5):
                ctx, drf = sets[5 * n + j]
                if slot < 0:
                    assert len(ctx) == 0 and len(drf) == 0
                    continue
                assert ctx.tolist() == list(range(lo, lo + ln))
                assert drf.tolist() == [wl.S + 5 * n + i for i in range(5)]
                assert pos0 == wl.anchors[b, n]


def test_bad_kept_anchor_is_reported(sd):
    wl = wk.make_workload("bad", B=1, S=300, N=8, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=3, tensors=False)
    a, k = wl.anchors.copy(), wl.keep.copy()
    a[0, 5] = wl.S - 1          # one past the last valid anchor
    a[0, 6] = -3
    rec, st, first_bad = gpu_index(sd, wl, a, k)
    assert st == sd.DSPARK_EANCHOR and first_bad == 5
    assert rec[0, 5].tolist() == [0, 0, 0, -2] and rec[0, 6].tolist() == [0, 0, 0, -2]
    assert rec[0, 7, 3] == 5    # later kept blocks keep consecutive slots


# ---------------------------------------------------------------------------
# forward parity
# ---------------------------------------------------------------------------

def test_cfg1_tiny_fp32(sd):
    log("cfg1 tiny fp32 (generic kernel)")
    check_full(wk.config(1), guard=64)


def test_cfg2_glm_layer(sd):
    log("cfg2 GLM layer B1 S2048 N64 (MFMA, head-split launch)")
    check_full(wk.config(2), guard=4096)


def test_cfg2_generic_kernel_bf16(sd):
    log("cfg2 through the generic kernel")
    check_full(wk.config(2), force_generic=True)


def test_cfg3_recipe_small(sd):
    log("cfg3 recipe B2 S1024 N64")
    check_full(wk.scaled(3, S=1024, N=64), form="gathered")


def test_cfg4_recipe_small(sd):
    log("cfg4 recipe B1 S4096 N128 (padding + clamped windows)")
    check_full(wk.scaled(4, S=4096, N=128), form="gathered", guard=4096)


def test_cfg4_recipe_shuffled_kept_anchors(sd):
    """The page draws N anchors at random and fixes no order; here the
    headline recipe's (anchor, keep) slots are permuted so that kept anchors
    are out of order and padding slots sit between them."""
    wl = wk.scaled(4, S=4096, N=128)
    perm = np.random.default_rng(44).permutation(wl.N)
    wl.anchors[0] = wl.anchors[0][perm]
    wl.keep[0] = wl.keep[0][perm]
    kept = wl.anchors[0][wl.keep[0] == 1]
    assert np.any(np.diff(kept) < 0)
    log("cfg4 recipe B1 S4096 N128, kept anchors shuffled")
    check_full(wl, form="gathered", guard=1024)


def test_cfg4_recipe_four_wave_launch(sd):
    log("cfg4 recipe B1 S4096 N600 (one workgroup per block)")
    check_full(wk.scaled(4, S=4096, N=600), form="gathered")


def test_four_wave_launch_with_shuffled_kept_anchors(sd):
    """Enough kept blocks for the four-wave launch (one workgroup per block,
    all 64 heads), with the kept anchors in random order: neighbouring slots'
    windows overlap partly, fully or not at all, in either direction."""
    wl = wk.scaled(4, S=4096, N=600)
    perm = np.random.default_rng(45).permutation(wl.N)
    wl.anchors[0] = wl.anchors[0][perm]
    wl.keep[0] = wl.keep[0][perm]
    kept = wl.anchors[0][wl.keep[0] == 1]
    assert len(kept) >= 400 and np.any(np.diff(kept) < 0)
    log("four-wave launch: B1 S4096 N600, kept anchors shuffled")
    check_full(wl, form="gathered", guard=1024)


def test_four_wave_launch_dense_windows_three_samples(sd):
    """The four-wave launch on three samples with anchors a few positions
    apart (windows almost equal) and clamped windows at each sample's start."""
    wl = wk.make_workload("ring-B3", B=3, S=900, N=320, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="headline", seed=83, recipe_args=dict(pad_frac=0.2, low_frac=0.2))
    assert int(wl.keep.sum()) >= 600
    log("four-wave launch: B3 S900 N320, dense anchors")
    check_full(wl, form="gathered", guard=1024)


@pytest.mark.parametrize("chunk", [1, 7, 64, 159, 160, 100000])
def test_chunk_sizes(sd, chunk):
    """Kept blocks processed in rounds of `chunk` (ragged last round, rounds
    past the kept count, the one-wave / four-wave attention launch switch)."""
    wl = wk.scaled(4, S=4096, N=224)
    log(f"cfg4 recipe B1 S4096 N224, chunk {chunk}")
    check_full(wl, form="gathered", guard=2048, chunk_blocks=chunk)


@pytest.mark.parametrize("chunk", [7, 48, 100])
def test_rounds_on_two_streams(sd, chunk):
    """Odd rounds on a second stream (joined back before the result is
    read): bit for bit the output of the same rounds on one stream, and
    within tolerance of the oracle."""
    import torch
    wl = wk.scaled(4, S=4096, N=224)
    log(f"cfg4 recipe B1 S4096 N224, chunk {chunk}, two streams")
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, guard=2048, chunk_blocks=chunk)
    single = run.run().result()
    run.out.fill_(float("nan"))
    aux = torch.cuda.Stream()
    ev = HipEventPool(2, timing=False)
    t = run.t
    sd.attn_fwd(run.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"],
                t["kr_blk"], t["w_uk"], t["w_uv"], run.anchors, run.keep, run.out, run.ws,
                chunk_blocks=chunk, aux_stream=aux, aux_events=ev.handles)
    got = run.result()
    ev.close()
    assert run.guards_intact()
    ref = O.forward(wl, 0, form="gathered")
    compare(got, ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what=f"two streams, chunk {chunk}")
    assert np.array_equal(np.nan_to_num(got, nan=7.0), np.nan_to_num(single, nan=7.0))


def test_stage_events_are_recorded_in_order(sd):
    import ctypes
    import torch
    wl = wk.scaled(4, S=2048, N=100)
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, chunk_blocks=16)
    n_chunks, chunk, n_ev = sd.attn_plan(run.desc, chunk_blocks=16)
    assert (n_chunks, chunk, n_ev) == (7, 16, 2 + 4 * 7)
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(n_ev):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    t = run.t
    with pytest.raises(sd.DSparkError):   # too few events is refused up front
        sd.attn_fwd(run.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"],
                    t["kr_blk"], t["w_uk"], t["w_uv"], run.anchors, run.keep, run.out, run.ws,
                    stage_events=evs[:-1], chunk_blocks=16)
    sd.attn_fwd(run.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"],
                t["kr_blk"], t["w_uk"], t["w_uv"], run.anchors, run.keep, run.out, run.ws,
                stage_events=evs, chunk_blocks=16)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    for a, b in zip(evs[:-1], evs[1:]):
        assert hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        assert ms.value >= 0.0
    for e in evs:
        hip.hipEventDestroy(e)
    compare(run.result(), O.forward(wl, 0, form="gathered"), wl.keep, BF16_MAX_ABS, BF16_REL_L2,
            what="with stage events")


def test_bound_call_matches_plain_call(sd):
    """BoundFwd (arguments marshalled once) runs the same forward."""
    import torch
    wl = wk.scaled(4, S=2048, N=96)
    r = ForwardRun(wl, 0, wl.anchors, wl.keep, chunk_blocks=32)
    ref = r.run().result()
    r.out.fill_(float("nan"))
    t = r.t
    n_chunks, chunk, n_ev = sd.attn_plan(r.desc, chunk_blocks=32)
    call = sd.BoundFwd(r.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"],
                       t["kr_blk"], t["w_uk"], t["w_uv"], r.anchors, r.keep, r.out, r.ws,
                       chunk_blocks=32, n_stage_events=n_ev)
    call()
    got = r.result()
    assert np.array_equal(np.nan_to_num(got, nan=7.0), np.nan_to_num(ref, nan=7.0))
    torch.cuda.synchronize()


@pytest.mark.parametrize("W", [1, 2, 16, 127, 128])
def test_window_sizes_on_mfma_path(sd, W):
    dims = dict(wk.GLM_DIMS, W=W)
    wl = wk.make_workload(f"W{W}", B=1, S=400, N=40, dims=dims, dtype="bf16", recipe="headline",
                          seed=40 + W, recipe_args=dict(low_frac=0.1) if W > 3 else
                          dict(low_frac=0.0))
    log(f"window {W}")
    check_full(wl, form="gathered")


def test_all_padding_and_anchor_zero(sd):
    wl = wk.make_workload("edge", B=2, S=256, N=6, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=77)
    wl.keep[0, :] = 0                      # sample 0: all padding, garbage anchors
    wl.anchors[0, :] = np.array([-5, 10**6, 0, 255, -1, 3])
    wl.anchors[1, :] = np.array([0, 1, 2, 3, 100, 200])   # A = 0: block keys only
    for a in wl.anchors[1]:
        wl.loss_mask[1, a] = wl.loss_mask[1, a + 1] = 1
    check_full(wl, form="gathered")


def test_anchor_at_last_valid_position_and_single_block(sd):
    """A = S - 2 (block positions up to S + 2, the top of the RoPE table)
    and N = 1 on the MFMA path."""
    wl = wk.make_workload("edge-top", B=1, S=300, N=1, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=81)
    wl.anchors[0, 0] = 298
    wl.loss_mask[0, 298] = wl.loss_mask[0, 299] = 1
    check_full(wl, form="dense")


def test_context_of_two_positions(sd):
    check_full(context_of_two(91), form="dense", guard=256)


def test_repeated_kept_anchors(sd):
    wl = repeated_anchors(93)
    a = wl.anchors[0][wl.keep[0] == 1]
    assert (wl.keep.sum() >= 160 and len(np.unique(a)) < len(a)), "case needs repeats"
    check_full(wl, form="gathered")


def test_three_samples_mixed_blocks(sd):
    """B = 3 with padding, clamped and full windows mixed in every sample."""
    wl = wk.make_workload("mixed-B3", B=3, S=700, N=37, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="headline", seed=82, recipe_args=dict(pad_frac=0.3, low_frac=0.2))
    check_full(wl, form="gathered", guard=1024)


def test_everything_padding_on_mfma_path(sd):
    wl = wk.make_workload("all-pad", B=2, S=256, N=50, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=83)
    wl.keep[:] = 0
    wl.anchors[:] = -3
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, guard=512).run()
    gpu = run.result()
    assert np.all(gpu == 0) and run.guards_intact()
    st, fb = sd.read_device_status(run.ws)
    assert st == sd.DSPARK_OK and fb == -1


def test_bad_anchor_rows_are_nan_and_reported(sd):
    wl = wk.make_workload("badfwd", B=1, S=512, N=20, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=9)
    a, k = wl.anchors.copy(), wl.keep.copy()
    a[0, 7] = 511            # S - 1: invalid
    run = ForwardRun(wl, 0, a, k).run()
    st, fb = sd.read_device_status(run.ws)
    assert st == sd.DSPARK_EANCHOR and fb == 7
    gpu = run.result()
    assert np.all(np.isnan(gpu[0, 35:40]))
    ok = k.copy()
    ok[0, 7] = 0
    ref = O.forward(wl, 0, a, ok, form="gathered")
    gpu[0, 35:40] = 0.0      # excluded from the comparison as a non-kept block
    compare(gpu, ref, ok, BF16_MAX_ABS, BF16_REL_L2, what="other blocks")


def test_explicit_softmax_scale(sd):
    wl = wk.scaled(4, S=1024, N=32)
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, softmax_scale=0.03).run()
    ref = O.forward(wl, 0, form="gathered", scale=0.03)
    compare(run.result(), ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="scale 0.03")


def test_deterministic(sd):
    wl = wk.scaled(4, S=2048, N=96)
    r = ForwardRun(wl, 0, wl.anchors, wl.keep)
    a = r.run().result()
    b = r.run().result()
    assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0))


# ---------------------------------------------------------------------------
# full benchmark sizes: sampled blocks
# ---------------------------------------------------------------------------

def check_sampled(wl, layer, ga, gk, oa, ok, n_random, seed):
    run = ForwardRun(wl, layer, ga, gk).run()
    gpu = run.result()
    st, fb = run.sd.read_device_status(run.ws)
    assert st == 0 and fb == -1
    pick = []
    for b in range(wl.B):
        pick += [(b, n) for n in sample_blocks(ok[b], oa[b], wl.W, n_random, seed + b)]
    ref = O.forward(wl, layer, oa, ok, form="gathered", blocks=pick)
    compare(gpu, ref, ok, BF16_MAX_ABS, BF16_REL_L2, what=f"{wl.name} layer {layer} "
            f"({len(pick)} sampled blocks)")


def test_cfg3_full_size_sampled(sd):
    wl = wk.config(3)
    log("cfg3 full size")
    ga, gk, oa, ok = anchors_for(wl)
    check_sampled(wl, 0, ga, gk, oa, ok, n_random=24, seed=3)


def test_cfg4_full_size_sampled(sd):
    wl = wk.config(4)
    log("cfg4 full size")
    ga, gk, oa, ok = anchors_for(wl)
    check_sampled(wl, 0, ga, gk, oa, ok, n_random=40, seed=4)


def test_cfg5_full_size_sampled(sd):
    wl = wk.config(5)
    log("cfg5 full size, 3 layers with shared anchors")
    ga, gk, oa, ok = anchors_for(wl)
    assert np.array_equal(ga, oa) and np.array_equal(gk, ok)
    for layer in range(3):
        check_sampled(wl, layer, ga, gk, oa, ok, n_random=12, seed=50 + layer)


# ---------------------------------------------------------------------------
# robustness: canaries, a live checker, NaN confinement
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_output_guard_regions_are_untouched(sd, dtype):
    """NaN canaries on both sides of `out` survive the call (MFMA path for
    bf16, generic path for fp32)."""
    wl = wk.scaled(4, S=700, N=24) if dtype == "bf16" else wk.config(1)
    check_full(wl, form="gathered", guard=8192)


def test_checker_is_live(sd):
    """The comparison fails when one output element of a kept block moves by
    more than the tolerance: the parity checks can see a wrong result."""
    wl = wk.scaled(4, S=700, N=24)
    run = ForwardRun(wl, 0, wl.anchors, wl.keep).run()
    gpu = run.result()
    ref = O.forward(wl, 0, form="gathered")
    compare(gpu, ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="unmodified")
    b, n = [(b, n) for b in range(wl.B) for n in range(wl.N) if wl.keep[b, n]][3]
    bad = gpu.copy()
    bad[b, 5 * n + 2, 7, 11] += 0.1
    with pytest.raises(AssertionError):
        compare(bad, ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="one element moved")
    pad = [(b, n) for b in range(wl.B) for n in range(wl.N) if not wl.keep[b, n]][0]
    bad = gpu.copy()
    bad[pad[0], 5 * pad[1], 0, 0] = 1e-3          # padding rows must stay exactly 0
    with pytest.raises(AssertionError):
        compare(bad, ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="padding row written")


@pytest.mark.parametrize("force_generic", [False, True])
def test_nan_in_one_context_row_stays_in_its_windows(sd, force_generic):
    """A NaN written into one context row's c^KV reaches exactly the kept
    blocks whose window contains that row (all their rows); every other row
    is bit for bit what it was."""
    import torch
    wl = wk.scaled(4, S=700, N=24)
    base = ForwardRun(wl, 0, wl.anchors, wl.keep, force_generic=force_generic).run().result()
    kept = [(0, n) for n in range(wl.N) if wl.keep[0, n]]
    A = int(wl.anchors[0, kept[len(kept) // 2][1]])
    p = A - 3
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, force_generic=force_generic)
    run.t["ckv_ctx"][0, p, 17] = float("nan")
    got = run.run().result()
    hit = {n for (_, n) in kept if max(0, int(wl.anchors[0, n]) - wl.W + 1) <= p < int(wl.anchors[0, n])}
    assert hit, "the poisoned row lies in no window"
    for n in range(wl.N):
        rows = got[0, 5 * n:5 * n + 5]
        if n in hit:
            assert np.all(np.isnan(rows)), n
        else:
            assert np.array_equal(rows, base[0, 5 * n:5 * n + 5]), n
    log(f"  NaN at context row {p}: {len(hit)} blocks see it, the other {wl.N - len(hit)} unchanged")


def test_forward_and_backward_replay_from_a_hip_graph(sd):
    """The forward and the backward are kernel launches only (no allocation,
    no memset, no synchronisation), so a caller can capture them in a HIP
    graph.  Each of three replays, with the program's own eager work and a
    synchronisation between them, gives the eager call's bits."""
    import torch
    from workloads.device import upload_anchors, upload_layer
    wl = wk.scaled(4, S=700, N=24)
    t = upload_layer(wl)
    a, k = upload_anchors(wl.anchors, wl.keep)
    desc = desc_for(wl)
    ins = (t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"], t["kr_blk"],
           t["w_uk"], t["w_uv"], a, k)
    B, L5, H = wl.B, wl.q_len, wl.H
    out = torch.empty((B, L5, H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sd.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    dout = torch.from_numpy(wk.make_dout(wl, seed=11)).view(torch.bfloat16).cuda()
    shapes = {"dq_nope": (B, L5, H, wl.d_c), "dq_rope": (B, L5, H, wl.d_r),
              "dckv_ctx": (B, wl.S, wl.D), "dkr_ctx": (B, wl.S, wl.d_r),
              "dckv_blk": (B, L5, wl.D), "dkr_blk": (B, L5, wl.d_r),
              "dw_uk": (H, wl.d_c, wl.D), "dw_uv": (H, wl.d_v, wl.D)}
    grads = {n: torch.empty(v, dtype=torch.bfloat16, device="cuda") for n, v in shapes.items()}

    def step():
        sd.attn_fwd(desc, *ins, out, ws)
        sd.attn_bwd(desc, *ins, dout, grads, ws, reuse_forward=True)

    step()
    torch.cuda.synchronize()
    eager = {"out": out.clone(), **{n: g.clone() for n, g in grads.items()}}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):            # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        for g in grads.values():
            g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager["out"]), r
        for n, g in grads.items():
            assert torch.equal(g, eager[n]), (r, n)
    log("  forward + backward: 3 graph replays bit-identical to the eager call")


# ---------------------------------------------------------------------------
# the one-launch forward (dspark_attn_opts.one_launch): absorb, attention and
# W_UV on different compute units, q_abs / o_lat through per-XCD L2 rings
# ---------------------------------------------------------------------------

def _mixed():
    return wk.make_workload("mixed-B3", B=3, S=700, N=37, dims=wk.GLM_DIMS, dtype="bf16",
                            recipe="headline", seed=82, recipe_args=dict(pad_frac=0.3, low_frac=0.2))


@pytest.mark.parametrize("case", ["cfg2", "cfg4-small", "cfg3-small", "mixed-B3", "window-16",
                                  "single-block"])
def test_one_launch_forward(sd, case):
    """More kept blocks than the 32 ring slots (several generations per
    slot), padding, clamped windows, B > 1, short windows, a single block."""
    if case == "cfg2":
        wl = wk.config(2)
    elif case == "cfg4-small":
        wl = wk.scaled(4, S=4096, N=600)
    elif case == "cfg3-small":
        wl = wk.scaled(3, S=1024, N=64)
    elif case == "mixed-B3":
        wl = _mixed()
    elif case == "window-16":
        wl = wk.make_workload("W16", B=1, S=400, N=40, dims=dict(wk.GLM_DIMS, W=16), dtype="bf16",
                              recipe="headline", seed=56, recipe_args=dict(low_frac=0.1))
    else:
        wl = wk.make_workload("edge-top", B=1, S=300, N=1, dims=wk.GLM_DIMS, dtype="bf16",
                              recipe="uniform", seed=81)
        wl.anchors[0, 0] = 298
        wl.loss_mask[0, 298] = wl.loss_mask[0, 299] = 1
    log(f"one-launch forward: {case}")
    check_full(wl, form="gathered", guard=2048, one_launch=True)


def test_one_launch_headline_size_sampled_blocks(sd):
    """Headline size (768 kept blocks: 24 generations per ring slot)."""
    wl = wk.config(4)
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, one_launch=True).run()
    gpu = run.result()
    st, _ = sd.read_device_status(run.ws)
    assert st == sd.DSPARK_OK, sd.last_error()
    pick = sample_blocks(wl.keep[0], wl.anchors[0], wl.W, n_random=24, seed=7)
    ref = O.forward(wl, 0, form="gathered", blocks=[(0, n) for n in pick])
    compare(gpu, ref, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="one-launch headline sampled")


def test_one_launch_repeats_bit_identically_and_matches_three_kernels(sd):
    """Every output is computed in a fixed order whatever compute unit takes
    its block, so two calls give the same bits; the three-kernel forward
    agrees within the bf16 tolerance (its roundings differ)."""
    wl = wk.scaled(4, S=2048, N=200)
    run = ForwardRun(wl, 0, wl.anchors, wl.keep, one_launch=True)
    a = run.run().result()
    run.out.fill_(float("nan"))
    b = run.run().result()
    assert np.array_equal(np.nan_to_num(a, nan=7.0), np.nan_to_num(b, nan=7.0))
    three = ForwardRun(wl, 0, wl.anchors, wl.keep).run().result()
    compare(a, three, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what="one-launch vs three kernels")


def test_one_launch_bad_anchor_rows_are_nan(sd):
    wl = wk.make_workload("badfwd", B=1, S=512, N=20, dims=wk.GLM_DIMS, dtype="bf16",
                          recipe="uniform", seed=9)
    a, k = wl.anchors.copy(), wl.keep.copy()
    a[0, 7] = 511
    run = ForwardRun(wl, 0, a, k, one_launch=True).run()
    st, fb = sd.read_device_status(run.ws)
    assert st == sd.DSPARK_EANCHOR and fb == 7
    gpu = run.result()
    assert np.all(np.isnan(gpu[0, 35:40]))
    ok = k.copy()
    ok[0, 7] = 0
    ref = O.forward(wl, 0, a, ok, form="gathered")
    gpu[0, 35:40] = 0.0
    compare(gpu, ref, ok, BF16_MAX_ABS, BF16_REL_L2, what="one-launch other blocks")
