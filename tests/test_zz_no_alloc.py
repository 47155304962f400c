"""The allocation-free forward (dspark_attn_fwd_noalloc) against the forward
with a caller workspace (dspark_attn_fwd), through the C ABI: two calls in a
row on the library's fixed scratch array, the second smaller, so that it
runs over what the first left there; then the generic path with a bad
anchor reported through the caller's status words."""
import numpy as np
import pytest

import workloads as wk
from gpu_util import BF16_MAX_ABS, BF16_REL_L2, F32_MAX_ABS, F32_REL_L2, ForwardRun, compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sd():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import speculative_decoding_draft_amd as sd
    return sd


def run_noalloc(sd, ref: ForwardRun, guard=1024):
    """The same call as `ref` through dspark_attn_fwd_noalloc, into a fresh
    NaN-filled output with NaN guard regions; returns (output, status,
    first_bad, guards intact)."""
    import torch
    t = ref.t
    n = ref.out.numel()
    full = torch.full((n + 2 * guard,), float("nan"), dtype=ref.out.dtype, device="cuda")
    out = full[guard:guard + n].view(ref.out.shape)
    status = torch.full((sd.STATUS_BYTES // 4,), -7, dtype=torch.int32, device="cuda")
    sd.attn_fwd_noalloc(ref.desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"],
                        t["ckv_blk"], t["kr_blk"], t["w_uk"], t["w_uv"], ref.anchors, ref.keep,
                        out, status=status)
    torch.cuda.synchronize()
    st, fb = sd.read_device_status(status)
    g = full.float().cpu().numpy()
    intact = bool(np.all(np.isnan(g[:guard])) and np.all(np.isnan(g[-guard:])))
    return out.float().cpu().numpy().astype(np.float64), st, fb, intact


def test_noalloc_matches_workspace_forward_on_two_calls_in_a_row(sd):
    # call 1: 1024 slots (768 kept) in rounds of ~100 blocks; call 2: 100
    # slots, one round, over the scratch contents call 1 left
    for name, wl in (("S=32768 N=1024 (768 kept)", wk.config(4)),
                     ("S=2048 N=100", wk.scaled(4, S=2048, N=100))):
        log(f"no-alloc forward: {name}")
        ref = ForwardRun(wl, 0, wl.anchors, wl.keep).run()
        want = ref.result()
        got, st, fb, intact = run_noalloc(sd, ref)
        assert st == sd.DSPARK_OK and fb == -1, sd.last_error()
        assert intact, "the output's guard regions were written"
        compare(got, want, wl.keep, BF16_MAX_ABS, BF16_REL_L2, what=f"no-alloc vs workspace {name}")


def test_noalloc_generic_path_reports_a_bad_anchor_through_status(sd):
    wl = wk.config(1)                       # fp32: the generic kernel
    a, k = wl.anchors.copy(), wl.keep.copy()
    k[:] = 1
    a[0, 2] = wl.S - 1                      # outside [0, S-2]
    log("no-alloc forward: generic path, bad anchor in block 2")
    ref = ForwardRun(wl, 0, a, k).run()
    want = ref.result()
    got, st, fb, intact = run_noalloc(sd, ref, guard=64)
    assert st == sd.DSPARK_EANCHOR and fb == 2
    assert intact
    assert np.all(np.isnan(got[0, 10:15])) and np.all(np.isnan(want[0, 10:15]))
    ok = k.copy()
    ok[0, 2] = 0
    got[0, 10:15] = 0.0
    want[0, 10:15] = 0.0
    compare(got, want, ok, F32_MAX_ABS, F32_REL_L2, what="no-alloc vs workspace, generic")


def test_noalloc_at_131072_positions_in_forty_rounds(sd):
    """S = 131072, N = 4096 sampler anchors (about 40 rounds of ~100 blocks
    through the fixed array): the same bits as the workspace forward, which
    runs every block in one round."""
    import torch
    wl = wk.config(5)
    ga = np.zeros((wl.B, wl.N), np.int32)
    gk = np.zeros((wl.B, wl.N), np.uint8)
    for b in range(wl.B):
        ga[b], gk[b] = sd.select_anchors_host(wl.loss_mask[b], wl.N, wl.sampler_seed + b)
    log(f"no-alloc forward: S=131072 N=4096 ({int(gk.sum())} kept)")
    ref = ForwardRun(wl, 0, ga, gk).run()
    torch.cuda.synchronize()
    got, st, fb, intact = run_noalloc(sd, ref, guard=4096)
    assert st == sd.DSPARK_OK and fb == -1, sd.last_error()
    assert intact
    want = ref.result()
    same = np.array_equal(np.nan_to_num(got, nan=7.0), np.nan_to_num(want, nan=7.0))
    log(f"  bit-identical to the workspace forward: {same}")
    compare(got, want, gk, BF16_MAX_ABS, BF16_REL_L2, what="no-alloc vs workspace S=131072")
