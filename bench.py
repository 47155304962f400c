"""Benchmark of the DSpark draft-attention forward (and backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]

A step is one dspark_attn_fwd call per layer (index build, absorb,
attention, W_UV with the rows of padding blocks) over the whole workload, with inputs resident in
HBM and the L2 not flushed between steps.  The headline workload is the
S=32768, N=1024 configuration (25% padding blocks, 5% clamped windows,
synthetic N(0,1) activations and N(0,1/512) weights).  Prints one JSON line.

Timing of the headline workload: exactly W warm-up steps; then 50 samples
of 10 back-to-back steps with one hipEvent on the launch stream between
samples (none inside a sample: an event between two calls delays the next
one by several microseconds), whose median time per step gives `value` and
`ms_per_step`; for several layers, a pass with events at layer boundaries
(per-layer medians); then a separate pass of calls with the library's stage
events between its kernels (per-kernel durations for the roofline); then
exactly K steps with no event at all between two synchronisations, whose
mean is reported as timing.timed_loop_ms_per_step.  The other four
configurations are measured the same way first and reported in the
`configs` object.

Useful FLOP count only what the absorbed method must compute for kept blocks
and visible keys: per kept block 5*H*(2*d_c*D + 2*(D+d_r)*v + 2*D*v + 2*D*d_v)
with v = min(A, W-1) + 5.  The roofline object takes the kernel with the
largest share of the step against the bf16 MFMA peak (its useful FLOP per
launch over its average launch duration), and compares the forward's
measured HBM traffic (rocprofv3 counters, when the kernels' sources are
those they were taken on) with the bytes the method needs (inputs read
once, output written once).

The same line carries a "backward" object: dspark_attn_bwd on the same
inputs with a seeded upstream gradient (--bwd-steps timed calls), its useful
TFLOP/s (gradient products only; see bwd_useful_flop) and per-launch times.
A "layer" object times dspark_mla_layer_fwd (the MLA block of one draft
layer: RMSNorms, projections, the attention, o_proj) on seeded hidden states
and weights of the page's shapes.  A "loss" object times dspark_loss_fwd (the
output head and loss: lm_head for the draft and the teacher, Markov bias,
confidence head, CE / L1 / BCE means) at V = 154880, d = 6144, r = 256 on the
same anchors.  A "decode" object times one inference-time drafting step for
64 sequences: appending 5 accepted positions to each draft cache ring,
the decode attention over the rings, and the rejection-sampling
verification of 5 drafted tokens at V = 154880.  The headline metric is the
forward's.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_PEAK_TFLOPS = 2516.6     # 256 CU * 2.4 GHz * 4096 FLOP/CU/clk, dense
MI355X_HBM_PEAK_GBS = 8000.0
STAGES = ("index", "absorb", "attention", "w_uv")
KERNEL_SOURCES = {"absorb": "absorb.hip", "attention": "attn.hip", "w_uv": "uv.hip",
                  "index": "prep.hip"}
# Measured HBM bytes per launch on the headline workload (one round of all
# blocks): rocprofv3 --pmc FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 (factors from a
# plain 256 MiB device copy), with the digest of the kernel's sources when the
# counters were taken.  A kernel whose sources changed since reports null.
# The headline's index is built inside the absorb launch (no preparation
# launch runs), so absorb's bytes include it.
PMC_TRAFFIC = {
    "absorb": (358_861_477, "01b07695fce01035"),
    "attention": (583_434_500, "4c469051f3ab5f15"),
    "w_uv": (436_550_001, "c350d3045986165b"),
}
PMC_SOURCE = "rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, profiles/attn_fwd_headline_S32768_N1024_counters.md"


# The same for the backward's launches (dspark_attn_bwd on the headline
# workload): the source files each kernel is built from.
BWD_KERNEL_SOURCES = {
    "attention_bwd": ("bwd_attn.hip", "bwd.hpp", "common.hpp", "kernels.hpp"),
    "dw": ("bwd_gemm.hip", "bwd.hpp", "common.hpp", "kernels.hpp"),
    "dkv": ("bwd_gemm.hip", "bwd.hpp", "common.hpp", "kernels.hpp"),
    "dq_nope": ("uv.hip", "common.hpp", "kernels.hpp"),
    "d_olat": ("absorb.hip", "common.hpp", "kernels.hpp"),
    "final": ("bwd_misc.hip", "bwd.hpp", "common.hpp", "kernels.hpp"),
}
BWD_PMC_TRAFFIC = {
    "attention_bwd": (1_293_601_290, "423619f69f79a403"),
    "dw": (757_902_599, "3ff6fdbc26332773"),
    "dkv": (1_001_676_042, "3ff6fdbc26332773"),
    "dq_nope": (358_924_480, "c350d3045986165b"),
    "d_olat": (394_464_495, "01b07695fce01035"),
    "final": (311_311_256, "4d1dd8f62b34ea4d"),
}


# Measured HBM bytes per call of the loss head's statistics pass (headline
# anchors, V = 154880, d = 6144, rank 256) and of the whole verification (its
# three launches; 64 sequences, K = 5, V = 154880): the same FETCH/WRITE
# scaling, with the files each is built from and their digest when taken.
SIDE_PMC_TRAFFIC = {
    "loss_stats": (3_882_859_940, ("loss.hip", "blas.hpp", "kernels.hpp"), "9133278bf6e34a79"),
    "verify": (436_689_308 + 398_406_720 + 4_409_600, ("decode.hip", "kernels.hpp"),
               "0e246a99590adc3e"),
}



def side_measured_traffic(key: str, applies: bool):
    if not applies:
        return None
    nbytes, files, digest = SIDE_PMC_TRAFFIC[key]
    return nbytes if files_digest(files) == digest else None


def files_digest(files) -> str:
    import hashlib
    csrc = os.path.join(ROOT, "speculative_decoding_draft_amd", "csrc")
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_digest(stage: str) -> str:
    return files_digest((KERNEL_SOURCES[stage], "common.hpp", "kernels.hpp"))


def bwd_measured_traffic(stage: str, workload: str):
    if stage not in BWD_PMC_TRAFFIC or not workload.startswith("headline"):
        return None
    nbytes, digest = BWD_PMC_TRAFFIC[stage]
    return nbytes if files_digest(BWD_KERNEL_SOURCES[stage]) == digest else None


def measured_traffic(stage: str, workload: str, chunk_blocks: int, n_blocks: int):
    if stage not in PMC_TRAFFIC or not workload.startswith("headline") or chunk_blocks < n_blocks:
        return None
    nbytes, digest = PMC_TRAFFIC[stage]
    return nbytes if kernel_digest(stage) == digest else None


def useful_flop(anchors, keep, W, H, D, d_c, d_r, d_v, block=5) -> int:
    total = 0
    for a, k in zip(np.asarray(anchors).ravel(), np.asarray(keep).ravel()):
        if k:
            v = min(int(a), W - 1) + block
            total += block * H * (2 * d_c * D + 2 * (D + d_r) * v + 2 * D * v + 2 * D * d_v)
    return total


def stage_bytes(wl, anchors, keep, chunk_blocks):
    """Algorithmic HBM bytes of each kernel launch (bf16 = 2 B), per chunk of
    `chunk_blocks` kept blocks taken in (b, n) order: every input the launch
    needs read once (its weights included), the context read as the union of
    the chunk's kept windows, each output written once (the last W_UV launch
    also writes the padding blocks' rows).  Returns
    {stage: [bytes of launch 0, launch 1, ...]}."""
    H, D, dc, dr, dv = wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v
    kept = [(b, int(anchors[b, n])) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    out = {"absorb": [], "attention": [], "w_uv": []}
    for c0 in range(0, max(len(kept), 1), chunk_blocks):
        part = kept[c0:c0 + chunk_blocks]
        rows = 5 * len(part)
        union = 0
        for b in range(wl.B):
            cover = np.zeros(wl.S, dtype=bool)
            for bb, a in part:
                if bb == b:
                    cover[max(0, a - wl.W + 1):a] = True
            union += int(cover.sum())
        out["absorb"].append(rows * H * (dc + D) * 2 + H * dc * D * 2)
        out["attention"].append(rows * H * (D + dr + D) * 2 + (union + rows) * (D + dr) * 2)
        out["w_uv"].append(rows * H * (D + dv) * 2 + H * dv * D * 2)
    # the last W_UV launch also writes the rows of padding blocks
    out["w_uv"][-1] += (wl.B * wl.N - len(kept)) * 5 * H * dv * 2
    return out


# Stage events of the MFMA backward, in launch order.  The two event slots
# after "index" mark launches folded into others (the anchor-order check into
# the index build, the accumulator clear into d_olat): their time counts as
# "index".
BWD_STAGES = ("index", "order", "clear", "absorb", "d_olat", "attention_bwd", "dkv",
              "dq_nope", "dw", "final")
BWD_FOLDED = ("order", "clear")


def bwd_useful_flop(anchors, keep, W, H, D, d_c, d_r, d_v, block=5) -> int:
    """Gradient products the backward must compute per kept block (the
    forward values it recomputes -- q_abs, scores, o_lat -- are not counted):
    per (query, head) 2 d_v D (W_UV^T dout) + 2 d_v D (dW_UV) + 2 D v (dP)
    + 2 (D + d_r) v (dq_abs, dq^R) + 4 D v + 2 d_r v (dc^KV, dk^R)
    + 2 d_c D (dq^C) + 2 d_c D (dW_UK); about twice the forward's count."""
    total = 0
    for a, k in zip(np.asarray(anchors).ravel(), np.asarray(keep).ravel()):
        if k:
            v = min(int(a), W - 1) + block
            total += block * H * (4 * d_v * D + 4 * d_c * D + 8 * D * v + 4 * d_r * v)
    return total


def bwd_stage_bytes(wl, anchors, keep):
    """Algorithmic HBM bytes of each backward launch (bf16 = 2 B, fp32
    accumulators 4 B): every input read once, every output written once,
    intermediates written by one launch and read by the next."""
    H, D, dc, dr, dv = wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v
    kept = [(b, int(anchors[b, n])) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    rows = 5 * len(kept)
    union = 0
    vsum = 0
    for b in range(wl.B):
        cover = np.zeros(wl.S, dtype=bool)
        for bb, a in kept:
            if bb == b:
                cover[max(0, a - wl.W + 1):a] = True
                vsum += min(a, wl.W - 1) + 5
        union += int(cover.sum())
    lat = rows * H * D * 2
    pm = len(kept) * 5 * H * 144 * 2
    # with ascending anchors in every sample the accumulator is not used
    # (per-block partials are gathered instead) and its clear is skipped
    ascending = all(np.all(np.diff(np.asarray(anchors[b])[np.asarray(keep[b]) != 0]) >= 0)
                    for b in range(wl.B))
    acc = 0 if ascending else wl.B * (wl.S + 5 * wl.N) * (D + dr) * 4
    part = vsum * (D + dr) * 4          # each block's partial rows
    out_kv = wl.B * (wl.S + 5 * wl.N) * (D + dr) * 2
    return {
        "absorb": rows * H * dc * 2 + H * dc * D * 2 + lat,
        "d_olat": rows * H * dv * 2 + H * dv * D * 2 + lat,
        "attention_bwd": 2 * lat + rows * H * dr * 2 + (union + rows) * (D + dr) * 2
                         + 2 * lat + rows * H * dr * 2 + 2 * pm + rows * H * dr * 2,
        "dkv": 2 * lat + rows * H * dr * 2 + 2 * pm + part,
        "dq_nope": lat + H * dc * D * 2 + rows * H * dc * 2,
        "dw": 2 * lat + rows * H * (dv + dc) * 2 + H * (dc + dv) * D * 2,
        "final": part + out_kv,
    }


def bench_backward(sd, torch, wl, tensors, a_dev, k_dev, anchors, keep, desc, sptr, hip,
                   steps, train_step=True):
    """Times dspark_attn_bwd on the same inputs (layer 0) with a seeded
    upstream gradient; per-launch durations from the library's stage events
    on one extra call."""
    import workloads as wk
    from workloads.device import to_torch
    t = tensors[0]
    dout = to_torch(wk.make_dout(wl, seed=11), wl.dtype, "cuda")
    B, S, L5, H = wl.B, wl.S, wl.q_len, wl.H
    shapes = {"dq_nope": (B, L5, H, wl.d_c), "dq_rope": (B, L5, H, wl.d_r),
              "dckv_ctx": (B, S, wl.D), "dkr_ctx": (B, S, wl.d_r),
              "dckv_blk": (B, L5, wl.D), "dkr_blk": (B, L5, wl.d_r),
              "dw_uk": (H, wl.d_c, wl.D), "dw_uv": (H, wl.d_v, wl.D)}
    g = {k: torch.empty(v, dtype=torch.bfloat16, device="cuda") for k, v in shapes.items()}
    ws = torch.empty(sd.bwd_workspace_size(desc), dtype=torch.uint8, device="cuda")
    args = (desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"], t["kr_blk"],
            t["w_uk"], t["w_uv"], a_dev, k_dev, dout, g, ws)
    w0, n_w = time.perf_counter(), 0
    while n_w < 3 or (time.perf_counter() - w0) < 0.1:
        sd.attn_bwd(*args, stream=sptr)
        n_w += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sd.attn_bwd(*args, stream=sptr)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    n_ev = sd.bwd_plan(desc)
    names = BWD_STAGES if n_ev == len(BWD_STAGES) + 1 else None
    # three instrumented calls back to back, per-stage medians: the first
    # call's event [0] lands on an idle stream, so its first stage also holds
    # the host's submission of the next launch
    evs = [hip.create(n_ev) for _ in range(3)]
    for ev in evs:
        sd.attn_bwd(*args, stream=sptr, stage_events=ev)
    torch.cuda.synchronize()
    stage_us = {}
    if names:
        for ev in evs:
            one = {}
            for i, s in enumerate(names):
                key = "index" if s in BWD_FOLDED else s
                one[key] = one.get(key, 0.0) + hip.elapsed_ms(ev[i], ev[i + 1]) * 1e3
            for key, v in one.items():
                stage_us.setdefault(key, []).append(v)
        stage_us = {k: float(np.median(v)) for k, v in stage_us.items()}
    for ev in evs:
        hip.destroy(ev)
    flop = bwd_useful_flop(anchors, keep, wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v)
    out = {"ms_per_step": round(wall * 1e3, 4), "steps": steps, "warmup": n_w,
           "useful_gflop_per_step": round(flop / 1e9, 3),
           "value": round(flop / wall / 1e12, 3), "unit": "TFLOP/s",
           "frac_of_bf16_peak": round(flop / wall / 1e12 / MI355X_BF16_PEAK_TFLOPS, 4),
           "stage_us": {k: round(v, 2) for k, v in stage_us.items()}}
    if stage_us:
        nb = bwd_stage_bytes(wl, anchors, keep)
        dom = max(stage_us, key=lambda s: stage_us[s])
        ach = nb[dom] / (stage_us[dom] * 1e-6) / 1e9
        out["stage_gbs"] = {k: round(nb[k] / (v * 1e-6) / 1e9, 1) for k, v in stage_us.items()
                            if k in nb and v > 0}
        out["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1),
                           "peak": MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(ach / MI355X_HBM_PEAK_GBS, 4),
                           "traffic": bwd_measured_traffic(dom, wl.name),
                           "avg_launch_us": round(stage_us[dom], 2),
                           "algorithmic_bytes_per_launch": nb[dom]}
    if not train_step:
        return out
    # a training step: the forward on the backward's workspace, then the
    # backward reusing its index and q_abs
    fout = torch.empty((B, L5, H, wl.d_v), dtype=torch.bfloat16, device="cuda")
    fargs = args[:11] + (fout, ws)
    for _ in range(3):
        sd.attn_fwd(*fargs, stream=sptr, for_backward=True)
        sd.attn_bwd(*args, stream=sptr, reuse_forward=2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sd.attn_fwd(*fargs, stream=sptr, for_backward=True)
        sd.attn_bwd(*args, stream=sptr, reuse_forward=2)
    torch.cuda.synchronize()
    step = (time.perf_counter() - t0) / steps
    fflop = useful_flop(anchors, keep, wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v)
    out["train_step"] = {"what": "dspark_attn_fwd then dspark_attn_bwd on one workspace "
                                 "(the forward leaves its softmax probabilities; reuse_forward 2: "
                                 "no index rebuild, no q_abs / o_lat / score recompute)",
                         "ms_per_step": round(step * 1e3, 4),
                         "useful_gflop_per_step": round((flop + fflop) / 1e9, 3),
                         "value": round((flop + fflop) / step / 1e12, 3), "unit": "TFLOP/s"}
    # the same step captured once in a HIP graph and replayed
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sd.attn_fwd(*fargs, for_backward=True)
            sd.attn_bwd(*args, reuse_forward=2)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sd.attn_fwd(*fargs, for_backward=True)
            sd.attn_bwd(*args, reuse_forward=2)
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        gstep = (time.perf_counter() - t0) / steps
        out["train_step"]["graph_ms_per_step"] = round(gstep * 1e3, 4)
    except Exception as e:      # the eager figure stands
        out["train_step"]["graph_error"] = f"{type(e).__name__}: {e}"
    return out


LAYER_STAGES = ("input_norm", "q_a", "q_b", "kv_a", "attention", "o_proj")


def layer_flop(wl, anchors, keep, hidden, q_rank):
    """FLOP of the MLA block on the rows the masked attention needs: the
    query-side projections and o_proj for the rows of kept blocks, kv_a for
    the union of the kept windows plus the kept blocks' own rows, and the
    attention's useful FLOP.  Returns (total, {stage: flop})."""
    H, D, dc, dr, dv = wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v
    kept = [(b, int(anchors[b, n])) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    rows = 5 * len(kept)
    union = 0
    for b in range(wl.B):
        cover = np.zeros(wl.S, dtype=bool)
        for bb, a in kept:
            if bb == b:
                cover[max(0, a - wl.W + 1):a] = True
        union += int(cover.sum())
    st = {"q_a": 2 * rows * hidden * q_rank,
          "q_b": 2 * rows * q_rank * H * (dc + dr),
          "kv_a": 2 * (union + rows) * hidden * (D + dr),
          "attention": useful_flop(anchors, keep, wl.W, H, D, dc, dr, dv),
          "o_proj": 2 * rows * H * dv * hidden}
    return sum(st.values()), st


def bench_layer(sd, torch, wl, tensors, a_dev, k_dev, anchors, keep, desc, sptr, hip, steps,
                hidden=6144, q_rank=2048, tune=True):
    """Times dspark_mla_layer_fwd (the MLA block of one draft layer) on the
    same attention inputs' workload, with seeded hidden states and weights of
    the page's shapes (d = 6144, q_lora_rank = 2048)."""
    import workloads as wk
    from workloads.device import to_torch
    li = wk.make_layer_inputs(wl, hidden, q_rank, seed=5)
    t = tensors[0]
    w = {k: to_torch(getattr(li, k), wl.dtype, "cuda") for k in ("g_in", "w_qa", "g_qa", "w_qb",
                                                                 "w_kva", "g_kva", "w_o")}
    w["w_uk"], w["w_uv"] = t["w_uk"], t["w_uv"]
    hd = to_torch(li.h_draft, wl.dtype, "cuda")
    hc = to_torch(li.h_ctx, wl.dtype, "cuda")
    del li
    ld = sd.make_layer_desc(desc, hidden, q_rank, max_kept_blocks=int(keep.sum()))
    out = torch.empty_like(hd)
    ws = torch.empty(sd.layer_workspace_size(ld), dtype=torch.uint8, device="cuda")
    args = (ld, hd, hc, w, a_dev, k_dev, out, ws)
    # pick the GEMM kernels for these shapes first (synchronous, seconds)
    t_tune = time.perf_counter()
    choices = None
    if tune:
        choices = sd.mla_layer_tune(*args, stream=sptr)
    else:
        sd.mla_layer_fwd(*args, stream=sptr)
    torch.cuda.synchronize()
    t_tune = time.perf_counter() - t_tune
    w0, n_w = time.perf_counter(), 0
    while n_w < 3 or (time.perf_counter() - w0) < 0.1:
        sd.mla_layer_fwd(*args, stream=sptr, gemm_choices=choices)
        n_w += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sd.mla_layer_fwd(*args, stream=sptr, gemm_choices=choices)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = hip.create(len(LAYER_STAGES) + 1)
    sd.mla_layer_fwd(*args, stream=sptr, stage_events=ev, gemm_choices=choices)
    torch.cuda.synchronize()
    stage_us = {s: hip.elapsed_ms(ev[i], ev[i + 1]) * 1e3 for i, s in enumerate(LAYER_STAGES)}
    hip.destroy(ev)
    flop, st_flop = layer_flop(wl, anchors, keep, hidden, q_rank)
    dom = max(("q_a", "q_b", "kv_a", "o_proj"), key=lambda s: stage_us[s])
    ach = st_flop[dom] / (stage_us[dom] * 1e-6) / 1e12
    return {"ms_per_step": round(wall * 1e3, 4), "steps": steps, "warmup": n_w,
            "hidden": hidden, "q_rank": q_rank, "gemm_tuning_s": round(t_tune, 2),
            "gemm_choices": choices.as_list() if choices is not None else None,
            "useful_gflop_per_step": round(flop / 1e9, 3),
            "value": round(flop / wall / 1e12, 3), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(flop / wall / 1e12 / MI355X_BF16_PEAK_TFLOPS, 4),
            "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
            "roofline": {"kernel": dom + " GEMM (rocBLAS)", "bound": "mfma",
                         "achieved": round(ach, 1), "peak": MI355X_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / MI355X_BF16_PEAK_TFLOPS, 4),
                         "traffic": None, "avg_launch_us": round(stage_us[dom], 2),
                         "algorithmic_flop_per_launch": st_flop[dom]}}


LOSS_STAGES = ("index_gather", "gemms", "stats", "l1", "terms_reduce")


def loss_flop(counted_steps, vocab, hidden, rank):
    """FLOP of the output head on the steps the eval mask counts (the only
    ones whose logits enter the loss): the lm_head for the draft and the
    teacher rows and the Markov bias.  Returns (total, {stage: flop})."""
    rows = int(counted_steps)
    st = {"lm_head_draft": 2 * rows * hidden * vocab, "lm_head_teacher": 2 * rows * hidden * vocab,
          "markov": 2 * rows * rank * vocab}
    return sum(st.values()), st


def bench_loss(sd, torch, wl, anchors, keep, sptr, hip, steps, vocab=154880, hidden=6144, rank=256,
               tune=True):
    """Times dspark_loss_fwd on seeded inputs of the page's shapes (V = 154880,
    d = 6144, markov rank 256) with the workload's anchors, keep mask and loss
    mask; max_kept_blocks is the number of kept blocks."""
    import workloads as wk
    from workloads.device import upload_loss
    from workloads.device import to_torch
    lh = wk.make_loss_inputs(wl, vocab, hidden, rank, seed=9)
    t = upload_loss(lh, wl.loss_mask, anchors, keep)
    # lm_head and markov_w2 side by side in one [V, d + r] array: the draft
    # and teacher logits are then one GEMM
    buf = to_torch(np.concatenate([lh.w_lm, lh.w_m2], axis=1), wl.dtype, "cuda")
    t["w_lm"], t["w_m2"] = buf, buf[:, hidden:]
    del lh
    kept = int(keep.sum())
    mk = lambda counted: sd.make_loss_desc(wl.B, wl.S, wl.N, vocab, hidden, rank, dtype=wl.dtype,
                                           max_kept_blocks=kept, w_lm_ld=hidden + rank,
                                           w_m2_ld=hidden + rank, max_counted_steps=counted)
    terms = torch.empty((4, wl.B, wl.N, 5), dtype=torch.float32, device="cuda")
    em = torch.empty((wl.B, wl.N, 5), dtype=torch.uint8, device="cuda")
    loss = torch.empty(5, dtype=torch.float32, device="cuda")
    # one call bounded by the kept blocks tells the counted steps; the timed
    # calls form the logits of exactly those rows
    d = mk(0)
    ws = torch.empty(sd.loss_workspace_size(d), dtype=torch.uint8, device="cuda")
    sd.loss_fwd(d, t, terms, em, loss, ws, stream=sptr)
    counted = sd.loss_read_status(ws, stream=sptr)[3]
    d = mk(counted)
    args = (d, t, terms, em, loss, ws)
    t_tune = time.perf_counter()
    choices = None
    if tune:
        choices = sd.loss_tune(*args, stream=sptr)
    else:
        sd.loss_fwd(*args, stream=sptr)
    torch.cuda.synchronize()
    t_tune = time.perf_counter() - t_tune
    st = sd.loss_read_status(ws, stream=sptr)
    if st[0] != 0:
        raise RuntimeError(f"loss status {st}")
    w0, n_w = time.perf_counter(), 0
    while n_w < 2 or (time.perf_counter() - w0) < 0.1:
        sd.loss_fwd(*args, stream=sptr, gemm_choices=choices)
        n_w += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        sd.loss_fwd(*args, stream=sptr, gemm_choices=choices)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    ev = hip.create(len(LOSS_STAGES) + 1)
    sd.loss_fwd(*args, stream=sptr, stage_events=ev, gemm_choices=choices)
    torch.cuda.synchronize()
    stage_us = {s: hip.elapsed_ms(ev[i], ev[i + 1]) * 1e3 for i, s in enumerate(LOSS_STAGES)}
    hip.destroy(ev)
    flop, st_flop = loss_flop(counted, vocab, hidden, rank)
    vals = loss.cpu().tolist()
    gemm_tfs = flop / (stage_us["gemms"] * 1e-6) / 1e12
    # the statistics pass reads the draft and teacher logits of the counted rows once
    live = int(em.sum().item())
    stat_bytes = 2 * live * vocab * 4
    stat_gbs = stat_bytes / (stage_us["stats"] * 1e-6) / 1e9
    return {"ms_per_step": round(wall * 1e3, 4), "steps": steps, "warmup": n_w,
            "vocab": vocab, "hidden": hidden, "markov_rank": rank, "kept_blocks": kept,
            "logit_rows": 2 * counted,
            "counted_steps": live, "gemm_tuning_s": round(t_tune, 2),
            "gemm_choices": choices.as_list() if choices is not None else None,
            "useful_gflop_per_step": round(flop / 1e9, 3),
            "value": round(flop / wall / 1e12, 3), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(flop / wall / 1e12 / MI355X_BF16_PEAK_TFLOPS, 4),
            "loss": {"total": vals[0], "ce": vals[1], "l1": vals[2], "bce": vals[3]},
            "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
            "roofline": {"kernel": "logits GEMM (rocBLAS: [H | e ; z | 0] [W_lm | W2]^T)",
                         "bound": "mfma", "achieved": round(gemm_tfs, 1),
                         "peak": MI355X_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gemm_tfs / MI355X_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "avg_launch_us": round(stage_us["gemms"], 2),
                         "algorithmic_flop_per_launch": flop},
            "stats_pass": {"bound": "hbm", "achieved": round(stat_gbs, 1),
                           "peak": MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(stat_gbs / MI355X_HBM_PEAK_GBS, 4),
                           "traffic": side_measured_traffic(
                               "loss_stats", wl.name.startswith("headline") and vocab == 154880
                               and hidden == 6144 and rank == 256),
                           "algorithmic_bytes_per_launch": stat_bytes}}


def bench_decode(sd, torch, hip, steps, B=64, K=5, vocab=154880, C=128):
    """One decode step for B sequences at GLM dims (W = 128, a ring of C
    slots per sequence): dspark_cache_append of 5 rows, dspark_decode_attn,
    and dspark_spec_verify (rejection sampling, K drafted tokens).  Anchors
    are drawn uniformly from [W, 10^6); inputs are seeded."""
    import workloads as wk
    from workloads.device import to_torch
    dims = wk.GLM_DIMS
    W = dims["W"]
    rng = np.random.default_rng(31)
    anchors = rng.integers(W, 10**6, size=B).astype(np.int32)
    di = wk.make_decode_inputs(B, dims, "bf16", 5, seed=31)
    dev = lambda a: to_torch(a, "bf16", "cuda")
    attn = sd.make_desc(B=B, S=0, N=1, window=W, n_heads=dims["H"], d_latent=dims["D"],
                        d_nope=dims["d_c"], d_rope=dims["d_r"], d_v=dims["d_v"], dtype="bf16")
    d = sd.make_decode_desc(attn, C)
    cache_ckv = torch.randn((B, C, dims["D"]), device="cuda").to(torch.bfloat16)
    cache_kr = torch.randn((B, C, dims["d_r"]), device="cuda").to(torch.bfloat16)
    new_ckv, new_kr = dev(di.ctx_ckv), dev(di.ctx_kr)
    pos0 = torch.tensor(anchors - 5, device="cuda")
    n_new = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    a_dev = torch.tensor(anchors, device="cuda")
    act = torch.ones(B, dtype=torch.uint8, device="cuda")
    qn, qr, cb, kb = dev(di.q_nope), dev(di.q_rope), dev(di.ckv_blk), dev(di.kr_blk)
    wuk, wuv = dev(di.w_uk), dev(di.w_uv)
    out = torch.empty((B, 5, dims["H"], dims["d_v"]), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(sd.decode_workspace_size(d), dtype=torch.uint8, device="cuda")
    dl, tl, u, _ = wk.make_verify_inputs(B, K, vocab, seed=37)
    tok = torch.from_numpy(np.argmax(dl, axis=2).astype(np.int32)).to("cuda")
    dl, tl, u = (torch.from_numpy(x).to("cuda") for x in (dl, tl, u))
    vd = sd.make_verify_desc(B, K, vocab)
    vws = torch.empty(sd.verify_workspace_size(vd), dtype=torch.uint8, device="cuda")
    ap, ov = torch.empty((B, K), device="cuda"), torch.empty((B, K), device="cuda")
    na = torch.empty(B, dtype=torch.int32, device="cuda")
    nt = torch.empty(B, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)

    def append():
        sd.cache_append(d, pos0, n_new, new_ckv, new_kr, cache_ckv, cache_kr, stream=sptr)

    def attend():
        sd.decode_attn(d, qn, qr, cache_ckv, cache_kr, cb, kb, wuk, wuv, a_dev, act, out, ws,
                       stream=sptr)

    def verify():
        sd.spec_verify(vd, dl, tl, tok, u, ap, ov, na, nt, vws, stream=sptr)

    res = {}
    ev = hip.create(2)
    for name, fn in (("append", append), ("attention", attend), ("verify", verify)):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        hip.record(ev[0], sptr)
        for _ in range(steps):
            fn()
        hip.record(ev[1], sptr)
        res[name] = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
    hip.destroy(ev)
    st, _ = sd.read_device_status(ws, stream=sptr)
    if st != 0:
        raise RuntimeError(f"decode status {st}")
    vbytes = (4 * K + 1) * B * vocab * 4
    vgbs = vbytes / (res["verify"] * 1e-6) / 1e9
    return {"sequences": B, "drafted_tokens": K, "vocab": vocab, "cache_slots": C, "window": W,
            "steps": steps, "us": {k: round(v, 2) for k, v in res.items()},
            "us_per_step": round(sum(res.values()), 2),
            "verify_roofline": {"bound": "hbm", "achieved": round(vgbs, 1),
                                "peak": MI355X_HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(vgbs / MI355X_HBM_PEAK_GBS, 4),
                                "traffic": side_measured_traffic(
                                    "verify", (B, K, vocab) == (64, 5, 154880)),
                                "algorithmic_bytes_per_launch": vbytes},
            "mean_accepted": float(na.float().mean().item())}


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch loaded (one runtime per
    process), so that they can be recorded by the library on torch's stream."""

    def __init__(self):
        import torch  # noqa: F401  (brings in the runtime)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        assert self.hip.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def cpu_baseline(wl, anchors, keep, budget_s: float = 15.0):
    """The fp64 oracle as it stands, on a bounded sample of the same
    workload's kept blocks (timed on the host, single process)."""
    import oracle as O
    kept = [(b, n) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    rng = np.random.default_rng(0)
    order = rng.permutation(len(kept))
    n_blocks, spent, done, own = 4, 0.0, [], 0
    while spent < budget_s and len(done) < len(kept):
        pick = [kept[i] for i in order[len(done):len(done) + n_blocks]]
        t0 = time.perf_counter()
        O.forward(wl, 0, anchors, keep, form="gathered", blocks=pick)
        spent += time.perf_counter() - t0
        done += pick
        own += oracle_forward_flop(wl, anchors, pick)
        n_blocks *= 2
    flop = sum(useful_flop([anchors[b, n]], [1], wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v)
               for b, n in done)
    blas = blas_info()
    return {"value": flop / spent / 1e12, "unit": "TFLOP/s", "cores": blas["threads"],
            "kind": "oracle", "blocks_per_s": len(done) / spent,
            "oracle_flop": own, "oracle_tflops": own / spent / 1e12,
            "host_cores": len(os.sched_getaffinity(0)), "blas": blas["name"],
            "blas_threads": blas["threads"], "precision": "fp64",
            "sample": f"{len(done)} random kept blocks of the same workload "
                      f"(fp64 numpy, gathered form, {spent:.1f} s)"}


def oracle_forward_flop(wl, anchors, pick) -> int:
    """What the oracle's gathered forward itself computes for one call over
    the blocks `pick`: per sample and head, K and V expanded at every column
    the picked rows see (2 (d_c + d_v) D per column: K's latent part and V),
    then per query row and head the scores and the weighted sum over its v
    visible keys (2 v (d_c + d_r) + 2 v d_v)."""
    total = 0
    for b in sorted({b for b, _ in pick}):
        cover = np.zeros(wl.S, dtype=bool)
        n_blk, vsum = 0, 0
        for bb, n in pick:
            if bb != b:
                continue
            a = int(anchors[b, n])
            cover[max(0, a - wl.W + 1):a] = True
            n_blk += 1
            vsum += min(a, wl.W - 1) + 5
        cols = int(cover.sum()) + 5 * n_blk
        total += wl.H * (cols * 2 * (wl.d_c + wl.d_v) * wl.D
                         + 5 * vsum * (2 * (wl.d_c + wl.d_r) + 2 * wl.d_v))
    return total


def blas_info() -> dict:
    """The BLAS library numpy's products run on and its thread count (the
    oracle's only multi-threaded part)."""
    try:
        import threadpoolctl
        libs = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = libs[0]
            return {"name": f"{i.get('internal_api', '?')} {i.get('version', '')}".strip(),
                    "threads": int(i.get("num_threads", 1))}
    except Exception:
        pass
    return {"name": "unknown", "threads": len(os.sched_getaffinity(0))}


def _oracle_threads() -> int:
    return blas_info()["threads"]


def _grow(run, items, budget_s, start=2):
    """run(sample) on growing slices of items (doubling) until budget_s of
    host time is spent; returns (items done, seconds)."""
    n, spent, done = start, 0.0, []
    while spent < budget_s and len(done) < len(items):
        pick = items[len(done):len(done) + n]
        t0 = time.perf_counter()
        run(pick)
        spent += time.perf_counter() - t0
        done += pick
        n *= 2
    return done, spent


def bwd_cpu_baseline(wl, anchors, keep, budget_s):
    """The oracle's backward (fp64, gathered form) on random kept blocks of the
    same workload, as useful TFLOP/s."""
    import oracle as O
    import workloads as wk
    dout = wk.make_dout(wl, seed=7)
    kept = [(b, n) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    order = [kept[i] for i in np.random.default_rng(1).permutation(len(kept))]
    done, spent = _grow(lambda pick: O.backward(wl, dout, anchors=anchors, keep=keep,
                                                form="gathered", blocks=pick), order, budget_s)
    flop = sum(bwd_useful_flop([anchors[b, n]], [1], wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v)
               for b, n in done)
    return {"value": flop / spent / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"{len(done)} random kept blocks of the same workload "
                                        f"(fp64 numpy, {spent:.1f} s)"}


def layer_cpu_baseline(budget_s, hidden=6144, q_rank=2048):
    """The oracle's MLA block (fp64) on the headline recipe at a smaller size
    (its projections run over every row), as useful TFLOP/s."""
    import oracle as O
    import workloads as wk
    flop = spent = 0.0
    runs = 0
    for S, N in ((512, 8), (1024, 16), (2048, 32)):
        wl = wk.scaled(4, S=S, N=N)
        li = wk.make_layer_inputs(wl, hidden, q_rank, seed=5)
        t0 = time.perf_counter()
        O.layer_forward(wl, li)
        spent += time.perf_counter() - t0
        flop += layer_flop(wl, wl.anchors, wl.keep, hidden, q_rank)[0]
        runs += 1
        if spent > budget_s:
            break
    return {"value": flop / spent / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"{runs} headline-recipe workloads up to S={S}, N={N} "
                                        f"(d=6144, q_lora_rank=2048; fp64 numpy, {spent:.1f} s)"}


def loss_cpu_baseline(wl, anchors, keep, budget_s, vocab=20000, hidden=6144, rank=256):
    """The oracle's output head and loss (fp64) on random kept blocks of the
    same anchors with a 20000-token vocabulary (its cost is linear in V), as
    useful TFLOP/s."""
    import oracle as O
    import workloads as wk
    lh = wk.make_loss_inputs(wl, vocab, hidden, rank, seed=9)
    kept = [(b, n) for b in range(wl.B) for n in range(wl.N) if keep[b, n]]
    order = [kept[i] for i in np.random.default_rng(2).permutation(len(kept))]
    done, spent = _grow(lambda pick: O.loss_head(lh, wl.loss_mask, anchors, keep, blocks=pick),
                        order, budget_s, start=8)
    flop = 2 * 5 * len(done) * vocab * (2 * hidden + rank)
    return {"value": flop / spent / 1e12, "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"{len(done)} random kept blocks, V={vocab} "
                                        f"(fp64 numpy, {spent:.1f} s)"}


def decode_cpu_baseline(budget_s, K=5, vocab=154880):
    """The oracle's decode step (decode attention over a ring and
    rejection-sampling verification at V = 154880, fp64) for sequences of the
    decode bench's shape, as sequences per second."""
    import oracle as O
    import workloads as wk
    dims = wk.GLM_DIMS
    B = 4
    di = wk.make_decode_inputs(B, dims, "bf16", 5, seed=31)
    C = dims["W"]
    ring = np.zeros((B, C, dims["D"]), np.uint16), np.zeros((B, C, dims["d_r"]), np.uint16)
    dl, tl, u, _ = wk.make_verify_inputs(B, K, vocab, seed=37)
    anchors = np.full(B, 5000, np.int32)
    spent, seqs = 0.0, 0
    while spent < budget_s:
        t0 = time.perf_counter()
        O.decode_attention(ring[0], ring[1], anchors, np.ones(B), di.q_nope, di.q_rope,
                           di.ckv_blk, di.kr_blk, di.w_uk, di.w_uv, dims["W"], 10000.0, "bf16")
        for b in range(B):
            O.spec_verify(dl[b], tl[b], np.argmax(dl[b], axis=1), u[b].astype(np.float64))
        spent += time.perf_counter() - t0
        seqs += B
    return {"value": seqs / spent, "unit": "sequences/s", "cores": _oracle_threads(),
            "kind": "oracle", "sample": f"{seqs} sequences (decode attention + verification, "
                                        f"fp64 numpy, {spent:.1f} s)"}


# ---------------------------------------------------------------------------
# the forward: one workload, timed three ways
# ---------------------------------------------------------------------------

def kernel_useful_flop(anchors, keep, W, H, D, d_c, d_r, d_v, block=5) -> dict:
    """The useful FLOP of each forward kernel (the split of useful_flop):
    absorb 2 d_c D, attention 2 (D + d_r) v + 2 D v, W_UV 2 D d_v per query
    row and head."""
    rows = v_rows = 0
    for a, k in zip(np.asarray(anchors).ravel(), np.asarray(keep).ravel()):
        if k:
            rows += block
            v_rows += block * (min(int(a), W - 1) + block)
    return {"absorb": rows * H * 2 * d_c * D,
            "attention": v_rows * H * (2 * (D + d_r) + 2 * D),
            "w_uv": rows * H * 2 * D * d_v}


def forward_algorithmic_bytes(wl, anchors, keep) -> int:
    """HBM bytes the method itself needs per forward call (inputs read once,
    output written once; bf16 = 2 B, fp32 = 4 B): the q^C and q^R rows of
    kept blocks, the context rows in the union of the kept windows, the
    kept blocks' own key rows, W_UK and W_UV, the anchors and keep flags,
    and every output row (zeros for padding blocks)."""
    H, D, dc, dr, dv = wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v
    el = 2 if wl.dtype == "bf16" else 4
    kept_rows = 5 * int(np.asarray(keep).sum())
    union = 0
    for b in range(wl.B):
        cover = np.zeros(wl.S, dtype=bool)
        for n in range(wl.N):
            if keep[b, n]:
                a = int(anchors[b, n])
                cover[max(0, a - wl.W + 1):a] = True
        union += int(cover.sum())
    return (kept_rows * H * (dc + dr) * el + (union + kept_rows) * (D + dr) * el
            + H * (dc + dv) * D * el + wl.B * wl.N * 5 + wl.B * 5 * wl.N * H * dv * el)


def prepare_forward(sd, torch, wl, chunk_blocks=0, aux_stream=False, one_launch=False):
    """Anchors, device tensors of every layer, outputs, workspace and one
    bound call per layer."""
    from workloads.device import upload_anchors, upload_layer
    if wl.anchor_source == "sampler":
        anchors = np.zeros((wl.B, wl.N), np.int32)
        keep = np.zeros((wl.B, wl.N), np.uint8)
        for b in range(wl.B):
            anchors[b], keep[b] = sd.select_anchors_host(wl.loss_mask[b], wl.N,
                                                         wl.sampler_seed + b)
    else:
        anchors, keep = wl.anchors, wl.keep
    L = len(wl.layers)
    tensors = [upload_layer(wl, i) for i in range(L)]
    a_dev, k_dev = upload_anchors(anchors, keep)
    desc = sd.make_desc(B=wl.B, S=wl.S, N=wl.N, window=wl.W, n_heads=wl.H, d_latent=wl.D,
                        d_nope=wl.d_c, d_rope=wl.d_r, d_v=wl.d_v, rope_base=wl.rope_base,
                        dtype=wl.dtype)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    outs = [torch.empty((wl.B, wl.q_len, wl.H, wl.d_v), dtype=tdt, device="cuda")
            for _ in range(L)]
    ws = torch.empty(sd.workspace_size(desc), dtype=torch.uint8, device="cuda")
    sptr = int(torch.cuda.current_stream().cuda_stream)
    n_chunks, chunk, n_ev = sd.attn_plan(desc, chunk_blocks=chunk_blocks, one_launch=one_launch)
    aux, aux_ev = None, None
    if aux_stream and n_chunks > 1:
        aux = torch.cuda.Stream()
        aux_ev = HIP.create(2)
    calls = [sd.BoundFwd(desc, t["q_nope"], t["q_rope"], t["ckv_ctx"], t["kr_ctx"], t["ckv_blk"],
                         t["kr_blk"], t["w_uk"], t["w_uv"], a_dev, k_dev, outs[l], ws, stream=sptr,
                         chunk_blocks=chunk_blocks, n_stage_events=n_ev, aux_stream=aux,
                         aux_events=aux_ev, one_launch=one_launch)
             for l, t in enumerate(tensors)]
    return dict(wl=wl, anchors=anchors, keep=keep, tensors=tensors, a_dev=a_dev, k_dev=k_dev,
                desc=desc, outs=outs, ws=ws, sptr=sptr, calls=calls, n_chunks=n_chunks,
                chunk=chunk, n_ev=n_ev, aux=aux, aux_ev=aux_ev, L=L, one_launch=one_launch)


def stage_times(ev, n_ev, n_chunks, live, one_launch=False):
    """Per-stage milliseconds of one instrumented call from its stage events:
    the index build, then absorb / attention / W_UV summed over the call's
    rounds (and each live round's own), or the generic kernel, or the
    one-launch kernel."""
    if n_ev == 3 and one_launch:   # [0] index + padding fill [1] one launch [2]
        return {"index+fill": HIP.elapsed_ms(ev[0], ev[1]),
                "one_launch": HIP.elapsed_ms(ev[1], ev[2])}, None
    if n_ev == 3:      # generic path: [0] index + RoPE table [1] kernel [2]
        return {"index+rope": HIP.elapsed_ms(ev[0], ev[1]),
                "generic": HIP.elapsed_ms(ev[1], ev[2])}, None
    out = {STAGES[0]: HIP.elapsed_ms(ev[0], ev[1])}
    per_round = {s: [] for s in STAGES[1:]}
    for c in range(n_chunks):
        marks = (ev[2 + 4 * c], ev[3 + 4 * c], ev[4 + 4 * c], ev[5 + 4 * c])
        for k, s in enumerate(STAGES[1:]):
            ms = HIP.elapsed_ms(marks[k], marks[k + 1])
            out[s] = out.get(s, 0.0) + ms
            if c < live:
                per_round[s].append(ms)
    return out, per_round


def measure_forward(torch, fw, steps, warmup, samples, sample_steps, stage_steps):
    """Warm-up (exactly `warmup` steps), then:
      1. `samples` samples of `sample_steps` back-to-back steps, with one
         hipEvent on the launch stream between samples (none inside one):
         the median over samples of the time per step;
      2. for several layers, 50 steps with an event at every layer boundary
         (per-layer medians);
      3. `stage_steps` calls per layer with the library's stage events
         between its kernels, after one such call that is dropped (those
         events order the kernels around them, so they stay out of the
         other passes);
      4. exactly `steps` steps with no event at all, between two
         synchronisations (its mean is reported beside the median).
    A step is one forward call per layer."""
    calls, L, sptr = fw["calls"], fw["L"], fw["sptr"]
    for _ in range(warmup):
        for call in calls:
            call()
    st, fb = fw["sd"].read_device_status(fw["ws"], stream=sptr)
    assert st == 0, fw["sd"].last_error()
    # 1. samples
    marks = HIP.create(samples + 1)
    HIP.record(marks[0], sptr)
    for i in range(samples):
        for _ in range(sample_steps):
            for call in calls:
                call()
        HIP.record(marks[i + 1], sptr)
    torch.cuda.synchronize()
    per_step = np.array([HIP.elapsed_ms(marks[j], marks[j + 1]) for j in range(samples)])
    per_step /= sample_steps
    HIP.destroy(marks)
    # 2. layers
    layer_ms = None
    if L > 1:
        n = 50
        marks = HIP.create(n * L + 1)
        HIP.record(marks[0], sptr)
        for i in range(n):
            for l, call in enumerate(calls):
                call()
                HIP.record(marks[i * L + l + 1], sptr)
        torch.cuda.synchronize()
        lay = np.array([HIP.elapsed_ms(marks[j], marks[j + 1])
                        for j in range(n * L)]).reshape(n, L)
        HIP.destroy(marks)
        layer_ms = [float(np.median(lay[:, l])) for l in range(L)]
    # 3. stage pass
    n_ev, n_chunks = fw["n_ev"], fw["n_chunks"]
    live = n_chunks if n_ev == 3 else min(n_chunks, -(-int(fw["keep"].sum()) // fw["chunk"]))
    per_stage, per_round = {}, None
    # one leading instrumented call is dropped: its event [0] lands on an
    # idle stream, so its first stage also holds the host's submission of
    # the next launch
    ev = HIP.create((stage_steps * L + 1) * n_ev)
    for i in range(stage_steps * L + 1):
        calls[(i - 1) % L].with_events(ev[i * n_ev:(i + 1) * n_ev])
    torch.cuda.synchronize()
    for j in range(1, stage_steps * L + 1):
        tot, rounds = stage_times(ev[j * n_ev:(j + 1) * n_ev], n_ev, n_chunks, live,
                                  fw["one_launch"])
        for s, v in tot.items():
            per_stage.setdefault(s, []).append(v)
        if rounds is not None:
            if per_round is None:
                per_round = {s: [] for s in rounds}
            for s, v in rounds.items():
                per_round[s].append(v)
    HIP.destroy(ev)
    # 4. the timed loop
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for call in calls:
            call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"median_ms": float(np.median(per_step)), "p10_ms": float(np.percentile(per_step, 10)),
            "p90_ms": float(np.percentile(per_step, 90)), "layer_median_ms": layer_ms,
            "loop_mean_ms": wall / max(steps, 1) * 1e3,
            "stage_us": {s: float(np.mean(v)) * 1e3 for s, v in per_stage.items()},
            "launch_us": ({s: float(np.mean(v)) * 1e3 for s, v in per_round.items()}
                          if per_round else None),
            "live_rounds": live}


def config_summary(k, fw, m) -> dict:
    """Compact per-configuration record for the `configs` object."""
    wl, anchors, keep = fw["wl"], fw["anchors"], fw["keep"]
    flop = useful_flop(anchors, keep, wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v) * fw["L"]
    kept = int(keep.sum()) * fw["L"]
    med = m["median_ms"] * 1e-3
    out = {"workload": wl.name, "dtype": wl.dtype, "kept_blocks": kept,
           "useful_gflop": round(flop / 1e9, 3), "median_ms": round(m["median_ms"], 4),
           "tflops": round(flop / med / 1e12, 2), "blocks_per_s": round(kept / med, 1),
           "frac_of_bf16_peak": round(flop / med / 1e12 / MI355X_BF16_PEAK_TFLOPS, 4),
           "stage_us": {s: round(v, 1) for s, v in m["stage_us"].items()}}
    if m["layer_median_ms"]:
        out["layer_median_ms"] = [round(v, 4) for v in m["layer_median_ms"]]
    return out


HIP = None


def main():
    global HIP
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--samples", type=int, default=50,
                    help="samples whose median time per step is reported (at least 50)")
    ap.add_argument("--sample-steps", type=int, default=10,
                    help="back-to-back steps per sample (events only between samples)")
    ap.add_argument("--stage-steps", type=int, default=10,
                    help="calls of the separate pass that records the library's stage events")
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--chunk-blocks", type=int, default=0,
                    help="kept blocks per kernel round (0: the library default)")
    ap.add_argument("--aux-stream", action="store_true",
                    help="run odd kernel rounds on a second stream (with --chunk-blocks)")
    ap.add_argument("--one-launch", action="store_true",
                    help="time the opt-in one-launch forward (dspark_attn_opts.one_launch) "
                         "instead of the three kernels")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other four configurations (the 'configs' object)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the backward measurement (the 'backward' object)")
    ap.add_argument("--bwd-steps", type=int, default=20)
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the MLA block measurement (the 'layer' object)")
    ap.add_argument("--layer-steps", type=int, default=10)
    ap.add_argument("--no-loss", action="store_true",
                    help="skip the output head and loss measurement (the 'loss' object)")
    ap.add_argument("--loss-steps", type=int, default=5)
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the inference-time drafting measurement (the 'decode' object)")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-train-step", action="store_true",
                    help="skip the forward + backward training-step timing (for counter runs: "
                         "its forward calls follow a backward that leaves their inputs cached)")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the rocBLAS kernel choice of the layer and loss objects (for "
                         "counter runs; their GEMM times are then rocBLAS's defaults')")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--side-budget", type=float, default=6.0,
                    help="host seconds for the oracle baselines of the backward, layer, loss "
                         "and decode objects")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="only run a plain device copy of this many MiB (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 2**20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))
        return

    import torch
    import workloads as wk
    import speculative_decoding_draft_amd as sd

    HIP = HipEvents()
    samples = max(args.samples, 50)
    R = max(args.sample_steps, 1)

    # the other configurations first, each freed before the next
    configs = {}
    if not args.no_configs:
        for k in (1, 2, 3, 4, 5):
            if k == args.config:
                continue
            log_progress(f"config {k}")
            fw = prepare_forward(sd, torch, wk.config(k))
            fw["sd"] = sd
            m = measure_forward(torch, fw, 0, args.warmup, samples, R, 5)
            configs[str(k)] = config_summary(k, fw, m)
            del fw
            torch.cuda.empty_cache()

    log_progress(f"config {args.config} (headline line)")
    wl = wk.config(args.config)
    fw = prepare_forward(sd, torch, wl, args.chunk_blocks, args.aux_stream, args.one_launch)
    fw["sd"] = sd
    anchors, keep, L = fw["anchors"], fw["keep"], fw["L"]
    K = args.steps
    m = measure_forward(torch, fw, K, args.warmup, samples, R, args.stage_steps)
    configs[str(args.config)] = config_summary(args.config, fw, m)

    flop = useful_flop(anchors, keep, wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v) * L
    kept_blocks = int(keep.sum()) * L
    med_s = m["median_ms"] * 1e-3
    value = flop / med_s / 1e12
    stage_us = m["stage_us"]
    fast = "attention" in stage_us
    result = {
        "metric": "DSpark draft-attn fwd useful TFLOP/s + blocks/s at S=32K, N=1024 (1 GPU)",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(m["median_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "S": wl.S, "N": wl.N, "W": wl.W,
                   "heads": wl.H, "layers": L, "kept_blocks_per_layer": int(keep.sum()),
                   "parallelism": "none (1 GPU)"},
        "timing": {"value_from": f"median over {samples} samples of {R} back-to-back steps "
                                 f"(one hipEvent on the launch stream between samples)",
                   "p10_ms": round(m["p10_ms"], 4), "p90_ms": round(m["p90_ms"], 4),
                   "timed_loop_ms_per_step": round(m["loop_mean_ms"], 4),
                   "timed_loop": f"{K} steps, no events, synchronised on both sides",
                   "stage_events": f"separate pass of {args.stage_steps} calls",
                   "l2_flushed": False},
        "blocks_per_s": round(kept_blocks / med_s, 1),
        "frac_of_bf16_peak": round(value / MI355X_BF16_PEAK_TFLOPS, 4),
        "useful_gflop_per_step": round(flop / 1e9, 3),
        "stage_us": {s: round(v, 2) for s, v in stage_us.items()},
        "chunks": {"chunk_blocks": fw["chunk"], "launches_per_kernel": m["live_rounds"],
                   "streams": 2 if fw["aux"] is not None else 1,
                   "one_launch": bool(args.one_launch)},
        "roofline": None,
        "cpu_baseline": None,
    }
    if fast:
        # the dominant kernel against the bf16 MFMA peak: its useful FLOP per
        # launch / its average launch duration (stage events)
        kflop = kernel_useful_flop(anchors, keep, wl.W, wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v)
        live = m["live_rounds"]
        dom = max(("absorb", "attention", "w_uv"), key=lambda s: stage_us[s])
        avg_launch_us = m["launch_us"][dom]
        flop_per_launch = kflop[dom] / live
        achieved = flop_per_launch / (avg_launch_us * 1e-6) / 1e12
        impl = stage_bytes(wl, anchors, keep, fw["chunk"])
        impl_bytes = float(np.mean(impl[dom][:live]))
        n_blocks = wl.B * wl.N
        measured = {s: measured_traffic(s, wl.name, fw["chunk"], n_blocks)
                    for s in ("absorb", "attention", "w_uv")}
        fwd_alg = forward_algorithmic_bytes(wl, anchors, keep)
        fwd_meas = (sum(measured.values()) if all(v is not None for v in measured.values())
                    else None)
        result["roofline"] = {
            "kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
            "peak": MI355X_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4),
            "traffic": measured[dom], "traffic_source": PMC_SOURCE,
            "avg_launch_us": round(avg_launch_us, 2),
            "useful_flop_per_launch": int(flop_per_launch),
            "implementation_bytes_per_launch": round(impl_bytes),
            "implementation_gbs": round(impl_bytes / (avg_launch_us * 1e-6) / 1e9, 1),
            "forward": {"algorithmic_bytes": fwd_alg, "measured_traffic": fwd_meas,
                        "traffic_ratio": (round(fwd_meas / fwd_alg, 3) if fwd_meas else None),
                        "useful_flop": int(flop / L),
                        "intensity_flop_per_byte": round(flop / L / fwd_alg, 1)}}
    if not args.no_cpu_baseline:
        log_progress("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(wl, anchors, keep, args.cpu_budget)
    tensors, a_dev, k_dev, desc, sptr = fw["tensors"], fw["a_dev"], fw["k_dev"], fw["desc"], fw["sptr"]
    if not args.no_bwd and wl.dtype == "bf16":
        log_progress("backward")
        try:
            result["backward"] = bench_backward(sd, torch, wl, tensors, a_dev, k_dev, anchors,
                                                keep, desc, sptr, HIP, args.bwd_steps,
                                                train_step=not args.no_train_step)
            if not args.no_cpu_baseline:
                result["backward"]["cpu_baseline"] = bwd_cpu_baseline(wl, anchors, keep,
                                                                       args.side_budget)
        except Exception as e:   # the forward line is still reported
            result["backward"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_layer and wl.dtype == "bf16":
        log_progress("layer")
        try:
            result["layer"] = bench_layer(sd, torch, wl, tensors, a_dev, k_dev, anchors, keep,
                                          desc, sptr, HIP, args.layer_steps, tune=not args.no_tune)
            if not args.no_cpu_baseline:
                result["layer"]["cpu_baseline"] = layer_cpu_baseline(args.side_budget)
        except Exception as e:   # the forward line is still reported
            result["layer"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_loss and wl.dtype == "bf16":
        log_progress("loss")
        try:
            result["loss"] = bench_loss(sd, torch, wl, anchors, keep, sptr, HIP, args.loss_steps,
                                        tune=not args.no_tune)
            if not args.no_cpu_baseline:
                result["loss"]["cpu_baseline"] = loss_cpu_baseline(wl, anchors, keep,
                                                                   args.side_budget)
        except Exception as e:   # the forward line is still reported
            result["loss"] = {"error": f"{type(e).__name__}: {e}"}
    if not args.no_decode and wl.dtype == "bf16":
        log_progress("decode")
        try:
            result["decode"] = bench_decode(sd, torch, HIP, args.decode_steps)
            if not args.no_cpu_baseline:
                result["decode"]["cpu_baseline"] = decode_cpu_baseline(args.side_budget)
        except Exception as e:   # the forward line is still reported
            result["decode"] = {"error": f"{type(e).__name__}: {e}"}
    # last, so that it stays in view at the end of the line
    result["configs"] = {k: configs[k] for k in sorted(configs)}
    print(json.dumps(result), flush=True)


def log_progress(what: str) -> None:
    print(f"[bench] {what}", file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
