"""Seeded synthetic inputs for the DSpark draft-attention forward.

This module is the only code shared by the fp64 oracle and the HIP path.  It
draws random numbers and lays them out; it contains none of the method's
arithmetic (no mask, no RoPE, no attention, no candidate-anchor rule).

Shapes follow the GLM-5.2 DSpark design page (parameter summary and the
"QKV construction" section): per draft layer the attention consumes

    q_nope  [B, 5N, H, d_c]   q_rope [B, 5N, H, d_r]   (unrotated)
    ckv_ctx [B, S, D]         kr_ctx [B, S, d_r]       (context latents)
    ckv_blk [B, 5N, D]        kr_blk [B, 5N, d_r]      (draft-block latents)
    w_uk    [H, d_c, D]       w_uv   [H, d_v, D]       (kv_b_proj split, out x in)
    anchors [B, N] int32      keep   [B, N] uint8

bf16 tensors are produced in fp32 and rounded to bf16 with round-to-nearest-
even here, and stored as raw uint16 bit patterns; both sides consume exactly
those values.  Activations are N(0, 1); weights are N(0, 1/D) (variance 1/D).

Anchors are never derived from the loss mask here.  A recipe either places
anchors itself and then forces loss_mask[A] = loss_mask[A+1] = 1 so that they
are valid by construction (positions are drawn from [0, S-3], because the
page resets loss_mask[S-1] to 0 on read), or it hands the loss mask and a
sampler seed to each side, which runs its own anchor sampler.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

BLOCK = 5

# GLM-5.2 DSpark draft attention dims (design page, parameter summary).
GLM_DIMS = dict(H=64, D=512, d_c=192, d_r=64, d_v=256, W=128)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); raw bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Layer:
    q_nope: np.ndarray
    q_rope: np.ndarray
    ckv_ctx: np.ndarray
    kr_ctx: np.ndarray
    ckv_blk: np.ndarray
    kr_blk: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    S: int
    N: int
    W: int
    H: int
    D: int
    d_c: int
    d_r: int
    d_v: int
    dtype: str                      # "bf16" (uint16 bit arrays) or "f32"
    rope_base: float
    loss_mask: np.ndarray           # [B, S] uint8
    anchors: Optional[np.ndarray]   # [B, N] int32, None when anchor_source == "sampler"
    keep: Optional[np.ndarray]      # [B, N] uint8
    anchor_source: str              # "given" or "sampler"
    sampler_seed: int
    layers: List[Layer]
    block: int = BLOCK

    @property
    def q_len(self) -> int:
        return self.block * self.N

    def desc(self) -> dict:
        return dict(B=self.B, S=self.S, N=self.N, block=self.block, window=self.W,
                    n_heads=self.H, d_latent=self.D, d_nope=self.d_c, d_rope=self.d_r,
                    d_v=self.d_v, rope_base=self.rope_base, dtype=self.dtype)


# --------------------------------------------------------------------------
# random tensors
# --------------------------------------------------------------------------

def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def _make_layer(rng, B, S, N, H, D, d_c, d_r, d_v, dtype) -> Layer:
    L5 = BLOCK * N
    wstd = float(1.0 / np.sqrt(D))
    # fixed draw order: q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv
    return Layer(
        q_nope=_normal(rng, (B, L5, H, d_c), 1.0, dtype),
        q_rope=_normal(rng, (B, L5, H, d_r), 1.0, dtype),
        ckv_ctx=_normal(rng, (B, S, D), 1.0, dtype),
        kr_ctx=_normal(rng, (B, S, d_r), 1.0, dtype),
        ckv_blk=_normal(rng, (B, L5, D), 1.0, dtype),
        kr_blk=_normal(rng, (B, L5, d_r), 1.0, dtype),
        w_uk=_normal(rng, (H, d_c, D), wstd, dtype),
        w_uv=_normal(rng, (H, d_v, D), wstd, dtype),
    )


def _force_valid(lm_row: np.ndarray, anchors_row: np.ndarray, keep_row: np.ndarray) -> None:
    for a, k in zip(anchors_row, keep_row):
        if k:
            lm_row[a] = 1
            lm_row[a + 1] = 1


# --------------------------------------------------------------------------
# anchor recipes (placement only; validity is forced, never tested here)
# --------------------------------------------------------------------------

def _recipe_uniform(rng, S, N, W, n_forced_low=0):
    """N distinct anchors uniform over [0, S-3]; the first n_forced_low of them
    are drawn from [0, W-2] (clamped windows)."""
    chosen = set()
    low = []
    while len(low) < n_forced_low:
        a = int(rng.integers(0, max(1, min(W - 1, S - 2))))
        if a not in chosen:
            chosen.add(a)
            low.append(a)
    while len(chosen) < N:
        chosen.add(int(rng.integers(0, S - 2)))
    anchors = np.array(sorted(chosen), dtype=np.int32)
    return anchors, np.ones(N, dtype=np.uint8)


def _recipe_clustered(rng, S, N, frac=0.30, cluster=8, span=64):
    """~frac of the anchors in clusters of `cluster` drawn without replacement
    from [c, c+span-1]; the rest uniform over the remaining positions."""
    n_cl = int(round(frac * N))
    chosen = set()
    while len(chosen) < n_cl:
        c = int(rng.integers(0, S - span - 1))
        take = min(cluster, n_cl - len(chosen))
        pool = [p for p in range(c, c + span) if p <= S - 3 and p not in chosen]
        if len(pool) < take:
            continue
        for p in rng.choice(np.array(pool), size=take, replace=False):
            chosen.add(int(p))
    while len(chosen) < N:
        chosen.add(int(rng.integers(0, S - 2)))
    anchors = np.array(sorted(chosen), dtype=np.int32)
    return anchors, np.ones(N, dtype=np.uint8)


def _recipe_headline(rng, S, N, W, pad_frac=0.25, low_frac=0.05):
    """pad_frac of the slots are padding (keep=0, garbage anchor values);
    low_frac of the slots hold clamped-window anchors in [0, W-2] that include
    0, 1 and W-2; the rest are uniform over [W-1, S-3].  Kept anchors ascend
    across slots."""
    n_pad = int(round(pad_frac * N))
    n_low = int(round(low_frac * N))
    n_hi = N - n_pad - n_low
    if n_low > W - 1 or n_hi > S - W - 1:
        raise ValueError(f"headline recipe: {n_low} clamped anchors need W - 1 >= {n_low} and "
                         f"{n_hi} others need S - W - 1 >= {n_hi} distinct positions")
    low = {0, 1, W - 2} if n_low >= 3 else set()
    while len(low) < n_low:
        low.add(int(rng.integers(0, W - 1)))
    hi = set()
    while len(hi) < n_hi:
        hi.add(int(rng.integers(W - 1, S - 2)))
    kept = np.array(sorted(low) + sorted(hi), dtype=np.int32)
    pad_slots = np.sort(rng.choice(N, size=n_pad, replace=False))
    keep = np.ones(N, dtype=np.uint8)
    keep[pad_slots] = 0
    anchors = np.empty(N, dtype=np.int32)
    anchors[keep == 1] = kept
    garbage = np.array([-1, S + 7, -(2 ** 31), 2 ** 31 - 1, S - 1, S], dtype=np.int64)
    anchors[keep == 0] = garbage[np.arange(n_pad) % len(garbage)].astype(np.int32)
    return anchors, keep


def make_workload(name: str, *, B: int, S: int, N: int, dims: dict, dtype: str,
                  recipe: str, seed: int, layers: int = 1, rope_base: float = 10000.0,
                  recipe_args: Optional[dict] = None, tensors: bool = True) -> Workload:
    recipe_args = recipe_args or {}
    H, D, d_c, d_r, d_v, W = (dims[k] for k in ("H", "D", "d_c", "d_r", "d_v", "W"))
    ss = np.random.SeedSequence(seed)
    s_lm, s_anchor, s_tensor = ss.spawn(3)
    rng_lm = np.random.Generator(np.random.PCG64(s_lm))
    rng_a = np.random.Generator(np.random.PCG64(s_anchor))
    rng_t = np.random.Generator(np.random.PCG64(s_tensor))

    lm = (rng_lm.random((B, S)) < 0.9).astype(np.uint8)
    anchors = keep = None
    source = "given"
    if recipe == "sampler":
        source = "sampler"
    else:
        anchors = np.empty((B, N), dtype=np.int32)
        keep = np.empty((B, N), dtype=np.uint8)
        for b in range(B):
            if recipe == "uniform":
                a, k = _recipe_uniform(rng_a, S, N, W, **recipe_args)
            elif recipe == "clustered":
                a, k = _recipe_clustered(rng_a, S, N, **recipe_args)
            elif recipe == "headline":
                a, k = _recipe_headline(rng_a, S, N, W, **recipe_args)
            else:
                raise ValueError(f"unknown anchor recipe {recipe!r}")
            anchors[b], keep[b] = a, k
            _force_valid(lm[b], a, k)
    lays = ([_make_layer(rng_t, B, S, N, H, D, d_c, d_r, d_v, dtype) for _ in range(layers)]
            if tensors else [])
    return Workload(name=name, B=B, S=S, N=N, W=W, H=H, D=D, d_c=d_c, d_r=d_r, d_v=d_v,
                    dtype=dtype, rope_base=rope_base,
                    loss_mask=lm, anchors=anchors, keep=keep, anchor_source=source,
                    sampler_seed=0x5EED0000 + (seed & 0xFFFF), layers=lays)


TINY_DIMS = dict(H=2, D=32, d_c=16, d_r=8, d_v=16, W=16)


def config(k: int, *, seed: Optional[int] = None, tensors: bool = True) -> Workload:
    """The five benchmark configurations at full size (1-based index).
    tensors=False skips the activations and weights (mask and anchors only)."""
    seed = 1000 + k if seed is None else seed
    if k == 1:
        return make_workload("tiny-fp32 B1 S48 N4 W16 H2", B=1, S=48, N=4, dims=TINY_DIMS,
                             dtype="f32", recipe="uniform", seed=seed, tensors=tensors,
                             recipe_args=dict(n_forced_low=1))
    if k == 2:
        return make_workload("glm-layer B1 S2048 N64", B=1, S=2048, N=64, dims=GLM_DIMS,
                             dtype="bf16", recipe="sampler", seed=seed, tensors=tensors)
    if k == 3:
        return make_workload("overlap B2 S8192 N512", B=2, S=8192, N=512, dims=GLM_DIMS,
                             dtype="bf16", recipe="clustered", seed=seed, tensors=tensors)
    if k == 4:
        return make_workload("headline B1 S32768 N1024", B=1, S=32768, N=1024, dims=GLM_DIMS,
                             dtype="bf16", recipe="headline", seed=seed, tensors=tensors)
    if k == 5:
        return make_workload("three-layer B1 S131072 N4096 L3", B=1, S=131072, N=4096,
                             dims=GLM_DIMS, dtype="bf16", recipe="sampler", seed=seed, tensors=tensors, layers=3)
    raise ValueError(k)


def scaled(k: int, *, S: int, N: int, B: Optional[int] = None, seed: Optional[int] = None,
           dims: Optional[dict] = None, dtype: Optional[str] = None) -> Workload:
    """A configuration's recipe at a smaller size (oracle-friendly parity cases)."""
    seed = 2000 + k if seed is None else seed
    dims = dims or (TINY_DIMS if k == 1 else GLM_DIMS)
    dtype = dtype or ("f32" if k == 1 else "bf16")
    recipe, args, Bd = {1: ("uniform", dict(n_forced_low=1), 1), 2: ("sampler", {}, 1),
                        3: ("clustered", {}, 2), 4: ("headline", {}, 1),
                        5: ("sampler", {}, 1)}[k]
    return make_workload(f"cfg{k}-scaled B{B or Bd} S{S} N{N}", B=B or Bd, S=S, N=N, dims=dims,
                         dtype=dtype, recipe=recipe, seed=seed, recipe_args=args,
                         layers=3 if k == 5 else 1)


def make_dout(wl: Workload, seed: int = 7) -> np.ndarray:
    """Upstream gradient of the attention output, [B, 5N, H, d_v], N(0, 1) in
    the workload's storage type (the input of a backward pass).  Drawn from
    its own seeded stream so that the forward inputs stay as they are."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.B, wl.S, wl.N])))
    return _normal(rng, (wl.B, wl.block * wl.N, wl.H, wl.d_v), 1.0, wl.dtype)


@dataclasses.dataclass
class LayerInputs:
    """Inputs of one draft layer's MLA block beyond the attention's own:
    the layer input H^(l) [B, 5N, d] (residual stream), H^ctx [B, S, d], the
    RMSNorm weights and the projections (out x in, like the page's
    parameter table)."""
    hidden: int
    q_rank: int
    rms_eps: float
    h_draft: np.ndarray     # [B, 5N, d]
    h_ctx: np.ndarray       # [B, S, d]
    g_in: np.ndarray        # [d]            input_layernorm
    w_qa: np.ndarray        # [q_rank, d]    q_a_proj
    g_qa: np.ndarray        # [q_rank]       q_a_layernorm
    w_qb: np.ndarray        # [H*(d_c+d_r), q_rank]  q_b_proj, per head d_c rows then d_r rows
    w_kva: np.ndarray       # [D + d_r, d]   kv_a_proj_with_mqa: c^KV rows then k^R rows
    g_kva: np.ndarray       # [D]            kv_a_layernorm
    w_o: np.ndarray         # [d, H*d_v]     o_proj


def make_layer_inputs(wl: Workload, hidden: int, q_rank: int, seed: int = 5,
                      rms_eps: float = 1e-6) -> LayerInputs:
    """Seeded inputs for the MLA block around the attention (same storage
    type as the workload): activations N(0, 1), RMSNorm weights 1 + N(0, 0.1^2),
    projection weights N(0, 1/fan_in).  The attention's W_UK / W_UV are the
    workload's own (kv_b_proj)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.B, wl.S, wl.N,
                                                                        hidden, q_rank])))
    dt = wl.dtype
    H, D, dc, dr, dv = wl.H, wl.D, wl.d_c, wl.d_r, wl.d_v

    def gain(n):
        x = 1.0 + 0.1 * rng.standard_normal(size=n, dtype=np.float32)
        return f32_to_bf16_bits(x) if dt == "bf16" else x.astype(np.float32)

    return LayerInputs(
        hidden=hidden, q_rank=q_rank, rms_eps=rms_eps,
        h_draft=_normal(rng, (wl.B, wl.block * wl.N, hidden), 1.0, dt),
        h_ctx=_normal(rng, (wl.B, wl.S, hidden), 1.0, dt),
        g_in=gain(hidden),
        w_qa=_normal(rng, (q_rank, hidden), float(1 / np.sqrt(hidden)), dt),
        g_qa=gain(q_rank),
        w_qb=_normal(rng, (H * (dc + dr), q_rank), float(1 / np.sqrt(q_rank)), dt),
        w_kva=_normal(rng, (D + dr, hidden), float(1 / np.sqrt(hidden)), dt),
        g_kva=gain(D),
        w_o=_normal(rng, (hidden, H * dv), float(1 / np.sqrt(H * dv)), dt),
    )


@dataclasses.dataclass
class LossInputs:
    """Inputs of the output head and loss (design page §5–§6) beyond the
    anchors, keep mask and loss mask of the workload: the token ids, the
    draft's final hidden states H^(L) [B, 5N, d], the Target's last hidden
    states z [B, S, d], the frozen lm_head [V, d], the Markov head
    (markov_w1 [V, r] as a lookup table, markov_w2 [V, r]) and the
    confidence head [d + r]."""
    vocab: int
    hidden: int
    rank: int
    dtype: str
    input_ids: np.ndarray   # [B, S] int32 in [0, V)
    h_final: np.ndarray     # [B, 5N, d]
    z: np.ndarray           # [B, S, d]
    w_lm: np.ndarray        # [V, d]
    w_m1: np.ndarray        # [V, r]
    w_m2: np.ndarray        # [V, r]
    w_conf: np.ndarray      # [d + r]


def make_loss_inputs(wl: Workload, vocab: int, hidden: int, rank: int = 256, seed: int = 9,
                     logit_std: float = 2.0, markov_std: float = 0.5) -> LossInputs:
    """Seeded inputs for the output head and loss, in the workload's storage
    type.  Token ids are uniform over the vocabulary.  Hidden rows are N(0, 1)
    times a per-row gain drawn uniformly from [0.1, 2], so that the draft and
    teacher distributions range from nearly flat to peaked and their L1
    distance spans (0, 2).  lm_head is N(0, logit_std^2 / d) (logits of
    standard deviation ~ logit_std x gain), markov_w1 N(0, 1), markov_w2
    N(0, markov_std^2 / r), the confidence head N(0, 1 / (d + r))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wl.B, wl.S, wl.N,
                                                                        vocab, hidden, rank])))
    dt = wl.dtype

    def rows(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= rng.uniform(0.1, 2.0, size=shape[:-1] + (1,)).astype(np.float32)
        return f32_to_bf16_bits(x) if dt == "bf16" else x

    ids = rng.integers(0, vocab, size=(wl.B, wl.S), dtype=np.int32)
    return LossInputs(
        vocab=vocab, hidden=hidden, rank=rank, dtype=dt, input_ids=ids,
        h_final=rows((wl.B, wl.block * wl.N, hidden)),
        z=rows((wl.B, wl.S, hidden)),
        w_lm=_normal(rng, (vocab, hidden), float(logit_std / np.sqrt(hidden)), dt),
        w_m1=_normal(rng, (vocab, rank), 1.0, dt),
        w_m2=_normal(rng, (vocab, rank), float(markov_std / np.sqrt(rank)), dt),
        w_conf=_normal(rng, (hidden + rank,), float(1 / np.sqrt(hidden + rank)), dt),
    )


@dataclasses.dataclass
class DecodeInputs:
    """One decode step's attention inputs for B sequences (one draft block
    each) and the most recent context rows of each sequence, to be written
    into the draft cache: ctx_ckv / ctx_kr [B, n_ctx, .] hold positions
    A - n_ctx .. A - 1 (rows at negative positions are unused)."""
    q_nope: np.ndarray    # [B, 5, H, d_c]
    q_rope: np.ndarray    # [B, 5, H, d_r]
    ckv_blk: np.ndarray   # [B, 5, D]
    kr_blk: np.ndarray    # [B, 5, d_r]
    w_uk: np.ndarray      # [H, d_c, D]
    w_uv: np.ndarray      # [H, d_v, D]
    ctx_ckv: np.ndarray   # [B, n_ctx, D]
    ctx_kr: np.ndarray    # [B, n_ctx, d_r]


def make_decode_inputs(B: int, dims: dict, dtype: str, n_ctx: int, seed: int = 13) -> DecodeInputs:
    """Activations N(0, 1), weights N(0, 1/D), as for a training layer."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, B, n_ctx])))
    H, D, d_c, d_r, d_v = (dims[k] for k in ("H", "D", "d_c", "d_r", "d_v"))
    wstd = float(1.0 / np.sqrt(D))
    return DecodeInputs(
        q_nope=_normal(rng, (B, BLOCK, H, d_c), 1.0, dtype),
        q_rope=_normal(rng, (B, BLOCK, H, d_r), 1.0, dtype),
        ckv_blk=_normal(rng, (B, BLOCK, D), 1.0, dtype),
        kr_blk=_normal(rng, (B, BLOCK, d_r), 1.0, dtype),
        w_uk=_normal(rng, (H, d_c, D), wstd, dtype),
        w_uv=_normal(rng, (H, d_v, D), wstd, dtype),
        ctx_ckv=_normal(rng, (B, n_ctx, D), 1.0, dtype),
        ctx_kr=_normal(rng, (B, n_ctx, d_r), 1.0, dtype),
    )


def make_verify_inputs(B: int, K: int, vocab: int, seed: int = 17, logit_std: float = 2.0,
                       noise_std: float = 0.7):
    """Draft logits [B, K, V] N(0, logit_std^2); target logits [B, K+1, V]:
    the draft's plus N(0, noise_std^2) for the first K rows (distributions
    that overlap partly), N(0, logit_std^2) for the last; uniforms [B, K+1]
    and [B, K] (the second set for drawing the drafted tokens) in [0, 1).
    All fp32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, B, K, vocab])))
    dl = rng.standard_normal((B, K, vocab), dtype=np.float32) * np.float32(logit_std)
    tl = np.empty((B, K + 1, vocab), dtype=np.float32)
    tl[:, :K] = dl + rng.standard_normal((B, K, vocab), dtype=np.float32) * np.float32(noise_std)
    tl[:, K] = rng.standard_normal((B, vocab), dtype=np.float32) * np.float32(logit_std)
    u = rng.random((B, K + 1), dtype=np.float32)
    u_draft = rng.random((B, K), dtype=np.float32)
    return dl, tl, u, u_draft
