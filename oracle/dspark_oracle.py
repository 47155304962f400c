"""fp64 oracle: the DSpark draft-attention forward as the design page defines it.

TEST INFRASTRUCTURE -- see the package docstring for who may import this.

Source: the GLM 5.2 DSpark training-design page ("GLM 5.2 DSpark 投机训练设计").
Sections cited below:
  * parameter summary (参数摘要): dims, SWA window W, block length 5;
  * §2 model inputs (模型输入): "Anchor sampling", "QKV construction";
  * §3 attention mask (注意力掩码): causal window, bidirectional block,
    padding block;
  * §4 MLA: "MLA Projection" (q^C/q^R, c^KV -> k^C, v; k^R), scale, "RoPE";
  * §6 training objective, "eval_mask" paragraph (loss_mask[S-1] := 0);
  * appendix A, option 2 (loss_mask[S-1] := 0 on read);
  * appendix "Attention implementation": the mask shape, the attention
    equation softmax(QK^T/sqrt(d) + Lambda(M)) V, and the dense eager/sdpa
    materialisation.

Readings where the page is silent or ambiguous (each also listed in the design
notes of the repository):
  * scale: the §4 value (d_c + d_r)^(-1/2), not the generic sqrt(d) of the
    appendix equation;
  * RoPE: base 10000, pair i = (2i, 2i+1) rotated counter-clockwise by
    p * base^(-2i/d_r) (interleaved adjacent pairs, §4 "RoPE");
  * weights: W_UK [H, d_c, D] and W_UV [H, d_v, D] (out x in), so that
    k^C_h = W_UK[h] c and v_h = W_UV[h] c;
  * padding rows have no defined output; this oracle returns NaN for them;
  * "pick N at random": the integer-only SplitMix64 partial Fisher-Yates
    spec in ``select_anchors``.

Everything is fp64.  bf16 inputs arrive as raw uint16 bit patterns and are
decoded exactly.

``backward`` returns the gradients of the same forward (chain rule on the
expanded form); it is pinned by central finite differences of ``loss``, by
closed forms and by torch's autograd of its masked SDPA in a special case.
"""
from __future__ import annotations

import numpy as np

BLOCK = 5
MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64: a bf16 value is the top 16 bits of an fp32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# anchors  (§2 "Anchor sampling"; §6 "eval_mask"; appendix A option 2)
# ---------------------------------------------------------------------------

def candidates(loss_mask_row: np.ndarray) -> np.ndarray:
    """Valid anchor positions, ascending.

    §2: A is a candidate iff A in [0, S-2], loss_mask[A] = 1 and
    loss_mask[A+1] = 1.  §6 / appendix A: on read, loss_mask[S-1] is set to 0
    (so x_{S-1} is neither an anchor nor a label).
    """
    lm = np.array(loss_mask_row, dtype=np.int64, copy=True)
    S = lm.shape[0]
    lm[S - 1] = 0
    out = []
    for a in range(0, S - 1):           # A in [0, S-2]
        if lm[a] == 1 and lm[a + 1] == 1:
            out.append(a)
    return np.array(out, dtype=np.int64)


class SplitMix64:
    """SplitMix64 (Steele, Lea & Flood, OOPSLA 2014; Vigna's splitmix64.c):
    the state advances by the golden-ratio increment 0x9E3779B97F4A7C15 and
    each output is the state passed through the variant-13 xor-shift-multiply
    finaliser (shifts 30, 27, 31; multipliers 0xBF58476D1CE4E5B9,
    0x94D049BB133111EB)."""

    def __init__(self, seed: int):
        self.state = seed & MASK64

    def next(self) -> int:
        self.state = (self.state + 0x9E3779B97F4A7C15) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)


def select_anchors(loss_mask_row: np.ndarray, num_anchors: int, seed: int):
    """§2 "Anchor sampling": draw N of the valid positions at random, N <=
    num_anchors; padding blocks fill the batch when fewer are valid (§3
    "Padding block").

    The page fixes neither the generator nor the draw, so this is the spec:
      C = candidates(loss_mask)
      |C| <= N : anchors = C then (N-|C|) padding slots (A = 0, keep = 0)
      |C| >  N : partial Fisher-Yates over C with SplitMix64(seed):
                 for i in 0..N-1: j = i + next() mod (|C| - i); swap C[i], C[j]
                 anchors = sorted(C[0:N]); keep = 1
    Returns (anchors int32 [N], keep uint8 [N]).
    """
    C = [int(c) for c in candidates(loss_mask_row)]
    N = int(num_anchors)
    anchors = np.zeros(N, dtype=np.int32)
    keep = np.zeros(N, dtype=np.uint8)
    if len(C) <= N:
        anchors[: len(C)] = C
        keep[: len(C)] = 1
        return anchors, keep
    rng = SplitMix64(seed)
    for i in range(N):
        j = i + rng.next() % (len(C) - i)
        C[i], C[j] = C[j], C[i]
    anchors[:] = sorted(C[:N])
    keep[:] = 1
    return anchors, keep


# ---------------------------------------------------------------------------
# KV axis, positions and mask  (§2 "QKV construction"; §3; appendix)
# ---------------------------------------------------------------------------

def positions(S: int, anchors_row: np.ndarray, block: int = BLOCK):
    """§2 "QKV construction" and §4 "RoPE": the KV axis is [S context ; N
    blocks of 5]; context positions are 0..S-1, block n has A_n..A_n+4; the
    queries use the second part of the axis."""
    pos_kv = list(range(S))
    for a in np.asarray(anchors_row).tolist():
        pos_kv.extend(int(a) + j for j in range(block))
    pos_kv = np.array(pos_kv, dtype=np.int64)
    return pos_kv, pos_kv[S:]


def mask_rows(S: int, N: int, W: int, anchors_row, keep_row, n: int, block: int = BLOCK):
    """The `block` rows of M belonging to block n, whole rows of length S+5N.

    §3: for kv < S, row q of a kept block sees A-W+1 <= kv < A (the same
    window for all 5 queries, not shifted with the offset; A itself excluded);
    for kv >= S it sees only its own block's 5 positions (bidirectional).
    A padding block (keep = 0) sees nothing.  The anchor of a padding block
    is never read.
    """
    L = S + block * N
    rows = np.zeros((block, L), dtype=bool)
    if not keep_row[n]:
        return rows
    A = int(anchors_row[n])
    kv = np.arange(L, dtype=np.int64)
    for j in range(block):          # every query of the block, evaluated on its own
        ctx_part = (kv < S) & (A - W + 1 <= kv) & (kv < A)
        draft_part = (kv >= S) & ((kv - S) // block == n)
        rows[j] = ctx_part | draft_part
    return rows


def build_mask(S: int, N: int, W: int, anchors_row, keep_row, block: int = BLOCK) -> np.ndarray:
    """Dense boolean M in {0,1}^{5N x (S+5N)} for one sample (appendix
    "Attention implementation": the eager/sdpa backend materialises exactly
    this tensor, broadcast over heads)."""
    return np.concatenate([mask_rows(S, N, W, anchors_row, keep_row, n, block)
                           for n in range(N)], axis=0)


def row_index_sets(M: np.ndarray, S: int):
    """Per row: (visible context columns, visible draft columns) as sorted
    int arrays, read off the materialised mask."""
    out = []
    for r in range(M.shape[0]):
        nz = np.nonzero(M[r])[0]
        out.append((nz[nz < S], nz[nz >= S]))
    return out


def block_index_records(S: int, N: int, W: int, anchors_row, keep_row, block: int = BLOCK,
                        ns=None):
    """Per block: (ctx_lo, ctx_len, pos0, keep) read off the block's mask rows:
    ctx_lo/ctx_len describe the visible context columns (which §3 makes a
    contiguous run), pos0 is the RoPE position of the block's first query.
    A padding block reports (0, 0, 0, 0).  ns: the blocks to fill (default
    all); the other rows stay 0."""
    recs = np.zeros((N, 4), dtype=np.int64)
    for n in (range(N) if ns is None else ns):
        if not keep_row[n]:
            continue
        rows = mask_rows(S, N, W, anchors_row, keep_row, n, block)
        ctx = np.nonzero(rows[0, :S])[0]
        lo = int(ctx[0]) if len(ctx) else int(anchors_row[n])
        recs[n] = (lo, len(ctx), int(anchors_row[n]), 1)
    return recs


# ---------------------------------------------------------------------------
# RoPE  (§4 "RoPE")
# ---------------------------------------------------------------------------

def rope_theta(d_r: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_r) for pair i = 0 .. d_r/2-1."""
    i = np.arange(d_r // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d_r)


def rope_interleaved(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate the d_r-wide rope slice by position, interleaved adjacent pairs
    (GLM rope_interleave = true): (x_{2i}, x_{2i+1}) ->
    (x_{2i} cos phi - x_{2i+1} sin phi, x_{2i} sin phi + x_{2i+1} cos phi),
    phi = pos * theta_i.  x has shape [..., T, d_r] (any leading dims are
    broadcast), pos has shape [T]."""
    x = np.asarray(x, dtype=np.float64)
    d_r = x.shape[-1]
    phi = np.asarray(pos, dtype=np.float64)[:, None] * rope_theta(d_r, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# ---------------------------------------------------------------------------
# expanded MLA per head  (§4 "MLA Projection")
# ---------------------------------------------------------------------------

def expand_head(ckv_all: np.ndarray, kr_rot_all: np.ndarray, w_uk: np.ndarray,
                w_uv: np.ndarray, h: int):
    """§4: c^KV expands through kv_b_proj into per-head k^C (d_c) and v (d_v);
    k^R is not expanded, it is rotated and copied to every head and
    concatenated: K_h = [k^C_h ; k^R] (d_c + d_r), V_h = v_h (d_v).
    Each key is a function of exactly its 576 = 512 + 64 cached numbers
    (parameter summary, "KV cache")."""
    Kc = ckv_all @ w_uk[h].T            # [L, d_c]
    K = np.concatenate([Kc, kr_rot_all], axis=1)
    V = ckv_all @ w_uv[h].T             # [L, d_v]
    return K, V


# ---------------------------------------------------------------------------
# attention  (appendix "Attention implementation"; §4 scale)
# ---------------------------------------------------------------------------

def softmax_scale(d_c: int, d_r: int) -> float:
    """§4: the attention scale is (d_c + d_r)^(-1/2) (1/16 for the GLM dims)."""
    return float(d_c + d_r) ** -0.5


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    m = np.max(logits, axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_dense(Q: np.ndarray, K: np.ndarray, V: np.ndarray, M: np.ndarray,
                 scale: float) -> np.ndarray:
    """Literal form: softmax(scale * Q K^T + Lambda(M)) V with Lambda = 0
    where M = 1 and -inf where M = 0.  Rows with no visible key (padding
    rows) have no defined value and come back as NaN."""
    logits = scale * (Q @ K.T)
    logits = np.where(M, logits, -np.inf)
    out = np.full((Q.shape[0], V.shape[1]), np.nan)
    live = M.any(axis=1)
    if live.any():
        out[live] = _softmax_rows(logits[live]) @ V
    return out


def attend_gathered(Q: np.ndarray, K: np.ndarray, V: np.ndarray, M: np.ndarray,
                    scale: float) -> np.ndarray:
    """Each row restricted to its visible columns {kv : M = 1}; identical to
    the literal form because exp(-inf) = 0."""
    out = np.full((Q.shape[0], V.shape[1]), np.nan)
    for r in range(Q.shape[0]):
        cols = np.nonzero(M[r])[0]
        if len(cols) == 0:
            continue
        w = _softmax_rows((scale * (K[cols] @ Q[r]))[None, :])[0]
        out[r] = w @ V[cols]
    return out


def _layer_f64(wl, layer):
    dt = wl.dtype
    return {name: _f64(getattr(layer, name), dt) for name in
            ("q_nope", "q_rope", "ckv_ctx", "kr_ctx", "ckv_blk", "kr_blk", "w_uk", "w_uv")}


def forward(wl, layer_idx: int = 0, anchors=None, keep=None, form: str = "dense",
            blocks=None, scale=None):
    """Reference output [B, 5N, H, d_v] (fp64; padding rows are NaN).

    wl: a ``workloads.Workload``.  anchors/keep default to the workload's.
    form: "dense" (literal masked softmax over the whole KV axis) or
    "gathered" (visible columns only).
    blocks: None for every block; otherwise a list of (b, n) pairs -- then
    only those blocks' rows are computed (their mask rows are still whole
    rows of length S+5N) and the keys are expanded only at the columns those
    rows see; every other row is NaN.
    scale: None for the §4 value; a float overrides it.
    """
    scale = softmax_scale(wl.d_c, wl.d_r) if scale is None else float(scale)
    anchors = wl.anchors if anchors is None else anchors
    keep = wl.keep if keep is None else keep
    B, S, N, W, H, bl = wl.B, wl.S, wl.N, wl.W, wl.H, wl.block
    x = _layer_f64(wl, wl.layers[layer_idx])
    out = np.full((B, bl * N, H, wl.d_v), np.nan)
    by_sample = {}
    if blocks is not None:
        for (b, n) in blocks:
            by_sample.setdefault(int(b), []).append(int(n))
    for b in range(B):
        if blocks is not None and b not in by_sample:
            continue
        pos_kv, pos_q = positions(S, anchors[b], bl)
        ckv_all = np.concatenate([x["ckv_ctx"][b], x["ckv_blk"][b]], axis=0)
        kr_rot = rope_interleaved(np.concatenate([x["kr_ctx"][b], x["kr_blk"][b]], axis=0),
                                  pos_kv, wl.rope_base)
        qr_rot = rope_interleaved(x["q_rope"][b].transpose(1, 0, 2), pos_q, wl.rope_base)
        if blocks is None:
            M = build_mask(S, N, W, anchors[b], keep[b], bl)
            rows = np.arange(bl * N)
        else:
            ns = sorted(set(by_sample[b]))
            M = np.concatenate([mask_rows(S, N, W, anchors[b], keep[b], n, bl) for n in ns], 0)
            rows = np.array([bl * n + j for n in ns for j in range(bl)])
            cols = np.nonzero(M.any(axis=0))[0]
            # only the visible columns are ever weighted; restrict the axis
            ckv_all, kr_rot, M = ckv_all[cols], kr_rot[cols], M[:, cols]
        for h in range(H):
            K, V = expand_head(ckv_all, kr_rot, x["w_uk"], x["w_uv"], h)
            Q = np.concatenate([x["q_nope"][b][rows, h, :], qr_rot[h][rows]], axis=1)
            if form == "dense":
                o = attend_dense(Q, K, V, M, scale)
            elif form == "gathered":
                o = attend_gathered(Q, K, V, M, scale)
            else:
                raise ValueError(form)
            out[b, rows, h, :] = o
    return out


def forward_absorbed(wl, layer_idx: int = 0, anchors=None, keep=None, scale=None):
    """The same forward computed in the absorbed latent form (used only to
    pin the identity the GPU path relies on):
      q_abs = W_UK[h]^T q^C,  score = scale * (q_abs . c^KV + q^R . k^R),
      o_lat = sum_k p_k c^KV_k,  out = W_UV[h] o_lat.
    Per-row loop over blocks, plain numpy."""
    scale = softmax_scale(wl.d_c, wl.d_r) if scale is None else float(scale)
    anchors = wl.anchors if anchors is None else anchors
    keep = wl.keep if keep is None else keep
    B, S, N, W, H, bl = wl.B, wl.S, wl.N, wl.W, wl.H, wl.block
    x = _layer_f64(wl, wl.layers[layer_idx])
    out = np.full((B, bl * N, H, wl.d_v), np.nan)
    for b in range(B):
        pos_kv, pos_q = positions(S, anchors[b], bl)
        ckv_all = np.concatenate([x["ckv_ctx"][b], x["ckv_blk"][b]], axis=0)
        kr_rot = rope_interleaved(np.concatenate([x["kr_ctx"][b], x["kr_blk"][b]], axis=0),
                                  pos_kv, wl.rope_base)
        qr_rot = rope_interleaved(x["q_rope"][b].transpose(1, 0, 2), pos_q, wl.rope_base)
        M = build_mask(S, N, W, anchors[b], keep[b], bl)
        for r in range(bl * N):
            cols = np.nonzero(M[r])[0]
            if len(cols) == 0:
                continue
            for h in range(H):
                q_abs = x["w_uk"][h].T @ x["q_nope"][b][r, h]
                s = scale * (ckv_all[cols] @ q_abs + kr_rot[cols] @ qr_rot[h][r])
                p = _softmax_rows(s[None, :])[0]
                o_lat = p @ ckv_all[cols]
                out[b, r, h] = x["w_uv"][h] @ o_lat
    return out


# ---------------------------------------------------------------------------
# backward  (gradient of the same masked attention; chain rule on the
# expanded form of §4 "MLA Projection" and the appendix equation)
# ---------------------------------------------------------------------------

def rope_interleaved_transpose(y: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """R(pos)^T y: the adjoint of ``rope_interleaved`` (rotation by -phi), which
    carries a gradient w.r.t. rotated vectors back to the unrotated ones."""
    y = np.asarray(y, dtype=np.float64)
    d_r = y.shape[-1]
    phi = np.asarray(pos, dtype=np.float64)[:, None] * rope_theta(d_r, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    y0, y1 = y[..., 0::2], y[..., 1::2]
    x = np.empty_like(y)
    x[..., 0::2] = y0 * c + y1 * s
    x[..., 1::2] = -y0 * s + y1 * c
    return x


def backward(wl, dout, layer_idx: int = 0, anchors=None, keep=None, form: str = "dense",
             blocks=None, scale=None):
    """Gradients of L = sum over kept rows of <dout, out> w.r.t. every input
    of the forward (fp64).

    The forward is softmax(scale * Q_h K_h^T + Lambda(M)) V_h per head with
    K_h = [c^KV W_UK[h]^T ; R k^R], V_h = c^KV W_UV[h]^T and
    Q_h = [q^C_h ; R q^R_h] (§4 "MLA Projection", appendix equation).  With
    G = dout (rows of padding blocks have no defined output and carry no
    gradient), the chain rule gives, per head:
      dV = P^T G,  dP = G V^T,  dS = P * (dP - rowsum(P * dP)),
      dQ = scale dS K,  dK = scale dS^T Q,
      dc^KV += dK[:, :d_c] W_UK[h] + dV W_UV[h],
      dW_UK[h] += dK[:, :d_c]^T c^KV,  dW_UV[h] += dV^T c^KV,
      d(R k^R) += dK[:, d_c:],  dq^C_h = dQ[:, :d_c],  d(R q^R_h) = dQ[:, d_c:],
    and the rotations are undone with R^T.

    dout: [B, 5N, H, d_v] in the workload's storage (bf16 bits or float).
    form: "dense" (the whole KV axis) or "gathered" (only the columns some
    computed row sees; identical because masked entries have P = 0).
    blocks: None for every block, else the (b, n) pairs whose rows carry
    gradient (the others are taken as dout = 0).
    Returns a dict of fp64 arrays named like the inputs with a "d" prefix.
    """
    scale = softmax_scale(wl.d_c, wl.d_r) if scale is None else float(scale)
    anchors = wl.anchors if anchors is None else anchors
    keep = wl.keep if keep is None else keep
    B, S, N, W, H, bl = wl.B, wl.S, wl.N, wl.W, wl.H, wl.block
    D, d_c, d_r, d_v = wl.D, wl.d_c, wl.d_r, wl.d_v
    x = _layer_f64(wl, wl.layers[layer_idx])
    G_all = _f64(dout, wl.dtype)
    L5 = bl * N
    g = {"dq_nope": np.zeros((B, L5, H, d_c)), "dq_rope": np.zeros((B, L5, H, d_r)),
         "dckv_ctx": np.zeros((B, S, D)), "dkr_ctx": np.zeros((B, S, d_r)),
         "dckv_blk": np.zeros((B, L5, D)), "dkr_blk": np.zeros((B, L5, d_r)),
         "dw_uk": np.zeros((H, d_c, D)), "dw_uv": np.zeros((H, d_v, D))}
    by_sample = {}
    if blocks is not None:
        for (b, n) in blocks:
            by_sample.setdefault(int(b), set()).add(int(n))
    for b in range(B):
        ns = sorted(by_sample.get(b, ())) if blocks is not None else list(range(N))
        ns = [n for n in ns if keep[b][n]]
        if not ns:
            continue
        pos_kv, pos_q = positions(S, anchors[b], bl)
        ckv_all = np.concatenate([x["ckv_ctx"][b], x["ckv_blk"][b]], axis=0)
        kr_rot = rope_interleaved(np.concatenate([x["kr_ctx"][b], x["kr_blk"][b]], axis=0),
                                  pos_kv, wl.rope_base)
        qr_rot = rope_interleaved(x["q_rope"][b].transpose(1, 0, 2), pos_q, wl.rope_base)
        M = np.concatenate([mask_rows(S, N, W, anchors[b], keep[b], n, bl) for n in ns], 0)
        rows = np.array([bl * n + j for n in ns for j in range(bl)])
        if form == "dense":
            cols = np.arange(S + L5)
        elif form == "gathered":
            cols = np.nonzero(M.any(axis=0))[0]
        else:
            raise ValueError(form)
        Mc, C, KR = M[:, cols], ckv_all[cols], kr_rot[cols]
        dC = np.zeros_like(C)
        dKR = np.zeros_like(KR)
        dqr_rot = np.zeros((H, L5, d_r))
        for h in range(H):
            Kc = C @ x["w_uk"][h].T
            K = np.concatenate([Kc, KR], axis=1)
            V = C @ x["w_uv"][h].T
            Q = np.concatenate([x["q_nope"][b][rows, h, :], qr_rot[h][rows]], axis=1)
            logits = np.where(Mc, scale * (Q @ K.T), -np.inf)
            P = np.zeros_like(logits)
            live = Mc.any(axis=1)
            P[live] = _softmax_rows(logits[live])
            Gh = G_all[b][rows, h, :]
            dV = P.T @ Gh
            dP = Gh @ V.T
            dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
            dQ = scale * (dS @ K)
            dK = scale * (dS.T @ Q)
            dKc = dK[:, :d_c]
            dC += dKc @ x["w_uk"][h] + dV @ x["w_uv"][h]
            g["dw_uk"][h] += dKc.T @ C
            g["dw_uv"][h] += dV.T @ C
            dKR += dK[:, d_c:]
            g["dq_nope"][b][rows, h, :] = dQ[:, :d_c]
            dqr_rot[h][rows] = dQ[:, d_c:]
        g["dq_rope"][b][rows] = rope_interleaved_transpose(dqr_rot[:, rows], pos_q[rows],
                                                           wl.rope_base).transpose(1, 0, 2)
        dkr_un = rope_interleaved_transpose(dKR, pos_kv[cols], wl.rope_base)
        ctx = cols < S
        g["dckv_ctx"][b][cols[ctx]] += dC[ctx]
        g["dkr_ctx"][b][cols[ctx]] += dkr_un[ctx]
        g["dckv_blk"][b][cols[~ctx] - S] += dC[~ctx]
        g["dkr_blk"][b][cols[~ctx] - S] += dkr_un[~ctx]
    return g


def loss(wl, dout, layer_idx: int = 0, anchors=None, keep=None, scale=None) -> float:
    """L = sum over kept rows of <dout, out>: the scalar whose gradient
    ``backward`` returns (used to pin it by finite differences)."""
    keep = wl.keep if keep is None else keep
    out = forward(wl, layer_idx, anchors, keep, form="dense", scale=scale)
    G = _f64(dout, wl.dtype)
    rows_kept = np.repeat(np.asarray(keep, dtype=bool), wl.block, axis=1)   # [B, 5N]
    return float(np.sum(np.where(rows_kept[:, :, None, None], out * G, 0.0)))


# ---------------------------------------------------------------------------
# the MLA block of one draft layer  (§4 "MLA Projection": input_layernorm,
# q_a_proj, q_a_layernorm, q_b_proj, kv_a_proj_with_mqa over [H^ctx ; h],
# kv_a_layernorm, the attention, o_proj added back to the residual)
# ---------------------------------------------------------------------------

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.  The page
    names the op (input_layernorm, q_a_layernorm, kv_a_layernorm) without a
    formula or epsilon; this is the standard definition with eps a
    parameter."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def layer_forward(wl, li, anchors=None, keep=None, scale=None, blocks=None):
    """H^(l) + o_proj(attention) for one draft layer (fp64), in the page's
    order (§4 "MLA Projection"):
      h    = RMSNorm(H^(l))                               input_layernorm
      c^Q  = RMSNorm(h W_qa^T)                            q_a_proj, q_a_layernorm
      [q^C ; q^R] per head = c^Q W_qb^T                   q_b_proj (n_h groups of (d_c, d_r))
      [c^KV ; k^R] = [H^ctx ; h] W_kva^T                  kv_a_proj_with_mqa
      c^KV <- RMSNorm(c^KV)                               kv_a_layernorm
      o    = attention(q, c^KV, k^R; W_UK, W_UV)          the forward above
      out  = H^(l) + o W_o^T                              o_proj, residual
    Rows of padding blocks have no attention output; they are NaN here.
    li: a ``workloads.LayerInputs``; W_UK / W_UV come from wl.layers[0].
    blocks: as in ``forward`` (only those blocks' rows are computed)."""
    import copy as _copy
    dt = wl.dtype
    B, S, N, H = wl.B, wl.S, wl.N, wl.H
    D, dc, dr, dv = wl.D, wl.d_c, wl.d_r, wl.d_v
    L5 = wl.block * N
    f = lambda a: _f64(a, dt)
    Hd, Hc = f(li.h_draft), f(li.h_ctx)
    # the rows the result needs: with `blocks`, only those blocks' draft rows
    # and the context rows of their windows are projected (the projections
    # are row-wise); the other rows stay 0 and are never read
    qrows = np.ones((B, L5), dtype=bool)
    crows = np.ones((B, S), dtype=bool)
    if blocks is not None:
        an = wl.anchors if anchors is None else anchors
        qrows[:] = False
        crows[:] = False
        for b, n in blocks:
            qrows[b, wl.block * n:wl.block * (n + 1)] = True
            A = int(an[b, n])
            if 0 <= A <= S - 2:
                crows[b, max(0, A - wl.W + 1):A] = True
    h = np.zeros_like(Hd)
    h[qrows] = rmsnorm(Hd[qrows], f(li.g_in), li.rms_eps)
    q = np.zeros((B, L5, H * (dc + dr)))
    cq = rmsnorm(h[qrows] @ f(li.w_qa).T, f(li.g_qa), li.rms_eps)
    q[qrows] = cq @ f(li.w_qb).T
    q = q.reshape(B, L5, H, dc + dr)
    kv_ctx = np.zeros((B, S, D + dr))
    kv_ctx[crows] = Hc[crows] @ f(li.w_kva).T
    kv_blk = np.zeros((B, L5, D + dr))
    kv_blk[qrows] = h[qrows] @ f(li.w_kva).T
    sub = _copy.copy(wl)
    sub.dtype = "f64"
    base = wl.layers[0]
    sub.layers = [type(base)(
        q_nope=q[..., :dc], q_rope=q[..., dc:],
        ckv_ctx=rmsnorm(kv_ctx[..., :D], f(li.g_kva), li.rms_eps), kr_ctx=kv_ctx[..., D:],
        ckv_blk=rmsnorm(kv_blk[..., :D], f(li.g_kva), li.rms_eps), kr_blk=kv_blk[..., D:],
        w_uk=f(base.w_uk), w_uv=f(base.w_uv))]
    o = forward(sub, 0, anchors, keep, form="gathered", blocks=blocks, scale=scale)
    out = np.full((B, L5, Hd.shape[-1]), np.nan)
    o2 = o.reshape(B, L5, H * dv)
    out[qrows] = Hd[qrows] + o2[qrows] @ f(li.w_o).T
    return out


# ---------------------------------------------------------------------------
# the output head and the training objective  (§5 "输出头": LM head, Markov
# head, confidence head; §6 "训练目标": labels, alignment, eval_mask, CE, L1,
# confidence BCE)
# ---------------------------------------------------------------------------

LOSS_ALPHAS = dict(ce=1.0, l1=0.9, conf=1.0)   # §6: dspark_*_alpha of the original recipe


def eval_mask(loss_mask, anchors, keep, block: int = BLOCK) -> np.ndarray:
    """§6 "eval_mask": step k of block n counts when A + k + 1 < S,
    loss_mask[A + k + 1] = 1 and the block is kept, with a prefix cumprod along
    the block (once a step is off, the later steps are off).  loss_mask[S-1] is
    set to 0 on read.  A kept block whose anchor lies outside [0, S-2] counts
    no step (its terms are NaN in ``loss_head``).  Returns [B, N, block] uint8."""
    lm = np.array(loss_mask, dtype=bool, copy=True)
    B, S = lm.shape
    lm[:, S - 1] = False
    N = np.asarray(anchors).shape[1]
    m = np.zeros((B, N, block), dtype=np.uint8)
    for b in range(B):
        for n in range(N):
            A = int(anchors[b, n])
            if not keep[b, n] or A < 0 or A > S - 2:
                continue
            on = True
            for k in range(block):
                p = A + k + 1
                on = on and p < S and bool(lm[b, p])
                m[b, n, k] = on
    return m


def draft_logits(h_rows, prev_ids, w_lm, w_m1, w_m2) -> np.ndarray:
    """§5: L = L^base + B(prev) for draft rows.  L^base = H^(L) W_lm^T (the
    frozen Target lm_head, [V, d]); B(prev) = markov_w1[prev] markov_w2^T: the
    Markov head embeds each position's predecessor token (the anchor at step 0,
    the gold token x_{A+k} at step k) into r dims with markov_w1 ([V, r], a
    lookup table) and maps it back to the vocabulary with markov_w2 ([V, r], no
    bias).  B does not read H^(L)."""
    e = np.asarray(w_m1, np.float64)[np.asarray(prev_ids)]
    return np.asarray(h_rows, np.float64) @ np.asarray(w_lm, np.float64).T \
        + e @ np.asarray(w_m2, np.float64).T


def teacher_logits(z_rows, w_lm) -> np.ndarray:
    """§6 "Alignment": T_k = lm_head(z_{A+k}) with the same frozen matrix."""
    return np.asarray(z_rows, np.float64) @ np.asarray(w_lm, np.float64).T


def confidence_logit(h_rows, prev_ids, w_m1, w_conf) -> np.ndarray:
    """§5 "Confidence head": a bias-free linear layer over the concatenation of
    H^(L) and the Markov embedding of prev (width d + r): one scalar per draft
    position.  w_conf is [d + r] (the H^(L) part first)."""
    e = np.asarray(w_m1, np.float64)[np.asarray(prev_ids)]
    x = np.concatenate([np.asarray(h_rows, np.float64), e], axis=-1)
    return x @ np.asarray(w_conf, np.float64)


def step_terms(L, T, y, c):
    """§6 per-step terms for rows of logits L (draft) and T (teacher), labels
    y and confidence logits c:
      ce  = -log softmax(L)[y]                      (CE against y_k)
      l1  = || softmax(L) - softmax(T) ||_1         (L1)
      a   = clip(1 - l1 / 2, 0, 1)                  (confidence target)
      bce = -(a log sigmoid(c) + (1 - a) log(1 - sigmoid(c)))   (BCE with logits)
    Returns (ce, l1, a, bce), each [rows]."""
    L = np.asarray(L, np.float64)
    T = np.asarray(T, np.float64)
    p = _softmax_rows(L)
    q = _softmax_rows(T)
    ce = -np.log(p[np.arange(L.shape[0]), np.asarray(y)])
    l1 = np.abs(p - q).sum(axis=1)
    a = np.clip(1.0 - 0.5 * l1, 0.0, 1.0)
    c = np.asarray(c, np.float64)
    log_sig = -np.logaddexp(0.0, -c)          # log sigmoid(c)
    log_1m = -np.logaddexp(0.0, c)            # log (1 - sigmoid(c))
    bce = -(a * log_sig + (1.0 - a) * log_1m)
    return ce, l1, a, bce


def loss_head(lh, loss_mask, anchors, keep, alphas=None, blocks=None):
    """The output head and the loss of §5–§6 for one batch (fp64).

    lh: a ``workloads.LossInputs`` (input_ids [B, S], H^(L) [B, 5N, d],
    z [B, S, d], w_lm [V, d], markov_w1 / markov_w2 [V, r], w_conf [d + r]).
    For step k of a kept block with anchor A: prev = x_{A+k}, label
    y_k = x_{A+k+1}, draft logits L_k from row 5n + k of H^(L), teacher logits
    T_k from z_{A+k}.  Per-step outputs (``ce``, ``l1``, ``conf`` -- the
    confidence logit -- and ``bce``, [B, N, 5]) are 0 where the eval mask is
    0 and NaN for every step of a kept block whose anchor lies outside
    [0, S-2].  The three terms are summed over the steps the eval mask keeps
    and divided by their count (0 when no step counts); ``total`` is
    alpha_ce ce + alpha_l1 l1 + alpha_conf bce (§6: 1, 0.9, 1).
    blocks: optional list of (b, n) -- only those blocks' steps are computed
    (the others are left 0); the means are then not formed (NaN)."""
    al = dict(LOSS_ALPHAS, **(alphas or {}))
    dt = lh.dtype
    f = lambda a: _f64(a, dt)
    ids = np.asarray(lh.input_ids)
    B, S = ids.shape
    N = np.asarray(anchors).shape[1]
    blk = BLOCK
    m = eval_mask(loss_mask, anchors, keep, blk)
    out = {k: np.zeros((B, N, blk)) for k in ("ce", "l1", "conf", "bce")}
    Hf, Z = f(lh.h_final), f(lh.z)
    w_lm, w1, w2, wc = f(lh.w_lm), f(lh.w_m1), f(lh.w_m2), f(lh.w_conf)
    todo = blocks if blocks is not None else [(b, n) for b in range(B) for n in range(N)]
    for b, n in todo:
        if not keep[b, n]:
            continue
        A = int(anchors[b, n])
        if A < 0 or A > S - 2:
            for k in out:
                out[k][b, n, :] = np.nan
            continue
        ks = [k for k in range(blk) if m[b, n, k]]
        if not ks:
            continue
        ks = np.array(ks)
        prev = ids[b, A + ks]
        rows = Hf[b, blk * n + ks]
        L = draft_logits(rows, prev, w_lm, w1, w2)
        T = teacher_logits(Z[b, A + ks], w_lm)
        c = confidence_logit(rows, prev, w1, wc)
        ce, l1, _, bce = step_terms(L, T, ids[b, A + ks + 1], c)
        out["ce"][b, n, ks], out["l1"][b, n, ks] = ce, l1
        out["conf"][b, n, ks], out["bce"][b, n, ks] = c, bce
    out["eval_mask"] = m
    cnt = int(m.sum())
    out["count"] = cnt
    if blocks is not None:
        means = {k: np.nan for k in ("ce", "l1", "bce")}
    else:
        means = {k: (float(out[k].sum() / cnt) if cnt else 0.0) for k in ("ce", "l1", "bce")}
        bad = any(np.isnan(out[k]).any() for k in ("ce", "l1", "bce"))
        if bad:
            means = {k: np.nan for k in means}
    out["mean_ce"], out["mean_l1"], out["mean_bce"] = means["ce"], means["l1"], means["bce"]
    out["total"] = al["ce"] * means["ce"] + al["l1"] * means["l1"] + al["conf"] * means["bce"]
    return out


# ---------------------------------------------------------------------------
# inference-time drafting: the windowed draft KV cache (parameter summary,
# "KV cache": a draft layer keeps about W cached tokens, 576 numbers each)
# and draft-then-verify with rejection sampling (the MTP / DSA explainer
# page's "Rejection Sampling" passage: acceptance sum_v min(p_v, q_v))
# ---------------------------------------------------------------------------

def ring_slot(pos, slots: int):
    """Slot of logical position pos in a draft cache of `slots` entries: the
    cache keeps the most recent positions, position p in slot p mod slots."""
    return np.asarray(pos) % slots


def decode_attention(cache_ckv, cache_kr, anchors, active, q_nope, q_rope, ckv_blk, kr_blk,
                     w_uk, w_uv, W: int, rope_base: float, dtype: str, scale=None):
    """The draft's attention for one block per sequence at decode time (fp64):
    the block [x_A, MASK x 4] sits at positions A..A+4 and sees, as in §3, the
    context positions [max(0, A-W+1), A) -- read from the ring cache at slot
    p mod C -- and its own 5 positions bidirectionally.  Keys, values and
    queries as in §4 "MLA Projection" and "RoPE", with the true positions.
    cache_ckv [B, C, D], cache_kr [B, C, d_r]; anchors [B]; active [B]
    (inactive sequences give NaN rows); q_nope [B, 5, H, d_c], q_rope
    [B, 5, H, d_r] (not rotated); ckv_blk [B, 5, D], kr_blk [B, 5, d_r].
    Returns [B, 5, H, d_v]."""
    f = lambda a: _f64(a, dtype)
    cc, ck, qn, qr = f(cache_ckv), f(cache_kr), f(q_nope), f(q_rope)
    cb, kb, wk, wv = f(ckv_blk), f(kr_blk), f(w_uk), f(w_uv)
    B, C = cc.shape[0], cc.shape[1]
    H, dc, dr, dv = qn.shape[2], qn.shape[3], qr.shape[3], wv.shape[1]
    scale = softmax_scale(dc, dr) if scale is None else float(scale)
    out = np.full((B, BLOCK, H, dv), np.nan)
    for b in range(B):
        if not active[b]:
            continue
        A = int(anchors[b])
        ctx = np.arange(max(0, A - W + 1), A)
        blk = A + np.arange(BLOCK)
        slots = ring_slot(ctx, C)
        ckv = np.concatenate([cc[b][slots], cb[b]], axis=0)
        kr = rope_interleaved(np.concatenate([ck[b][slots], kb[b]], axis=0),
                              np.concatenate([ctx, blk]), rope_base)
        qrot = rope_interleaved(qr[b].transpose(1, 0, 2), blk, rope_base)     # [H, 5, d_r]
        for h in range(H):
            K, V = expand_head(ckv, kr, wk, wv, h)
            Q = np.concatenate([qn[b][:, h, :], qrot[h]], axis=1)
            out[b, :, h, :] = _softmax_rows(scale * (Q @ K.T)) @ V
    return out


def softmax_t(logits, temperature: float = 1.0) -> np.ndarray:
    """softmax(logits / T) over the last axis."""
    return _softmax_rows(np.asarray(logits, np.float64) / float(temperature))


def acceptance(p, q) -> np.ndarray:
    """The explainer page's acceptance rate: sum_v min(p_v, q_v) (for the
    draft distribution q and the target distribution p)."""
    return np.minimum(np.asarray(p, np.float64), np.asarray(q, np.float64)).sum(axis=-1)


def sample_inverse_cdf(weights, u: float) -> int:
    """Draw from the distribution proportional to the non-negative `weights`
    with the uniform u in [0, 1): the first index whose cumulative weight
    exceeds u times the total."""
    w = np.asarray(weights, np.float64)
    c = np.cumsum(w)
    return int(np.argmax(c > u * c[-1]))


def spec_verify(draft_logits, target_logits, draft_tokens, u, mode: str = "rejection",
                temperature: float = 1.0):
    """Verification of K drafted tokens of one sequence (fp64).

    draft_logits [K, V] give q_k, target_logits [K + 1, V] give p_k
    (p_k scores the token after the k-th drafted position; p_K is the
    target's distribution after the last one); draft_tokens [K]; u [K + 1]
    uniforms in [0, 1).  Both distributions are softmax(logits / T).
    "rejection" (rejection sampling): token k is accepted when
    u_k < a_k = min(1, p_k(x_k) / q_k(x_k)); at the first rejection j the next
    token is drawn from the residual max(0, p_j - q_j) (normalised) with u_K;
    when all K are accepted it is drawn from p_K with u_K.  "target_only":
    token k is accepted when it is the target's top choice (the lowest index
    among ties); the next token is p_j's (or p_K's) top choice.
    Returns dict(n_accept, next_token, accept_prob [K] (a_k for every k),
    overlap [K] = sum_v min(p_k, q_k))."""
    q = softmax_t(draft_logits, temperature)
    p = softmax_t(target_logits, temperature)
    K = q.shape[0]
    x = np.asarray(draft_tokens)
    with np.errstate(divide="ignore", over="ignore"):
        a = np.minimum(1.0, np.exp(np.log(p[np.arange(K), x]) - np.log(q[np.arange(K), x])))
    res = dict(accept_prob=a, overlap=acceptance(p[:K], q))
    j = K
    for k in range(K):
        ok = (u[k] < a[k]) if mode == "rejection" else (int(x[k]) == int(np.argmax(p[k])))
        if not ok:
            j = k
            break
    if mode == "rejection":
        w = np.maximum(0.0, p[j] - q[j]) if j < K else p[K]
        if w.sum() == 0.0:          # p_j = q_j: the residual is empty; draw from p_j
            w = p[j]
        nxt = sample_inverse_cdf(w, float(u[K]))
    elif mode == "target_only":
        nxt = int(np.argmax(p[j]))
    else:
        raise ValueError(mode)
    res["n_accept"], res["next_token"] = j, nxt
    return res
