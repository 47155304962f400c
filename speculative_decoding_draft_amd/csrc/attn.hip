// Masked latent attention for one draft block: scores over the 576 cached
// numbers per key, softmax, P . c^KV over 512 dims.  bf16 MFMA, fp32
// accumulation.
//
// What a block sees (GLM 5.2 DSpark training-design page, §3 "attention
// mask"): the context window [ctx_lo, A) and its own 5 draft positions; a
// padding block sees nothing.  Scores (§4 "MLA Projection" in absorbed form,
// scale of §4): s = scale * (q_abs . c^KV + RoPE(q^R) . RoPE(k^R)); the
// attention is the appendix equation softmax(s + Lambda(M)) V with V
// deferred: o_lat = sum_k p_k c^KV_k / sum_k p_k, and W_UV is applied later.
//
// One workgroup stages the block's keys (<= 127 context rows + 5 block rows,
// c^KV 512 + rotated k^R 64 each, ~152 KB) in LDS once and shares them across
// all heads it owns; each wave owns 16 heads, i.e. 80 (query, head) rows as 5
// MFMA column tiles of 16 heads (one per query).  With few blocks, a
// workgroup owns 16 heads and each of its five waves one query (one column
// tile), so that four workgroups per block finish sooner.  Scores are computed
// transposed (keys x rows) so that the probabilities land in registers in the
// layout the P.V MFMA takes as its B operand; V^T fragments come straight out
// of the row-major c^KV tile with ds_read_b64_tr_b16.  With at most 132 keys
// the softmax is exact (no rescaling).
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kCkvStride = kD + 8;    // bf16 per staged c^KV row (1040 B)

constexpr int kKrStride = kDr + 8;    // bf16 per staged k^R row (144 B)
constexpr int kMaxKt = (kMaxKeys + 15) / 16;   // 9 key tiles
constexpr float kLog2e = 1.4426950408889634f;

// WRITE_P: also write the normalised probabilities, rounded to bf16, for a
// backward that reuses them (pmat: [slot][5 H rows][144 key slots], row =
// t H + h; keys past nkeys hold 0).
template <int WAVES, int QW, bool WRITE_P>
__global__ __launch_bounds__(WAVES * 64) void attn_kernel(
    const bf16* __restrict__ q_rope, const bf16* __restrict__ ckv_ctx,
    const bf16* __restrict__ kr_ctx, const bf16* __restrict__ ckv_blk,
    const bf16* __restrict__ kr_blk, const int4* __restrict__ srec,
    const int32_t* __restrict__ status,
    const bf16* __restrict__ q_abs, bf16* __restrict__ o_lat, bf16* __restrict__ pmat,
    int S, int N, int L5, int slot0, int nslots, float scale, uint32_t ctx_bytes,
    uint32_t blk_bytes, RopeTheta turns_per_pos) {
    __shared__ __attribute__((aligned(16))) bf16 ckv_l[kMaxKeys * kCkvStride];
    __shared__ __attribute__((aligned(16))) bf16 kr_l[kMaxKeys * kKrStride];
    __shared__ float2 qcs[kBlock * (kDr / 2)];
    __shared__ double turns[kDr / 2];        // theta_i / 2pi

    constexpr int kThreads = WAVES * 64;
    // QW = 5: each wave owns 16 heads and all 5 queries (a workgroup owns
    // 16 * WAVES heads).  QW = 1: five waves share 16 heads and each owns one
    // query, so that a workgroup finishes ~5x sooner when few blocks leave
    // most compute units idle.
    static_assert(QW == kBlock || WAVES * QW == kBlock, "queries per wave");
    constexpr int kHeadGroups = (QW == kBlock) ? WAVES : 1;   // 16-head groups per workgroup
    constexpr int kGroups = 4 / kHeadGroups;  // workgroups per block
    // live slots of this chunk; the grid covers the chunk's capacity, so
    // spread the live ones evenly over the XCDs
    const int n_here = min(nslots, status[kStKeptCount] - slot0);
    const int lid = xcd_balance(blockIdx.x, n_here * kGroups);
    if (lid < 0) return;
    // slots are taken in descending order: W_UV then walks its rows upwards
    // and first reads the o_lat rows written last (still in the Infinity
    // Cache)
    const int local = n_here - 1 - lid / kGroups;   // slot within the chunk
    const int hg0 = (lid % kGroups) * kHeadGroups;  // first 16-head group of this workgroup
    const int tid = threadIdx.x;
    // wave index as a scalar: the key staging below selects its source
    // tensor per wave, which must be visible to the compiler as uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int head = (hg0 + (QW == kBlock ? wave : 0)) * 16 + l16;   // B-operand column
    const int tq0 = (QW == kBlock) ? 0 : wave * QW;   // this wave's first query
    for (int i = tid; i < kDr / 2; i += kThreads) turns[i] = turns_per_pos.t[i];
    __syncthreads();

    // Q fragments of the first k-steps (all latent) are requested first:
    // they depend on the slot only
    constexpr int kKs = (kD + kDr) / 32;           // 18 k-steps: 16 latent + 2 rope
    constexpr int kPf = 3;                         // prefetch distance (k-steps)
    static_assert(kPf <= kD / 32, "prefetched k-steps are latent ones");
    const bf16* qa = q_abs + ((size_t)kBlock * (slot0 + local) * kH + head) * kD + g * 8;
    bf16x8 qbuf[kPf][QW];
#pragma unroll
    for (int p = 0; p < kPf; ++p)
#pragma unroll
        for (int t = 0; t < QW; ++t) qbuf[p][t] = gld16(qa + (size_t)(tq0 + t) * kH * kD + p * 32);

    const int4 rec = srec[slot0 + local];      // {ctx_lo, ctx_len, pos0, block}
    const int blk = rec.w;
    const int b = blk / N, n = blk % N;
    const size_t qrow0 = (size_t)b * L5 + (size_t)kBlock * n;
    const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z;
    const int nkeys = ctx_len + kBlock;

    // k^R is rotated on the way in: batch the loads, then rotate and store.
    // With four waves one batch covers every key; its loads are issued before
    // the c^KV copies so that the rotation only waits for them (vmcnt retires
    // in order) and overlaps the copies.
    constexpr int kKrChunks = kDr / 8;             // 16-byte chunks per k^R row
    constexpr int kKrBatch = 5;
    constexpr int kKrIters =                       // 1 with four waves
        (kMaxKeys * kKrChunks + kThreads * kKrBatch - 1) / (kThreads * kKrBatch);
    bf16x8 xr[kKrBatch];
    int xpos[kKrBatch];
    auto kr_load = [&](int bi) {
        const int base = bi * kThreads * kKrBatch;
#pragma unroll
        for (int u = 0; u < kKrBatch; ++u) {
            // unconditional (clamped) loads so that the batch is issued back to back
            int e = base + u * kThreads + tid;
            e = (e < nkeys * kKrChunks) ? e : nkeys * kKrChunks - 1;
            const int s = e / kKrChunks, ch = e % kKrChunks;
            const bool is_ctx = s < ctx_len;
            const bf16* src = is_ctx ? kr_ctx + ((size_t)b * S + ctx_lo + s) * kDr
                                     : kr_blk + (qrow0 + (s - ctx_len)) * kDr;
            xpos[u] = is_ctx ? ctx_lo + s : pos0 + (s - ctx_len);
            xr[u] = gld16(src + ch * 8);
        }
    };
    auto kr_store = [&](int bi) {
        const int base = bi * kThreads * kKrBatch;
#pragma unroll
        for (int u = 0; u < kKrBatch; ++u) {
            const int e = base + u * kThreads + tid;
            if (e < nkeys * kKrChunks) {
                const int s = e / kKrChunks, ch = e % kKrChunks;
                bf16x8 y;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float2 cs = rope_cs(turns, xpos[u], ch * 4 + q);
                    const float x0 = (float)xr[u][2 * q], x1 = (float)xr[u][2 * q + 1];
                    const float2 y2 = rope_rot(x0, x1, cs);
                    y[2 * q] = (bf16)y2.x;
                    y[2 * q + 1] = (bf16)y2.y;
                }
                st16(&kr_l[s * kKrStride + ch * 8], y);
            }
        }
    };
    if constexpr (kKrIters == 1) kr_load(0);

    // ---- stage the keys: slot s < ctx_len is context row ctx_lo + s, the
    // rest are the block's own positions.  c^KV rows go straight to LDS, one
    // wave instruction per 1 KB row.
    // A fixed number of copies per wave (slots past the last key receive a
    // copy of the last key and are never read) keeps the wait counts after
    // this loop exact.  The buffer form of the copy is counted by vmcnt only.
    constexpr int kSlotsPerWave = (kMaxKeys + WAVES - 1) / WAVES;
    const __amdgpu_buffer_rsrc_t ctx_rsrc = buffer_rsrc(ckv_ctx, ctx_bytes);
    const __amdgpu_buffer_rsrc_t blk_rsrc = buffer_rsrc(ckv_blk, blk_bytes);
#pragma unroll
    for (int i = 0; i < kSlotsPerWave; ++i) {
        const int slot = wave + i * WAVES;
        if (kMaxKeys % WAVES != 0 && slot >= kMaxKeys) break;   // uniform per wave
        const int s = (slot < nkeys) ? slot : nkeys - 1;
        const bool is_ctx = s < ctx_len;
        const uint32_t row =
            is_ctx ? (uint32_t)(b * S + ctx_lo + s) : (uint32_t)(qrow0 + (s - ctx_len));
        buffer_copy_16(is_ctx ? ctx_rsrc : blk_rsrc, (row * kD + lane * 8) * 2,
                       &ckv_l[slot * kCkvStride]);
    }

    const bf16* qr = q_rope + (qrow0 * kH + head) * kDr + g * 8;
    auto q_frag = [&](int ks, int t) -> bf16x8 {
        return (ks < kD / 32) ? gld16(qa + (size_t)(tq0 + t) * kH * kD + ks * 32)
                              : gld16(qr + (size_t)(tq0 + t) * kH * kDr + (ks - kD / 32) * 32);
    };

    if constexpr (kKrIters == 1) {
        kr_store(0);
    } else {
#pragma unroll
        for (int bi = 0; bi < kKrIters; ++bi) {
            kr_load(bi);
            kr_store(bi);
        }
    }
    // cos/sin of the block's 5 query positions (q^R is rotated in registers)
    for (int e = tid; e < kBlock * (kDr / 2); e += kThreads)
        qcs[e] = rope_cs(turns, pos0 + e / (kDr / 2), e % (kDr / 2));
    // the c^KV copies (the last memory operations issued) are counted by vmcnt
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    __syncthreads();

    // ---- scores, transposed: St[kt][t] = keys (16 kt + 4g + i) x head, query t
    f32x4 st[kMaxKt][QW];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
        for (int t = 0; t < QW; ++t) st[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    int krow[kMaxKt];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt) {
        const int r = kt * 16 + l16;
        krow[kt] = (r < nkeys) ? r : nkeys - 1;    // rows past the end are masked below
    }

    // latent k-steps read c^KV in the permuted order q_abs is stored in (two
    // 8-byte pieces: dims 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3); rope
    // k-steps read k^R in natural order and rotate q^R in registers.  All 9
    // key tiles are always processed (rows past the end are masked), so the
    // A fragments of k-step ks + 1 can be read while k-step ks computes.
    auto a_frag = [&](int ks, int kt) -> bf16x8 {
        if (ks < kD / 32) {
            const bf16* ap = &ckv_l[krow[kt] * kCkvStride + ks * 32 + g * 4];
            return cat(ld8(ap), ld8(ap + 16));
        }
        return ld16(&kr_l[krow[kt] * kKrStride + (ks - kD / 32) * 32 + g * 8]);
    };
    bf16x8 acur[kMaxKt];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = a_frag(0, kt);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        bf16x8 bq[QW];
#pragma unroll
        for (int t = 0; t < QW; ++t) bq[t] = qbuf[ks % kPf][t];
        if (ks + kPf < kKs) {
#pragma unroll
            for (int t = 0; t < QW; ++t) qbuf[ks % kPf][t] = q_frag(ks + kPf, t);
        }
        if (ks >= kD / 32) {
            const int kr = ks - kD / 32;
#pragma unroll
            for (int t = 0; t < QW; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float2 cs = qcs[(tq0 + t) * (kDr / 2) + kr * 16 + g * 4 + q];
                    const float x0 = (float)bq[t][2 * q], x1 = (float)bq[t][2 * q + 1];
                    const float2 y2 = rope_rot(x0, x1, cs);
                    bq[t][2 * q] = (bf16)y2.x;
                    bq[t][2 * q + 1] = (bf16)y2.y;
                }
            }
        }
        bf16x8 anext[kMaxKt];
        if (ks + 1 < kKs) {
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) anext[kt] = a_frag(ks + 1, kt);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
            for (int t = 0; t < QW; ++t) st[kt][t] = mfma_16x16x32(acur[kt], bq[t], st[kt][t]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < kKs) {
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = anext[kt];
        }
    }

    // ---- softmax per (query t, head): keys are spread over i, kt and the
    // four lane groups g (lanes l, l^16, l^32, l^48).  Keys at or past nkeys
    // are masked: inline for the last tile, and in a separate pass over the
    // other tiles when the window is clamped (nkeys < 128).  exp2 is the
    // hardware instruction: arguments are <= 0 and results below 2^-126
    // (relative to the row maximum, which contributes 1) flush to 0.
    if (nkeys < (kMaxKt - 1) * 16) {
#pragma unroll
        for (int kt = 0; kt < kMaxKt - 1; ++kt)
#pragma unroll
            for (int t = 0; t < QW; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt * 16 + g * 4 + i >= nkeys) st[kt][t][i] = -INFINITY;
    }
    auto score = [&](int kt, int t, int i) -> float {
        if (kt == kMaxKt - 1 && kt * 16 + g * 4 + i >= nkeys) return -INFINITY;
        return st[kt][t][i];
    };
    const float c2 = scale * kLog2e;
    float inv[QW];
    bf16x4 pr[kMaxKt][QW];
#pragma unroll
    for (int t = 0; t < QW; ++t) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) m = fmaxf(m, score(kt, t, i));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float mc = m * c2;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(score(kt, t, i), c2, -mc));
                pr[kt][t][i] = (bf16)p;
                sum += p;
            }
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        inv[t] = __builtin_amdgcn_rcpf(sum);    // sum >= 1
        if constexpr (WRITE_P) {
            bf16* dst = pmat + (((size_t)kBlock * (slot0 + local) + tq0 + t) * kH + head) * kKeySlots +
                        g * 4;
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (bf16)((float)pr[kt][t][i] * inv[t]);
                gst8(dst + kt * 16, v);
            }
        }
    }

    // ---- o_lat^T = c^KV^T P^T in 64-dim chunks; lane holds dims
    // 64c + 16mt + 4g + i of head `head`, query t
    bf16* ol = o_lat + ((size_t)kBlock * (slot0 + local) * kH + head) * kD + g * 8;
    const int tr_row = g * 4 + (l16 >> 2);      // transpose-read row inside a 16-key group
    const int tr_col = (l16 & 3) * 4;
    // A (V^T) fragments of step (c, kk) + 1 are read while step (c, kk)
    // computes; kk < 4 covers keys 32kk .. 32kk + 31 (16x16x32), kk = 4 the
    // last tile, keys 128 .. 143 (16x16x16)
    constexpr int kKk = (kMaxKt + 1) / 2;      // 5
    auto v_rows = [&](int kk, int& r0, int& r1) {
        r0 = 32 * kk + tr_row;
        r1 = r0 + 16;
        r0 = (r0 < nkeys) ? r0 : nkeys - 1;
        r1 = (r1 < nkeys) ? r1 : nkeys - 1;
    };
    auto v_frag = [&](int c, int kk, int mt) -> bf16x8 {
        int r0, r1;
        v_rows(kk, r0, r1);
        const int col = c * 64 + mt * 16 + tr_col;
        const bf16x4 lo = lds_read_tr(&ckv_l[r0 * kCkvStride + col]);
        if (kk == kKk - 1) return cat(lo, lo);          // upper half unused
        return cat(lo, lds_read_tr(&ckv_l[r1 * kCkvStride + col]));
    };
    bf16x8 vcur[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) vcur[mt] = v_frag(0, 0, mt);
#pragma unroll
    for (int c = 0; c < kD / 64; ++c) {
        f32x4 o[4][QW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int t = 0; t < QW; ++t) o[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKk; ++kk) {
            const bool last = (c == kD / 64 - 1) && (kk == kKk - 1);
            const int nc = (kk == kKk - 1) ? c + 1 : c;
            const int nkk = (kk == kKk - 1) ? 0 : kk + 1;
            bf16x8 vnext[4];
            if (!last) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) vnext[mt] = v_frag(nc, nkk, mt);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (kk < kKk - 1) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                    for (int t = 0; t < QW; ++t)
                        o[mt][t] = mfma_16x16x32(vcur[mt], cat(pr[2 * kk][t], pr[2 * kk + 1][t]), o[mt][t]);
            } else {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const bf16x4 lo = __builtin_shufflevector(vcur[mt], vcur[mt], 0, 1, 2, 3);
#pragma unroll
                    for (int t = 0; t < QW; ++t) o[mt][t] = mfma_16x16x16(lo, pr[2 * kk][t], o[mt][t]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!last) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) vcur[mt] = vnext[mt];
            }
        }
#pragma unroll
        for (int t = 0; t < QW; ++t) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const f32x4 a0 = o[2 * pp][t], a1 = o[2 * pp + 1][t];
                bf16x8 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = (bf16)(a0[i] * inv[t]);
                    v[4 + i] = (bf16)(a1[i] * inv[t]);
                }
                gst16(ol + (size_t)(tq0 + t) * kH * kD + c * 64 + pp * 32, v);
            }
        }
    }
}

}  // namespace

hipError_t launch_attn(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                       const RopeTheta& th, hipStream_t s, bf16* pmat) {
    // few blocks: four workgroups per block (16 heads each, one wave per
    // query) so that more compute units take part
    const uint32_t ctx_bytes = (uint32_t)((size_t)p.B * p.S * kD * sizeof(bf16));
    const uint32_t blk_bytes = (uint32_t)((size_t)p.B * p.L5 * kD * sizeof(bf16));
    RopeTheta turns{};
    for (int k = 0; k < kDr / 2; ++k) turns.t[k] = th.t[k] * 0.15915494309189533577;  // 1 / 2pi
    const bool split = c.nslots < 160;
    const int groups = split ? 4 : 1;
    int grid = c.nslots * groups;
    grid = (grid + 7) / 8 * 8;
    auto go = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, (const bf16*)in.q_rope,
                           (const bf16*)in.ckv_ctx, (const bf16*)in.kr_ctx,
                           (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk, ws.srec,
                           ws.status, ws.qabs, ws.olat, pmat, p.S, p.N, p.L5,
                           c.slot0, c.nslots, p.scale, ctx_bytes, blk_bytes, turns);
    };
    if (split)
        pmat ? go(attn_kernel<kBlock, 1, true>, kBlock * 64)
             : go(attn_kernel<kBlock, 1, false>, kBlock * 64);
    else
        pmat ? go(attn_kernel<4, kBlock, true>, 256) : go(attn_kernel<4, kBlock, false>, 256);
    return hipGetLastError();
}

}  // namespace dspark
