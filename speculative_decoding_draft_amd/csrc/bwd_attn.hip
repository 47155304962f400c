// Backward of the masked latent attention, per draft block (MFMA path).
//
// For one kept block the workgroup stages the block's keys in LDS exactly as
// the forward does (c^KV rows and rotated k^R of the window [ctx_lo, A) and
// the block's 5 positions; GLM 5.2 DSpark training-design page, §3
// "attention mask" and §4 "RoPE") and shares them over the 64 heads (one
// wave per 16 heads, 80 (query, head) rows per wave).  From the chain rule on
// softmax(scale * Q K^T + Lambda(M)) V in the absorbed form (appendix
// "Attention implementation", §4 "MLA Projection"), with e_k the
// exponentials and l their sum (P_k = e_k / l):
//   scores (as the forward) -> P = e / l, rounded to bf16 once (the P every
//                             product below uses), written out for dc^KV
//   o_lat   = C^T P                              (for dW_UV)
//   dP_k    = d_olat . c_k                       (d_olat = W_UV^T dout, precomputed)
//   D       = sum_k P_k dP_k
//   dS'_k   = scale * P_k (dP_k - D)             written out for the dc^KV products
//   dq_abs  = C^T dS'                            (dq^C = W_UK dq_abs follows)
//   dq^R    = R^T (K_R^T dS')                    rotated back at the query position
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation, in the
// forward's orientation: scores transposed (keys x rows), so P and dS' sit
// in registers as the B operand of the C^T products, whose A operand comes
// out of the row-major c^KV tile with the transposing LDS load.
#include "bwd.hpp"

namespace dspark {

namespace {

constexpr int kCkvStride = kD + 8;    // bf16 per staged c^KV row (1040 B)
constexpr int kKrStride = kDr + 8;    // bf16 per staged k^R row (144 B)
constexpr int kMaxKt = (kMaxKeys + 15) / 16;   // 9 key tiles
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// The same bf16 values, as a fresh value the compiler cannot match with
// earlier conversions of them (otherwise it keeps 180 fp32 copies of P alive
// from the softmax to the dS' step).
__device__ inline bf16x4 fresh(bf16x4 v) {
    uint2 u = __builtin_bit_cast(uint2, v);
    __asm__ volatile("" : "+v"(u.x), "+v"(u.y));
    return __builtin_bit_cast(bf16x4, u);
}

// WRITE_OLAT: also write o_lat (a backward without a forward before it).
// LOAD_P: the forward on this workspace wrote P (normalised, bf16); skip the
// scores and the softmax and read it.
template <bool WRITE_OLAT, bool LOAD_P>
__global__ __launch_bounds__(kThreads) void bwd_attn_kernel(
    const bf16* __restrict__ q_rope, const bf16* __restrict__ ckv_ctx,
    const bf16* __restrict__ kr_ctx, const bf16* __restrict__ ckv_blk,
    const bf16* __restrict__ kr_blk, const int4* __restrict__ srec,
    const int32_t* __restrict__ status, const bf16* __restrict__ q_abs,
    const bf16* __restrict__ dolat, bf16* __restrict__ o_lat, bf16* __restrict__ dqabs,
    bf16* __restrict__ qrot, bf16* __restrict__ pmat, bf16* __restrict__ dsmat,
    bf16* __restrict__ dq_rope, int S, int N, int L5, float scale, uint32_t ctx_bytes,
    uint32_t blk_bytes, RopeTheta turns_per_pos) {
    __shared__ __attribute__((aligned(16))) bf16 ckv_l[kMaxKeys * kCkvStride];
    __shared__ __attribute__((aligned(16))) bf16 kr_l[kMaxKeys * kKrStride];
    __shared__ float2 qcs[kBlock * (kDr / 2)];
    __shared__ double turns[kDr / 2];        // theta_i / 2pi

    const int n_here = status[kStKeptCount];
    // slots are taken in descending order: the d_olat rows the absorb
    // kernel wrote last (still in the Infinity Cache) are read first, and
    // the dc^KV kernel, which walks the slots upwards, then first reads the
    // P / dS' rows written last
    const int lid = xcd_balance(blockIdx.x, n_here);
    if (lid < 0) return;
    const int slot = n_here - 1 - lid;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int head = wave * 16 + l16;           // this lane's head (B-operand column)
    for (int i = tid; i < kDr / 2; i += kThreads) turns[i] = turns_per_pos.t[i];
    __syncthreads();

    constexpr int kKs = (kD + kDr) / 32;           // 18 k-steps: 16 latent + 2 rope
    constexpr int kKl = kD / 32;                   // 16 latent k-steps
    constexpr int kPf = 3;                         // prefetch distance (k-steps)
    const size_t lat_row = (size_t)kBlock * slot * kH + head;   // latent row of (t = 0, head)
    const bf16* qa = q_abs + lat_row * kD + g * 8;
    const bf16* da = dolat + lat_row * kD + g * 8;
    bf16x8 qbuf[kPf][kBlock];
    if constexpr (!LOAD_P) {
#pragma unroll
        for (int p = 0; p < kPf; ++p)
#pragma unroll
            for (int t = 0; t < kBlock; ++t) qbuf[p][t] = gld16(qa + (size_t)t * kH * kD + p * 32);
    }

    const int4 rec = srec[slot];               // {ctx_lo, ctx_len, pos0, block}
    const int blk = rec.w;
    const int b = blk / N, n = blk % N;
    const size_t qrow0 = (size_t)b * L5 + (size_t)kBlock * n;
    const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z;
    const int nkeys = ctx_len + kBlock;

    // ---- stage the keys (the forward's staging): k^R rotated on the way in,
    // c^KV rows straight to LDS, one wave instruction per 1 KB row
    constexpr int kKrChunks = kDr / 8;
    constexpr int kKrBatch = 5;
    static_assert(kMaxKeys * kKrChunks <= kThreads * kKrBatch, "one k^R batch");
    bf16x8 xr[kKrBatch];
    int xpos[kKrBatch];
#pragma unroll
    for (int u = 0; u < kKrBatch; ++u) {
        int e = u * kThreads + tid;
        e = (e < nkeys * kKrChunks) ? e : nkeys * kKrChunks - 1;
        const int s = e / kKrChunks, ch = e % kKrChunks;
        const bool is_ctx = s < ctx_len;
        const bf16* src = is_ctx ? kr_ctx + ((size_t)b * S + ctx_lo + s) * kDr
                                 : kr_blk + (qrow0 + (s - ctx_len)) * kDr;
        xpos[u] = is_ctx ? ctx_lo + s : pos0 + (s - ctx_len);
        xr[u] = gld16(src + ch * 8);
    }
    static_assert(kMaxKeys % kWaves == 0, "slots per wave");
    const __amdgpu_buffer_rsrc_t ctx_rsrc = buffer_rsrc(ckv_ctx, ctx_bytes);
    const __amdgpu_buffer_rsrc_t blk_rsrc = buffer_rsrc(ckv_blk, blk_bytes);
#pragma unroll
    for (int i = 0; i < kMaxKeys / kWaves; ++i) {
        const int sl = wave + i * kWaves;
        const int s = (sl < nkeys) ? sl : nkeys - 1;
        const bool is_ctx = s < ctx_len;
        const uint32_t row =
            is_ctx ? (uint32_t)(b * S + ctx_lo + s) : (uint32_t)(qrow0 + (s - ctx_len));
        buffer_copy_16(is_ctx ? ctx_rsrc : blk_rsrc, (row * kD + lane * 8) * 2,
                       &ckv_l[sl * kCkvStride]);
    }
    const bf16* qr = q_rope + (qrow0 * kH + head) * kDr + g * 8;
    auto q_frag = [&](int ks, int t) -> bf16x8 {
        return (ks < kKl) ? gld16(qa + (size_t)t * kH * kD + ks * 32)
                          : gld16(qr + (size_t)t * kH * kDr + (ks - kKl) * 32);
    };
#pragma unroll
    for (int u = 0; u < kKrBatch; ++u) {
        const int e = u * kThreads + tid;
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
    for (int e = tid; e < kBlock * (kDr / 2); e += kThreads)
        qcs[e] = rope_cs(turns, pos0 + e / (kDr / 2), e % (kDr / 2));
    __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
    __syncthreads();

    int krow[kMaxKt];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt) {
        const int r = kt * 16 + l16;
        krow[kt] = (r < nkeys) ? r : nkeys - 1;    // rows past the end are masked
    }
    // A fragments (keys x 32 dims) in the permuted order the latent rows use
    // for latent k-steps, natural order for the rope k-steps
    auto a_frag = [&](int ks, int kt) -> bf16x8 {
        if (ks < kKl) {
            const bf16* ap = &ckv_l[krow[kt] * kCkvStride + ks * 32 + g * 4];
            return cat(ld8(ap), ld8(ap + 16));
        }
        return ld16(&kr_l[krow[kt] * kKrStride + (ks - kKl) * 32 + g * 8]);
    };

    // ---- scores, transposed: st[kt][t] = keys (16 kt + 4g + i) x head, query t
    f32x4 st[kMaxKt][kBlock];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
        for (int t = 0; t < kBlock; ++t) st[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 acur[kMaxKt];
    bf16* qro = qrot + lat_row * kDr + g * 8;
    const size_t pm_row = (size_t)slot * kBlock * kH + head;
    // P (normalised, bf16): query t, key slots 16 kt + 4g + i of this lane's head
    bf16x4 pr[kMaxKt][kBlock];
    if constexpr (LOAD_P) {
        // the forward wrote P; the rotated q^R rows the k^R gradient products
        // read are still to be written
#pragma unroll
        for (int kr = 0; kr < kDr / 32; ++kr) {
#pragma unroll
            for (int t = 0; t < kBlock; ++t) {
                bf16x8 x = gld16(qr + (size_t)t * kH * kDr + kr * 32);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float2 cs = qcs[t * (kDr / 2) + kr * 16 + g * 4 + q];
                    const float x0 = (float)x[2 * q], x1 = (float)x[2 * q + 1];
                    const float2 y2 = rope_rot(x0, x1, cs);
                    x[2 * q] = (bf16)y2.x;
                    x[2 * q + 1] = (bf16)y2.y;
                }
                gst16(qro + (size_t)t * kH * kDr + kr * 32, x);
            }
        }
#pragma unroll
        for (int t = 0; t < kBlock; ++t)
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt)
                pr[kt][t] = gld8(pmat + (pm_row + (size_t)t * kH) * kKeySlots + g * 4 + kt * 16);
    } else {
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = a_frag(0, kt);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            bf16x8 bq[kBlock];
#pragma unroll
            for (int t = 0; t < kBlock; ++t) bq[t] = qbuf[ks % kPf][t];
            if (ks + kPf < kKs) {
#pragma unroll
                for (int t = 0; t < kBlock; ++t) qbuf[ks % kPf][t] = q_frag(ks + kPf, t);
            }
            if (ks >= kKl) {
                const int kr = ks - kKl;
#pragma unroll
                for (int t = 0; t < kBlock; ++t) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float2 cs = qcs[t * (kDr / 2) + kr * 16 + g * 4 + q];
                        const float x0 = (float)bq[t][2 * q], x1 = (float)bq[t][2 * q + 1];
                        const float2 y2 = rope_rot(x0, x1, cs);
                        bq[t][2 * q] = (bf16)y2.x;
                        bq[t][2 * q + 1] = (bf16)y2.y;
                    }
                    // the rotated q^R, for the k^R gradient products
                    gst16(qro + (size_t)t * kH * kDr + kr * 32, bq[t]);
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
                for (int t = 0; t < kBlock; ++t) st[kt][t] = mfma_16x16x32(acur[kt], bq[t], st[kt][t]);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kKs) {
#pragma unroll
                for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = anext[kt];
            }
        }
        // ---- softmax: keys past nkeys are masked (exp2 of -inf is 0)
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
            for (int t = 0; t < kBlock; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt * 16 + g * 4 + i >= nkeys) st[kt][t][i] = -INFINITY;
        const float c2 = scale * kLog2e;
        float inv[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) {
            float m = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, st[kt][t][i]);
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            const float mc = m * c2;
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][t][i], c2, -mc));
                    pr[kt][t][i] = (bf16)p;
                    sum += p;
                }
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            inv[t] = __builtin_amdgcn_rcpf(sum);    // sum >= 1
            // P = e / l per (row = t*H + head, key slot), rounded to bf16: kept in
            // registers for every product below and written for the dc^KV ones
            bf16* dst = pmat + (pm_row + (size_t)t * kH) * kKeySlots + g * 4;
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) pr[kt][t][i] = (bf16)((float)pr[kt][t][i] * inv[t]);
                gst8(dst + kt * 16, pr[kt][t]);
            }
        }
    }

    // ---- C^T W^T in 64-dim chunks (W = P or dS', keys as k): the lane holds
    // dims 64c + 16mt + 4g + i of head `head`, query t; rows are stored in
    // the permuted latent order, scaled per query by mul[t]
    const int tr_row = g * 4 + (l16 >> 2);
    const int tr_col = (l16 & 3) * 4;
    constexpr int kKk = (kMaxKt + 1) / 2;      // 5: 4 of 32 keys, then keys 128 .. 143
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
        if (kk == kKk - 1) return cat(lo, lo);
        return cat(lo, lds_read_tr(&ckv_l[r1 * kCkvStride + col]));
    };
    auto ct_pass = [&](const bf16x4 (&w)[kMaxKt][kBlock], const float (&mul)[kBlock],
                       bf16* out_base) {
        bf16* ol = out_base + lat_row * kD + g * 8;
        bf16x8 vcur[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) vcur[mt] = v_frag(0, 0, mt);
#pragma unroll
        for (int c = 0; c < kD / 64; ++c) {
            f32x4 o[4][kBlock];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int t = 0; t < kBlock; ++t) o[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
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
                        for (int t = 0; t < kBlock; ++t)
                            o[mt][t] = mfma_16x16x32(vcur[mt], cat(w[2 * kk][t], w[2 * kk + 1][t]),
                                                     o[mt][t]);
                } else {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        const bf16x4 lo = __builtin_shufflevector(vcur[mt], vcur[mt], 0, 1, 2, 3);
#pragma unroll
                        for (int t = 0; t < kBlock; ++t)
                            o[mt][t] = mfma_16x16x16(lo, w[2 * kk][t], o[mt][t]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (!last) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) vcur[mt] = vnext[mt];
                }
            }
#pragma unroll
            for (int t = 0; t < kBlock; ++t) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const f32x4 a0 = o[2 * pp][t], a1 = o[2 * pp + 1][t];
                    bf16x8 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = (bf16)(a0[i] * mul[t]);
                        v[4 + i] = (bf16)(a1[i] * mul[t]);
                    }
                    gst16(ol + (size_t)t * kH * kD + c * 64 + pp * 32, v);
                }
            }
        }
    };
    // o_lat feeds only dW_UV; without WRITE_OLAT the forward's rows, already
    // in the workspace, serve instead (a separate instantiation: a runtime
    // branch here costs registers)
    const float one[kBlock] = {1.f, 1.f, 1.f, 1.f, 1.f};
    if constexpr (WRITE_OLAT) ct_pass(pr, one, o_lat);

    // ---- dP (transposed, keys x rows) = C . d_olat over the 16 latent k-steps
#pragma unroll
    for (int p = 0; p < kPf; ++p)
#pragma unroll
        for (int t = 0; t < kBlock; ++t) qbuf[p][t] = gld16(da + (size_t)t * kH * kD + p * 32);
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
        for (int t = 0; t < kBlock; ++t) st[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = a_frag(0, kt);
#pragma unroll
    for (int ks = 0; ks < kKl; ++ks) {
        bf16x8 bq[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) bq[t] = qbuf[ks % kPf][t];
        if (ks + kPf < kKl) {
#pragma unroll
            for (int t = 0; t < kBlock; ++t)
                qbuf[ks % kPf][t] = gld16(da + (size_t)t * kH * kD + (ks + kPf) * 32);
        }
        bf16x8 anext[kMaxKt];
        if (ks + 1 < kKl) {
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) anext[kt] = a_frag(ks + 1, kt);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
            for (int t = 0; t < kBlock; ++t) st[kt][t] = mfma_16x16x32(acur[kt], bq[t], st[kt][t]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < kKl) {
#pragma unroll
            for (int kt = 0; kt < kMaxKt; ++kt) acur[kt] = anext[kt];
        }
    }

    // ---- dS' = scale * P (dP - D), D = sum_k P_k dP_k (keys past nkeys have
    // e = 0); written out for the dc^KV products and kept for the rest
#pragma unroll
    for (int t = 0; t < kBlock; ++t) {
        float dsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
            pr[kt][t] = fresh(pr[kt][t]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dsum += (float)pr[kt][t][i] * st[kt][t][i];
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        const float dd = dsum;
        const float f = scale;
        bf16* dst = dsmat + (pm_row + (size_t)t * kH) * kKeySlots + g * 4;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pr[kt][t][i] = (bf16)(f * (float)pr[kt][t][i] * (st[kt][t][i] - dd));
            gst8(dst + kt * 16, pr[kt][t]);
        }
    }

    // ---- dq_abs = C^T dS'
    ct_pass(pr, one, dqabs);

    // ---- d(R q^R) = K_R^T dS' (64 dims), rotated back to dq^R
    {
        f32x4 o[4][kBlock];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int t = 0; t < kBlock; ++t) o[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // Every update of an accumulator is a 16x16x32 MFMA (the last key
        // tile, keys 128 .. 143, pads its k-slots with zeros) and the key
        // steps are kept apart: a 16x16x16 MFMA issued right after a
        // 16x16x32 one into the same accumulator has read a stale
        // accumulator for its first two elements here.
        const bf16x4 zero4 = {};
#pragma unroll
        for (int kk = 0; kk < kKk; ++kk) {
            int r0, r1;
            v_rows(kk, r0, r1);
            bf16x8 a[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int col = mt * 16 + tr_col;
                const bf16x4 lo = lds_read_tr(&kr_l[r0 * kKrStride + col]);
                a[mt] = (kk < kKk - 1) ? cat(lo, lds_read_tr(&kr_l[r1 * kKrStride + col]))
                                       : cat(lo, lo);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int t = 0; t < kBlock; ++t) {
                    const bf16x8 w = (kk < kKk - 1) ? cat(pr[2 * kk][t], pr[2 * kk + 1][t])
                                                    : cat(pr[2 * kk][t], zero4);
                    o[mt][t] = mfma_16x16x32(a[mt], w, o[mt][t]);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane holds dims 16 mt + 4g + i: pairs (4g, 4g+1) and (4g+2, 4g+3)
#pragma unroll
        for (int t = 0; t < kBlock; ++t) {
            bf16* dst = dq_rope + ((qrow0 + t) * kH + head) * kDr + 4 * g;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                bf16x4 v;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float2 cs = qcs[t * (kDr / 2) + 8 * mt + 2 * g + q];
                    const float y0 = o[mt][t][2 * q], y1 = o[mt][t][2 * q + 1];
                    v[2 * q] = (bf16)(y0 * cs.x + y1 * cs.y);
                    v[2 * q + 1] = (bf16)(-y0 * cs.y + y1 * cs.x);
                }
                gst8(dst + 16 * mt, v);
            }
        }
    }
}

}  // namespace

hipError_t launch_bwd_attn(const Problem& p, const Inputs& in, const BwdGrads& g,
                           const BwdWork& w, const RopeTheta& th, hipStream_t s, bool write_olat,
                           bool load_p) {
    const uint32_t ctx_bytes = (uint32_t)((size_t)p.B * p.S * kD * sizeof(bf16));
    const uint32_t blk_bytes = (uint32_t)((size_t)p.B * p.L5 * kD * sizeof(bf16));
    RopeTheta turns{};
    for (int k = 0; k < kDr / 2; ++k) turns.t[k] = th.t[k] * 0.15915494309189533577;  // 1 / 2pi
    int grid = p.B * p.N;
    grid = (grid + 7) / 8 * 8;
    // a backward that writes o_lat has no forward's P to load
    auto* kernel = write_olat ? bwd_attn_kernel<true, false>
                   : load_p   ? bwd_attn_kernel<false, true>
                              : bwd_attn_kernel<false, false>;
    hipLaunchKernelGGL(kernel, dim3(grid),
                       dim3(kThreads), 0, s,
                       (const bf16*)in.q_rope, (const bf16*)in.ckv_ctx, (const bf16*)in.kr_ctx,
                       (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk, w.fwd.srec, w.fwd.status,
                       w.fwd.qabs, w.dolat, w.fwd.olat, w.dqabs, w.qrot, w.pmat, w.dsmat,
                       (bf16*)g.dq_rope, p.S, p.N, p.L5, p.scale, ctx_bytes, blk_bytes, turns);
    return hipGetLastError();
}

}  // namespace dspark
