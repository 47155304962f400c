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
// MFMA column tiles of 16 heads (one per query).  Scores are computed
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

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void attn_kernel(
    const bf16* __restrict__ q_rope, const bf16* __restrict__ ckv_ctx,
    const bf16* __restrict__ kr_ctx, const bf16* __restrict__ ckv_blk,
    const bf16* __restrict__ kr_blk, bf16* __restrict__ out, const int4* __restrict__ idx,
    const float2* __restrict__ rope, const bf16* __restrict__ q_abs, bf16* __restrict__ o_lat,
    int S, int N, int L5, int total_blocks, int rows_max, float scale) {
    __shared__ __attribute__((aligned(16))) bf16 ckv_l[kMaxKeys * kCkvStride];
    __shared__ __attribute__((aligned(16))) bf16 kr_l[kMaxKeys * kKrStride];
    __shared__ float2 qcs[kBlock * (kDr / 2)];

    constexpr int kThreads = WAVES * 64;
    constexpr int kGroups = 4 / WAVES;        // workgroups per block
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int blk = lid / kGroups;
    if (blk >= total_blocks) return;
    const int hg0 = (lid % kGroups) * WAVES;  // first 16-head group of this workgroup
    const int tid = threadIdx.x;
    const int b = blk / N, n = blk % N;
    const size_t qrow0 = (size_t)b * L5 + (size_t)kBlock * n;
    const int4 rec = idx[blk];

    if (rec.w < 0) {   // padding block -> 0, kept block with a bad anchor -> NaN
        const bf16 fill = (rec.w == -1) ? (bf16)0.0f : (bf16)__builtin_nanf("");
        bf16x8 fv;
        for (int e = 0; e < 8; ++e) fv[e] = fill;
        constexpr int kChunks = WAVES * 16 * kDv / 8;    // 16-byte chunks per query row
        for (int e = tid; e < kBlock * kChunks; e += kThreads) {
            const int j = e / kChunks, c = e % kChunks;
            st16(out + ((qrow0 + j) * kH + hg0 * 16) * kDv + (size_t)c * 8, fv);
        }
        return;
    }
    const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z, slot = rec.w;
    const int nkeys = ctx_len + kBlock;

    // ---- stage the keys: slot s < ctx_len is context row ctx_lo + s, the
    // rest are the block's own positions; k^R is rotated on the way in
    for (int e = tid; e < nkeys * (kD / 8); e += kThreads) {
        const int s = e / (kD / 8), ch = e % (kD / 8);
        const bf16* src = (s < ctx_len)
                              ? ckv_ctx + ((size_t)b * S + ctx_lo + s) * kD
                              : ckv_blk + (qrow0 + (s - ctx_len)) * kD;
        st16(&ckv_l[s * kCkvStride + ch * 8], ld16(src + ch * 8));
    }
    for (int e = tid; e < nkeys * (kDr / 8); e += kThreads) {
        const int s = e / (kDr / 8), ch = e % (kDr / 8);
        const bool is_ctx = s < ctx_len;
        const bf16* src = is_ctx ? kr_ctx + ((size_t)b * S + ctx_lo + s) * kDr
                                 : kr_blk + (qrow0 + (s - ctx_len)) * kDr;
        const int pos = is_ctx ? ctx_lo + s : pos0 + (s - ctx_len);
        const bf16x8 x = ld16(src + ch * 8);
        bf16x8 y;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float2 cs = rope[(size_t)pos * (kDr / 2) + ch * 4 + q];
            const float x0 = (float)x[2 * q], x1 = (float)x[2 * q + 1];
            y[2 * q] = (bf16)(x0 * cs.x - x1 * cs.y);
            y[2 * q + 1] = (bf16)(x0 * cs.y + x1 * cs.x);
        }
        st16(&kr_l[s * kKrStride + ch * 8], y);
    }
    for (int e = tid; e < kBlock * (kDr / 2); e += kThreads)
        qcs[e] = rope[(size_t)(pos0 + e / (kDr / 2)) * (kDr / 2) + e % (kDr / 2)];
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int head = (hg0 + wave) * 16 + l16;   // this lane's head (B-operand column)
    const int nkt = (nkeys + 15) >> 4;

    // ---- scores, transposed: St[kt][t] = keys (16 kt + 4g + i) x head, query t
    f32x4 st[kMaxKt][kBlock];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt)
#pragma unroll
        for (int t = 0; t < kBlock; ++t) st[kt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    int krow[kMaxKt];
#pragma unroll
    for (int kt = 0; kt < kMaxKt; ++kt) {
        const int r = kt * 16 + l16;
        krow[kt] = (r < nkeys) ? r : nkeys - 1;    // rows past the end are masked below
    }

    // latent part: 16 k-steps of 32 dims; q_abs is stored in the permuted
    // order that matches the two 8-byte c^KV reads below
    const bf16* qa = q_abs + ((size_t)head * rows_max + (size_t)kBlock * slot) * kD + g * 8;
#pragma unroll 2
    for (int ks = 0; ks < kD / 32; ++ks) {
        bf16x8 bq[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) bq[t] = ld16(qa + t * kD + ks * 32);
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
            if (kt < nkt) {
                const bf16* ap = &ckv_l[krow[kt] * kCkvStride + ks * 32 + g * 4];
                const bf16x8 af = cat(ld8(ap), ld8(ap + 16));
#pragma unroll
                for (int t = 0; t < kBlock; ++t) st[kt][t] = mfma_16x16x32(af, bq[t], st[kt][t]);
            }
        }
    }
    // rope part: 2 k-steps of 32 dims, q^R rotated in registers
    const bf16* qr = q_rope + (qrow0 * kH + head) * kDr + g * 8;
#pragma unroll
    for (int ks = 0; ks < kDr / 32; ++ks) {
        bf16x8 bq[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) {
            const bf16x8 x = ld16(qr + (size_t)t * kH * kDr + ks * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 cs = qcs[t * (kDr / 2) + ks * 16 + g * 4 + q];
                const float x0 = (float)x[2 * q], x1 = (float)x[2 * q + 1];
                bq[t][2 * q] = (bf16)(x0 * cs.x - x1 * cs.y);
                bq[t][2 * q + 1] = (bf16)(x0 * cs.y + x1 * cs.x);
            }
        }
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
            if (kt < nkt) {
                const bf16x8 af = ld16(&kr_l[krow[kt] * kKrStride + ks * 32 + g * 8]);
#pragma unroll
                for (int t = 0; t < kBlock; ++t) st[kt][t] = mfma_16x16x32(af, bq[t], st[kt][t]);
            }
        }
    }

    // ---- softmax per (query t, head): keys are spread over i, kt and the
    // four lane groups g (lanes l, l^16, l^32, l^48)
    const float c2 = scale * kLog2e;
    float inv[kBlock];
    bf16x4 pr[kMaxKt][kBlock];
#pragma unroll
    for (int t = 0; t < kBlock; ++t) {
        float m = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
            if (kt < nkt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = kt * 16 + g * 4 + i;
                    const float x = (key < nkeys) ? st[kt][t][i] : -INFINITY;
                    st[kt][t][i] = x;
                    m = fmaxf(m, x);
                }
            }
        }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        const float mc = m * c2;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < kMaxKt; ++kt) {
            if (kt < nkt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = exp2f(fmaf(st[kt][t][i], c2, -mc));
                    pr[kt][t][i] = (bf16)p;
                    sum += p;
                }
            } else {
                pr[kt][t] = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            }
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        inv[t] = 1.0f / sum;
    }

    // ---- o_lat^T = c^KV^T P^T in 64-dim chunks; lane holds dims
    // 64c + 16mt + 4g + i of head `head`, query t
    bf16* ol = o_lat + ((size_t)head * rows_max + (size_t)kBlock * slot) * kD + g * 8;
    const int tr_row = g * 4 + (l16 >> 2);      // transpose-read row inside a 16-key group
    const int tr_col = (l16 & 3) * 4;
#pragma unroll 1
    for (int c = 0; c < kD / 64; ++c) {
        f32x4 o[4][kBlock];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int t = 0; t < kBlock; ++t) o[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < (kMaxKt + 1) / 2; ++kk) {
            if (2 * kk + 1 < nkt) {
                int r0 = 32 * kk + tr_row, r1 = r0 + 16;
                r0 = (r0 < nkeys) ? r0 : nkeys - 1;
                r1 = (r1 < nkeys) ? r1 : nkeys - 1;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int col = c * 64 + mt * 16 + tr_col;
                    const bf16x8 af = cat(lds_read_tr(&ckv_l[r0 * kCkvStride + col]),
                                          lds_read_tr(&ckv_l[r1 * kCkvStride + col]));
#pragma unroll
                    for (int t = 0; t < kBlock; ++t)
                        o[mt][t] = mfma_16x16x32(af, cat(pr[2 * kk][t], pr[2 * kk + 1][t]), o[mt][t]);
                }
            } else if (2 * kk < nkt) {
                int r0 = 32 * kk + tr_row;
                r0 = (r0 < nkeys) ? r0 : nkeys - 1;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int col = c * 64 + mt * 16 + tr_col;
                    const bf16x4 af = lds_read_tr(&ckv_l[r0 * kCkvStride + col]);
#pragma unroll
                    for (int t = 0; t < kBlock; ++t) o[mt][t] = mfma_16x16x16(af, pr[2 * kk][t], o[mt][t]);
                }
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
                    v[i] = (bf16)(a0[i] * inv[t]);
                    v[4 + i] = (bf16)(a1[i] * inv[t]);
                }
                st16(ol + t * kD + c * 64 + pp * 32, v);
            }
        }
    }
}

}  // namespace

hipError_t launch_attn(const Problem& p, const Inputs& in, const Workspace& ws, hipStream_t s) {
    const int total = p.B * p.N;
    // small batches: split the 64 heads over four single-wave workgroups so
    // that more compute units take part
    const bool split = total < 512;
    const int groups = split ? 4 : 1;
    int grid = total * groups;
    grid = (grid + 7) / 8 * 8;
    if (split) {
        hipLaunchKernelGGL(attn_kernel<1>, dim3(grid), dim3(64), 0, s, (const bf16*)in.q_rope,
                           (const bf16*)in.ckv_ctx, (const bf16*)in.kr_ctx,
                           (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk, (bf16*)in.out, ws.idx,
                           ws.rope, ws.qabs, ws.olat, p.S, p.N, p.L5, total, p.rows_max, p.scale);
    } else {
        hipLaunchKernelGGL(attn_kernel<4>, dim3(grid), dim3(256), 0, s, (const bf16*)in.q_rope,
                           (const bf16*)in.ckv_ctx, (const bf16*)in.kr_ctx,
                           (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk, (bf16*)in.out, ws.idx,
                           ws.rope, ws.qabs, ws.olat, p.S, p.N, p.L5, total, p.rows_max, p.scale);
    }
    return hipGetLastError();
}

}  // namespace dspark
