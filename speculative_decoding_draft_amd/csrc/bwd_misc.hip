// Backward of the masked latent attention: accumulator clearing, the
// generic kernel (any dims, fp32 arithmetic) and the final pass that turns
// the fp32 accumulators into the gradient tensors.
//
// Gradients follow from the chain rule on the attention of the GLM 5.2
// DSpark training-design page (appendix "Attention implementation":
// softmax(scale * Q K^T + Lambda(M)) V, with the keys and values of §4 "MLA
// Projection" and the rotation of §4 "RoPE"), taken in the absorbed latent
// form.  Per kept block, head h and query j, with P the softmax weights over
// the visible keys k and G = dout[j, h]:
//   d_olat_j = W_UV[h]^T G                      (gradient of o_lat)
//   dP_jk    = d_olat_j . c_k,  D_j = sum_k P_jk dP_jk
//   dS'_jk   = scale * P_jk (dP_jk - D_j)       (gradient of the logits, times scale)
//   dq_abs_j = sum_k dS'_jk c_k  ->  dq^C_j = W_UK[h] dq_abs_j
//   d(R q^R)_j = sum_k dS'_jk (R k^R)_k          ->  dq^R_j = R^T (...)
//   dc_k    += sum_j P_jk d_olat_j + dS'_jk q_abs_j
//   d(R k^R)_k += sum_j dS'_jk (R q^R)_j         ->  dk^R_k = R^T (...)
//   dW_UV[h] += sum_j G (o_lat_j)^T,  dW_UK[h] += sum_j q^C_j (dq_abs_j)^T
// The sums over heads and over the blocks whose windows share a context row
// are accumulated in fp32 (device atomics).
#include <algorithm>

#include "bwd.hpp"

namespace dspark {

namespace {

template <typename T> __device__ inline float ldf(const T* p, size_t i);
template <> __device__ inline float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ldf<bf16>(const bf16* p, size_t i) { return (float)p[i]; }
template <typename T> __device__ inline void stf(T* p, size_t i, float v);
template <> __device__ inline void stf<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ inline void stf<bf16>(bf16* p, size_t i, float v) { p[i] = (bf16)v; }

__global__ void zero_kernel(float4* __restrict__ p, size_t n4, const int32_t* only_if) {
    if (only_if && *only_if == 0) return;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = z;
}

// A backward told to reuse the forward's index and latents checks that the
// workspace's last index build was for this descriptor and path.
__global__ __launch_bounds__(256) void reuse_check_kernel(int32_t* __restrict__ status,
                                                          int4* __restrict__ idx, int total,
                                                          int32_t expect, int32_t expect2) {
    const int32_t tag = status[kStPathTag];
    if (tag == expect || (expect2 != 0 && tag == expect2)) {
        if (blockIdx.x == 0 && threadIdx.x == 0) status[kStReuseBad] = 0;
        return;
    }
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x)
        idx[i] = make_int4(0, 0, 0, -1);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        status[kStReuseBad] = 1;
        status[kStKeptCount] = 0;
        status[kStFirstBad] = -1;
    }
}

struct GradSpans {
    void* ptr[8];
    size_t n[8];      // elements
};

__global__ __launch_bounds__(256) void reuse_fill_kernel(const int32_t* __restrict__ status,
                                                         GradSpans g, int elem) {
    if (status[kStReuseBad] == 0) return;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (int t = 0; t < 8; ++t) {
        if (!g.ptr[t]) continue;
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < g.n[t]; i += stride) {
            if (elem == 2) static_cast<uint16_t*>(g.ptr[t])[i] = 0x7FC0u;
            else static_cast<uint32_t*>(g.ptr[t])[i] = 0x7FC00000u;
        }
    }
}

int vmax_of(const Problem& p) {
    const int ctx_max = (p.W - 1 < p.S - 2) ? p.W - 1 : (p.S - 2 > 0 ? p.S - 2 : 0);
    return ctx_max + kBlock;
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_generic_kernel(
    Problem p, const T* __restrict__ q_nope, const T* __restrict__ q_rope,
    const T* __restrict__ ckv_ctx, const T* __restrict__ kr_ctx, const T* __restrict__ ckv_blk,
    const T* __restrict__ kr_blk, const T* __restrict__ w_uk, const T* __restrict__ w_uv,
    const T* __restrict__ dout, T* __restrict__ dq_nope, T* __restrict__ dq_rope,
    float* __restrict__ acc, float* __restrict__ wacc, const int4* __restrict__ idx,
    const float2* __restrict__ rope, int vmax) {
    extern __shared__ float sm[];
    const int blk = blockIdx.x;            // b * N + n
    const int h = blockIdx.y;
    const int b = blk / p.N, n = blk % p.N;
    const int tid = threadIdx.x;
    const int D = p.D, dr = p.dr, pairs = p.dr / 2, dc = p.dc, dv = p.dv;
    const int4 rec = idx[blk];
    if (rec.w < 0) return;                 // not computed; rows filled by the final pass
    const size_t qrow0 = (size_t)b * p.L5 + (size_t)kBlock * n;
    const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z;
    const int nkeys = ctx_len + kBlock;
    const size_t arow0 = (size_t)b * (p.S + p.L5);   // accumulator rows of sample b

    float* qa = sm;                        // [5][D]  q_abs
    float* qr = qa + kBlock * D;           // [5][dr] rotated q^R
    float* dol = qr + kBlock * dr;         // [5][D]  W_UV^T dout
    float* ol = dol + kBlock * D;          // [5][D]  o_lat
    float* dqa = ol + kBlock * D;          // [5][D]  dq_abs
    float* P = dqa + kBlock * D;           // [5][vmax] weights
    float* dS = P + kBlock * vmax;         // [5][vmax] dP, then scale * dS

    auto key_row = [&](int s, const T*& ckv, const T*& kr, size_t& row, int& pos) {
        const bool is_ctx = s < ctx_len;
        row = is_ctx ? ((size_t)b * p.S + ctx_lo + s) : (qrow0 + (s - ctx_len));
        ckv = is_ctx ? ckv_ctx : ckv_blk;
        kr = is_ctx ? kr_ctx : kr_blk;
        pos = is_ctx ? ctx_lo + s : pos0 + (s - ctx_len);
    };
    auto kr_rot = [&](const T* kr, size_t row, int pos, int i, float& y0, float& y1) {
        const float x0 = ldf(kr, row * dr + 2 * i), x1 = ldf(kr, row * dr + 2 * i + 1);
        const float2 cs = rope[(size_t)pos * pairs + i];
        y0 = x0 * cs.x - x1 * cs.y;
        y1 = x0 * cs.y + x1 * cs.x;
    };

    for (int e = tid; e < kBlock * D; e += blockDim.x) {
        const int j = e / D, d = e % D;
        const size_t qo = ((qrow0 + j) * p.H + h) * dc;
        const size_t go = ((qrow0 + j) * p.H + h) * dv;
        float a = 0.f, g = 0.f;
        for (int c = 0; c < dc; ++c) a += ldf(q_nope, qo + c) * ldf(w_uk, ((size_t)h * dc + c) * D + d);
        for (int v = 0; v < dv; ++v) g += ldf(dout, go + v) * ldf(w_uv, ((size_t)h * dv + v) * D + d);
        qa[e] = a;
        dol[e] = g;
    }
    for (int e = tid; e < kBlock * pairs; e += blockDim.x) {
        const int j = e / pairs, i = e % pairs;
        const size_t qo = ((qrow0 + j) * p.H + h) * dr;
        const float x0 = ldf(q_rope, qo + 2 * i), x1 = ldf(q_rope, qo + 2 * i + 1);
        const float2 cs = rope[(size_t)(pos0 + j) * pairs + i];
        qr[j * dr + 2 * i] = x0 * cs.x - x1 * cs.y;
        qr[j * dr + 2 * i + 1] = x0 * cs.y + x1 * cs.x;
    }
    __syncthreads();

    // scores, and dP_jk = d_olat_j . c_k
    for (int e = tid; e < kBlock * nkeys; e += blockDim.x) {
        const int j = e / nkeys, s = e % nkeys;
        const T *ckv, *kr;
        size_t row;
        int pos;
        key_row(s, ckv, kr, row, pos);
        float sc = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
            const float c = ldf(ckv, row * D + d);
            sc += qa[j * D + d] * c;
            dp += dol[j * D + d] * c;
        }
        for (int i = 0; i < pairs; ++i) {
            float y0, y1;
            kr_rot(kr, row, pos, i, y0, y1);
            sc += qr[j * dr + 2 * i] * y0 + qr[j * dr + 2 * i + 1] * y1;
        }
        P[j * vmax + s] = sc * p.scale;
        dS[j * vmax + s] = dp;
    }
    __syncthreads();
    if (tid < kBlock) {
        float m = -INFINITY;
        for (int s = 0; s < nkeys; ++s) m = fmaxf(m, P[tid * vmax + s]);
        float sum = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            const float w = expf(P[tid * vmax + s] - m);
            P[tid * vmax + s] = w;
            sum += w;
        }
        const float inv = 1.0f / sum;
        float dsum = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            P[tid * vmax + s] *= inv;
            dsum += P[tid * vmax + s] * dS[tid * vmax + s];
        }
        for (int s = 0; s < nkeys; ++s)
            dS[tid * vmax + s] = p.scale * P[tid * vmax + s] * (dS[tid * vmax + s] - dsum);
    }
    __syncthreads();

    // o_lat and dq_abs
    for (int e = tid; e < kBlock * D; e += blockDim.x) {
        const int j = e / D, d = e % D;
        float o = 0.f, q = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            const T *ckv, *kr;
            size_t row;
            int pos;
            key_row(s, ckv, kr, row, pos);
            const float c = ldf(ckv, row * D + d);
            o += P[j * vmax + s] * c;
            q += dS[j * vmax + s] * c;
        }
        ol[e] = o;
        dqa[e] = q;
    }
    // d(R q^R) -> dq^R = R^T (...)
    for (int e = tid; e < kBlock * pairs; e += blockDim.x) {
        const int j = e / pairs, i = e % pairs;
        float g0 = 0.f, g1 = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            const T *ckv, *kr;
            size_t row;
            int pos;
            key_row(s, ckv, kr, row, pos);
            float y0, y1;
            kr_rot(kr, row, pos, i, y0, y1);
            g0 += dS[j * vmax + s] * y0;
            g1 += dS[j * vmax + s] * y1;
        }
        const float2 cs = rope[(size_t)(pos0 + j) * pairs + i];
        const size_t qo = ((qrow0 + j) * p.H + h) * dr;
        stf(dq_rope, qo + 2 * i, g0 * cs.x + g1 * cs.y);
        stf(dq_rope, qo + 2 * i + 1, -g0 * cs.y + g1 * cs.x);
    }
    __syncthreads();

    // dq^C = W_UK[h] dq_abs
    for (int e = tid; e < kBlock * dc; e += blockDim.x) {
        const int j = e / dc, c = e % dc;
        float a = 0.f;
        for (int d = 0; d < D; ++d) a += ldf(w_uk, ((size_t)h * dc + c) * D + d) * dqa[j * D + d];
        stf(dq_nope, ((qrow0 + j) * p.H + h) * dc + c, a);
    }
    // per-key sums: dc_k and d(R k^R)_k
    for (int e = tid; e < nkeys * (D + dr); e += blockDim.x) {
        const int s = e / (D + dr), d = e % (D + dr);
        float a = 0.f;
        if (d < D) {
            for (int j = 0; j < kBlock; ++j)
                a += P[j * vmax + s] * dol[j * D + d] + dS[j * vmax + s] * qa[j * D + d];
        } else {
            for (int j = 0; j < kBlock; ++j) a += dS[j * vmax + s] * qr[j * dr + (d - D)];
        }
        const size_t arow = arow0 + ((s < ctx_len) ? (size_t)(ctx_lo + s)
                                                   : (size_t)p.S + kBlock * n + (s - ctx_len));
        atomicAdd(&acc[arow * (D + dr) + d], a);
    }
    // weight gradients
    for (int e = tid; e < (dc + dv) * D; e += blockDim.x) {
        const int r = e / D, d = e % D;
        float a = 0.f;
        if (r < dc) {
            for (int j = 0; j < kBlock; ++j)
                a += ldf(q_nope, ((qrow0 + j) * p.H + h) * dc + r) * dqa[j * D + d];
        } else {
            for (int j = 0; j < kBlock; ++j)
                a += ldf(dout, ((qrow0 + j) * p.H + h) * dv + (r - dc)) * ol[j * D + d];
        }
        atomicAdd(&wacc[((size_t)h * (dc + dv) + r) * D + d], a);
    }
}

// One workgroup per accumulator row (grid-stride), threads over element
// pairs: c^KV pairs are converted, k^R pairs rotated back with R^T.
template <typename T>
__global__ __launch_bounds__(256) void bwd_finalize_kernel(
    Problem p, const float* __restrict__ acc, const float* __restrict__ wacc,
    T* __restrict__ dckv_ctx, T* __restrict__ dkr_ctx, T* __restrict__ dckv_blk,
    T* __restrict__ dkr_blk, T* __restrict__ dq_nope, T* __restrict__ dq_rope,
    T* __restrict__ dw_uk, T* __restrict__ dw_uv, const int4* __restrict__ idx,
    const float2* __restrict__ table, RopeTheta turns, int weights) {
    __shared__ double tn[kMaxRopePairs];
    const int D = p.D, dr = p.dr, pairs = p.dr / 2;
    if (!table) {
        for (int i = threadIdx.x; i < pairs; i += blockDim.x) tn[i] = turns.t[i];
        __syncthreads();
    }
    auto cs_of = [&](int pos, int i) -> float2 {
        return table ? table[(size_t)pos * pairs + i] : rope_cs(tn, pos, i);
    };
    const size_t rows_per_b = (size_t)p.S + p.L5;
    const size_t n_rows = (size_t)p.B * rows_per_b;
    const int half = (D + dr) / 2;
    for (size_t r = blockIdx.x; r < n_rows; r += gridDim.x) {
        const int b = (int)(r / rows_per_b);
        const int rr = (int)(r % rows_per_b);
        T *ckv_out, *kr_out;
        int pos = 0;
        bool live = true;
        if (rr < p.S) {
            ckv_out = dckv_ctx + ((size_t)b * p.S + rr) * D;
            kr_out = dkr_ctx + ((size_t)b * p.S + rr) * dr;
            pos = rr;
        } else {
            const int q = rr - p.S, n = q / kBlock, j = q % kBlock;
            const int4 rec = idx[(size_t)b * p.N + n];
            live = rec.w >= 0;
            pos = live ? rec.z + j : 0;
            ckv_out = dckv_blk + ((size_t)b * p.L5 + q) * D;
            kr_out = dkr_blk + ((size_t)b * p.L5 + q) * dr;
        }
        const float* a = acc + r * (size_t)(D + dr);
        for (int e = threadIdx.x; e < half; e += blockDim.x) {
            const int k = 2 * e;
            const float x0 = live ? a[k] : 0.f, x1 = live ? a[k + 1] : 0.f;
            if (k < D) {
                stf(ckv_out, k, x0);
                stf(ckv_out, k + 1, x1);
            } else {
                const int i = (k - D) / 2;
                const float2 cs = cs_of(pos, i);
                stf(kr_out, k - D, x0 * cs.x + x1 * cs.y);
                stf(kr_out, k - D + 1, -x0 * cs.y + x1 * cs.x);
            }
        }
    }
    // query-gradient rows of blocks that were not computed
    const size_t qw = (size_t)p.H * (p.dc + dr);
    for (size_t blk = blockIdx.x; blk < (size_t)p.B * p.N; blk += gridDim.x) {
        const int4 rec = idx[blk];
        if (rec.w >= 0) continue;
        const float fill = (rec.w == -1) ? 0.0f : __builtin_nanf("");
        const size_t b = blk / p.N, n = blk % p.N;
        const size_t qrow0 = b * p.L5 + kBlock * n;
        for (size_t e = threadIdx.x; e < kBlock * qw; e += blockDim.x) {
            const size_t j = e / qw, w = e % qw;
            const size_t h = w / (p.dc + dr), c = w % (p.dc + dr);
            if (c < (size_t)p.dc)
                stf(dq_nope, ((qrow0 + j) * p.H + h) * p.dc + c, fill);
            else
                stf(dq_rope, ((qrow0 + j) * p.H + h) * dr + (c - p.dc), fill);
        }
    }
    if (weights) {
        const size_t per_h = (size_t)(p.dc + p.dv) * D;
        const size_t total = (size_t)p.H * per_h;
        for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
             e += (size_t)gridDim.x * blockDim.x) {
            const size_t h = e / per_h, w = e % per_h;
            const size_t r = w / D, d = w % D;
            if (r < (size_t)p.dc)
                stf(dw_uk, (h * p.dc + r) * D + d, wacc[e]);
            else
                stf(dw_uv, (h * p.dv + (r - p.dc)) * D + d, wacc[e]);
        }
    }
}

// First slot in [0, n) whose key (sample, anchor) is greater than (b, a);
// slots are ordered by that key when the anchors ascend.
__device__ inline int first_after(const int4* __restrict__ srec, int n, int N, int b, int a) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const int4 r = srec[mid];
        const int rb = r.w / N;
        if (rb > b || (rb == b && r.z > a)) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// One 64-lane group per row (4 rows per workgroup of 256).  A row is 144
// float4: lane l holds float4 l and 64 + l (c^KV dims 4l.., 256 + 4l..), and
// lanes 0..15 also float4 128 + l (k^R dims 4l .. 4l+3, rotated back).
__global__ __launch_bounds__(256) void gather_kernel(
    Problem p, const float* __restrict__ part, const float* __restrict__ acc,
    const int4* __restrict__ srec, const int4* __restrict__ idx,
    const int32_t* __restrict__ status, bf16* __restrict__ dckv_ctx, bf16* __restrict__ dkr_ctx,
    bf16* __restrict__ dckv_blk, bf16* __restrict__ dkr_blk, bf16* __restrict__ dq_nope,
    bf16* __restrict__ dq_rope, RopeTheta turns) {
    __shared__ double tn[kDr / 2];
    for (int i = threadIdx.x; i < kDr / 2; i += blockDim.x) tn[i] = turns.t[i];
    __syncthreads();
    const bool unsorted = status[kStUnsorted] != 0;
    const int n_live = status[kStKeptCount];
    // sub is wave-uniform: the index records are then read with scalar loads
    // (the binary searches below run on the scalar cache)
    const int lane = threadIdx.x & 63, sub = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t rows_per_b = (size_t)p.S + p.L5;
    const size_t n_rows = (size_t)p.B * rows_per_b;
    for (size_t r = (size_t)blockIdx.x * 4 + sub; r < n_rows; r += (size_t)gridDim.x * 4) {
        const int b = (int)(r / rows_per_b);
        const int rr = (int)(r % rows_per_b);
        float4 v[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int nv = (lane < kDr / 4) ? 3 : 2;
        int pos = rr;
        bf16 *ckv_out, *kr_out;
        bool live = true;
        if (rr < p.S) {
            ckv_out = dckv_ctx + ((size_t)b * p.S + rr) * kD;
            kr_out = dkr_ctx + ((size_t)b * p.S + rr) * kDr;
        } else {
            const int q = rr - p.S, n = q / kBlock, j = q % kBlock;
            const int4 rec = idx[(size_t)b * p.N + n];
            live = rec.w >= 0;
            pos = live ? rec.z + j : 0;
            ckv_out = dckv_blk + ((size_t)b * p.L5 + q) * kD;
            kr_out = dkr_blk + ((size_t)b * p.L5 + q) * kDr;
        }
        auto add_row = [&](const float* src) {
            const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (k < nv) {
                    const float4 x = s4[lane + 64 * k];
                    v[k].x += x.x; v[k].y += x.y; v[k].z += x.z; v[k].w += x.w;
                }
            }
        };
        if (live) {
            if (unsorted) {
                add_row(acc + r * (kD + kDr));
            } else if (rr < p.S) {
                // the blocks whose windows [A-W+1, A) hold row rr: r < A <= rr + W - 1
                const int s0 = first_after(srec, n_live, p.N, b, rr);
                const int s1 = first_after(srec, n_live, p.N, b, rr + p.W - 1);
                // up to four covering blocks' loads in flight at once
                for (int sl = s0; sl < s1; sl += 4) {
                    float4 x[4][3];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (sl + u < s1) {
                            const int4 rec = srec[sl + u];
                            const float4* s4 = reinterpret_cast<const float4*>(
                                part + ((size_t)(sl + u) * kMaxKeys + (rr - rec.x)) * (kD + kDr));
#pragma unroll
                            for (int k = 0; k < 3; ++k)
                                if (k < nv) x[u][k] = s4[lane + 64 * k];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        if (sl + u < s1) {
#pragma unroll
                            for (int k = 0; k < 3; ++k) {
                                if (k < nv) {
                                    v[k].x += x[u][k].x; v[k].y += x[u][k].y;
                                    v[k].z += x[u][k].z; v[k].w += x[u][k].w;
                                }
                            }
                        }
                    }
                }
            } else {
                const int q = rr - p.S, n = q / kBlock, j = q % kBlock;
                const int4 rec = idx[(size_t)b * p.N + n];
                add_row(part + ((size_t)rec.w * kMaxKeys + rec.y + j) * (kD + kDr));
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 4 * (lane + 64 * k);
            gst8(ckv_out + e, bf16x4{(bf16)v[k].x, (bf16)v[k].y, (bf16)v[k].z, (bf16)v[k].w});
        }
        if (nv == 3) {
            const int e = 4 * lane;                   // k^R dims e .. e+3: pairs e/2, e/2+1
            const float2 c0 = rope_cs(tn, pos, e / 2), c1 = rope_cs(tn, pos, e / 2 + 1);
            const float4 y = v[2];
            gst8(kr_out + e, bf16x4{(bf16)(y.x * c0.x + y.y * c0.y), (bf16)(-y.x * c0.y + y.y * c0.x),
                                    (bf16)(y.z * c1.x + y.w * c1.y), (bf16)(-y.z * c1.y + y.w * c1.x)});
        }
    }
    // query-gradient rows of blocks that were not computed: 0 (padding) or
    // NaN (kept, bad anchor)
    const size_t qw = (size_t)kH * (kDc + kDr);
    for (size_t blk = blockIdx.x; blk < (size_t)p.B * p.N; blk += gridDim.x) {
        const int4 rec = idx[blk];
        if (rec.w >= 0) continue;
        const bf16 f = (bf16)((rec.w == -1) ? 0.0f : __builtin_nanf(""));
        const bf16x4 fill = {f, f, f, f};
        const size_t b = blk / p.N, n = blk % p.N;
        const size_t qrow0 = b * p.L5 + kBlock * n;
        for (size_t e = threadIdx.x; e < kBlock * qw / 4; e += blockDim.x) {
            const size_t j = (4 * e) / qw, w = (4 * e) % qw;
            const size_t h = w / (kDc + kDr), c = w % (kDc + kDr);
            if (c < (size_t)kDc)
                gst8(dq_nope + ((qrow0 + j) * kH + h) * kDc + c, fill);
            else
                gst8(dq_rope + ((qrow0 + j) * kH + h) * kDr + (c - kDc), fill);
        }
    }
}

}  // namespace

hipError_t launch_bwd_reuse_check(const Problem& p, const BwdWork& w, int32_t expect,
                                  int32_t expect2, hipStream_t s) {
    const int total = p.B * p.N;
    const int grid = std::max(1, std::min(256, (total + 255) / 256));
    hipLaunchKernelGGL(reuse_check_kernel, dim3(grid), dim3(256), 0, s, w.fwd.status, w.fwd.idx,
                       total, expect, expect2);
    return hipGetLastError();
}

hipError_t launch_bwd_reuse_fill(const Problem& p, const BwdGrads& g, const BwdWork& w,
                                 int elem, hipStream_t s) {
    const size_t B = p.B, L5 = p.L5, S = p.S, H = p.H;
    GradSpans sp{{g.dq_nope, g.dq_rope, g.dckv_ctx, g.dkr_ctx, g.dckv_blk, g.dkr_blk, g.dw_uk,
                  g.dw_uv},
                 {B * L5 * H * p.dc, B * L5 * H * p.dr, B * S * p.D, B * S * p.dr, B * L5 * p.D,
                  B * L5 * p.dr, H * p.dc * p.D, H * p.dv * p.D}};
    hipLaunchKernelGGL(reuse_fill_kernel, dim3(256), dim3(256), 0, s, w.fwd.status, sp, elem);
    return hipGetLastError();
}

hipError_t launch_bwd_gather(const Problem& p, const BwdGrads& g, const BwdWork& w,
                             const RopeTheta& th, hipStream_t s) {
    RopeTheta turns{};
    for (int k = 0; k < kDr / 2; ++k) turns.t[k] = th.t[k] * 0.15915494309189533577;  // 1 / 2pi
    const size_t rows = (size_t)p.B * ((size_t)p.S + p.L5);
    const size_t want = (rows + 3) / 4;
    const int grid = (int)(want < 16384 ? want : 16384);
    hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(256), 0, s, p, w.part, w.acc, w.fwd.srec,
                       w.fwd.idx, w.fwd.status, (bf16*)g.dckv_ctx, (bf16*)g.dkr_ctx,
                       (bf16*)g.dckv_blk, (bf16*)g.dkr_blk, (bf16*)g.dq_nope, (bf16*)g.dq_rope,
                       turns);
    return hipGetLastError();
}

hipError_t launch_bwd_zero(float* p, size_t n, const int32_t* only_if, hipStream_t s) {
    // rounded up to whole float4: every workspace area starts 256-byte
    // aligned and is padded to a multiple of 256 bytes
    const size_t n4 = (n + 3) / 4;
    if (n4 == 0) return hipSuccess;
    const size_t want = (n4 + 255) / 256;
    const int grid = (int)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<float4*>(p),
                       n4, only_if);
    return hipGetLastError();
}

size_t bwd_generic_lds_bytes(const Problem& p) {
    const size_t vmax = (size_t)vmax_of(p);
    return sizeof(float) * (size_t)kBlock * (4 * (size_t)p.D + p.dr + 2 * vmax);
}

hipError_t launch_bwd_generic(const Problem& p, bool bf16_io, const Inputs& in,
                              const BwdGrads& g, const BwdWork& w, hipStream_t s) {
    const dim3 grid(p.B * p.N, p.H);
    const size_t lds = bwd_generic_lds_bytes(p);
    const int vmax = vmax_of(p);
    if (bf16_io) {
        hipLaunchKernelGGL(bwd_generic_kernel<bf16>, grid, dim3(256), lds, s, p,
                           (const bf16*)in.q_nope, (const bf16*)in.q_rope,
                           (const bf16*)in.ckv_ctx, (const bf16*)in.kr_ctx,
                           (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk,
                           (const bf16*)in.w_uk, (const bf16*)in.w_uv, (const bf16*)g.dout,
                           (bf16*)g.dq_nope, (bf16*)g.dq_rope, w.acc, w.wacc, w.fwd.idx,
                           w.fwd.rope, vmax);
    } else {
        hipLaunchKernelGGL(bwd_generic_kernel<float>, grid, dim3(256), lds, s, p,
                           (const float*)in.q_nope, (const float*)in.q_rope,
                           (const float*)in.ckv_ctx, (const float*)in.kr_ctx,
                           (const float*)in.ckv_blk, (const float*)in.kr_blk,
                           (const float*)in.w_uk, (const float*)in.w_uv, (const float*)g.dout,
                           (float*)g.dq_nope, (float*)g.dq_rope, w.acc, w.wacc, w.fwd.idx,
                           w.fwd.rope, vmax);
    }
    return hipGetLastError();
}

hipError_t launch_bwd_finalize(const Problem& p, bool bf16_io, const BwdGrads& g,
                               const BwdWork& w, const int4* idx, const float2* table,
                               const RopeTheta& th, bool weights, hipStream_t s) {
    // without a table the kernel evaluates the angles from turns, theta_i / 2pi
    RopeTheta turns{};
    for (int k = 0; k < p.dr / 2 && k < kMaxRopePairs; ++k)
        turns.t[k] = th.t[k] * 0.15915494309189533577;
    const size_t rows = (size_t)p.B * ((size_t)p.S + p.L5);
    const int grid = (int)(rows < 8192 ? (rows > 0 ? rows : 1) : 8192);
    if (bf16_io) {
        hipLaunchKernelGGL(bwd_finalize_kernel<bf16>, dim3(grid), dim3(256), 0, s, p, w.acc,
                           w.wacc, (bf16*)g.dckv_ctx, (bf16*)g.dkr_ctx, (bf16*)g.dckv_blk,
                           (bf16*)g.dkr_blk, (bf16*)g.dq_nope, (bf16*)g.dq_rope,
                           (bf16*)g.dw_uk, (bf16*)g.dw_uv, idx, table, turns, weights ? 1 : 0);
    } else {
        hipLaunchKernelGGL(bwd_finalize_kernel<float>, dim3(grid), dim3(256), 0, s, p, w.acc,
                           w.wacc, (float*)g.dckv_ctx, (float*)g.dkr_ctx, (float*)g.dckv_blk,
                           (float*)g.dkr_blk, (float*)g.dq_nope, (float*)g.dq_rope,
                           (float*)g.dw_uk, (float*)g.dw_uv, idx, table, turns,
                           weights ? 1 : 0);
    }
    return hipGetLastError();
}

}  // namespace dspark
