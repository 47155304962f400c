// Generic DSpark draft-attention forward: any dims, fp32 arithmetic, fp32 or
// bf16 storage.  One workgroup per (block, head).  It follows the absorbed
// latent form (q_abs = W_UK[h]^T q^C; scores over c^KV and rotated k^R;
// o_lat = P c^KV; out = W_UV[h] o_lat), which equals the expanded form of the
// design page's §4 "MLA Projection" exactly in real arithmetic.
//
// Used for the small fp32 configuration and for shapes outside the MFMA fast
// path; it is not tuned.
#include "kernels.hpp"

namespace dspark {

namespace {

template <typename T> __device__ inline float ldf(const T* p, size_t i);
template <> __device__ inline float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ldf<bf16>(const bf16* p, size_t i) { return (float)p[i]; }
template <typename T> __device__ inline void stf(T* p, size_t i, float v);
template <> __device__ inline void stf<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ inline void stf<bf16>(bf16* p, size_t i, float v) { p[i] = (bf16)v; }

template <typename T>
__global__ __launch_bounds__(256) void generic_kernel(Problem p, const T* __restrict__ q_nope,
                                                      const T* __restrict__ q_rope,
                                                      const T* __restrict__ ckv_ctx,
                                                      const T* __restrict__ kr_ctx,
                                                      const T* __restrict__ ckv_blk,
                                                      const T* __restrict__ kr_blk,
                                                      const T* __restrict__ w_uk,
                                                      const T* __restrict__ w_uv, T* __restrict__ out,
                                                      const int4* __restrict__ idx,
                                                      const float2* __restrict__ rope, int vmax) {
    extern __shared__ float sm[];
    const int blk = blockIdx.x;            // b * N + n
    const int h = blockIdx.y;
    const int b = blk / p.N, n = blk % p.N;
    const int tid = threadIdx.x;
    const int D = p.D, dr = p.dr, pairs = p.dr / 2;
    const int4 rec = idx[blk];
    const size_t qrow0 = (size_t)b * p.L5 + (size_t)kBlock * n;   // first query row of the block

    if (rec.w < 0) {   // padding block -> 0; kept block with a bad anchor -> NaN
        const float fill = (rec.w == -1) ? 0.0f : __builtin_nanf("");
        for (int e = tid; e < kBlock * p.dv; e += blockDim.x) {
            const int j = e / p.dv, v = e % p.dv;
            stf(out, ((qrow0 + j) * p.H + h) * p.dv + v, fill);
        }
        return;
    }
    const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z;
    const int nkeys = ctx_len + kBlock;

    float* qa = sm;                          // [5][D]   q_abs
    float* qr = qa + kBlock * D;             // [5][dr]  rotated q^R
    float* sc = qr + kBlock * dr;            // [5][vmax] scores, then weights
    float* ol = sc + kBlock * vmax;          // [5][D]   o_lat
    float* inv = ol + kBlock * D;            // [5]      1 / row sum

    // q_abs[j][d] = sum_c q^C[j][c] W_UK[h][c][d]
    for (int e = tid; e < kBlock * D; e += blockDim.x) {
        const int j = e / D, d = e % D;
        const size_t qo = ((qrow0 + j) * p.H + h) * p.dc;
        float acc = 0.f;
        for (int c = 0; c < p.dc; ++c)
            acc += ldf(q_nope, qo + c) * ldf(w_uk, ((size_t)h * p.dc + c) * D + d);
        qa[e] = acc;
    }
    // rotated q^R at position A + j
    for (int e = tid; e < kBlock * pairs; e += blockDim.x) {
        const int j = e / pairs, i = e % pairs;
        const size_t qo = ((qrow0 + j) * p.H + h) * dr;
        const float x0 = ldf(q_rope, qo + 2 * i), x1 = ldf(q_rope, qo + 2 * i + 1);
        const float2 cs = rope[(size_t)(pos0 + j) * pairs + i];
        qr[j * dr + 2 * i] = x0 * cs.x - x1 * cs.y;
        qr[j * dr + 2 * i + 1] = x0 * cs.y + x1 * cs.x;
    }
    __syncthreads();

    // scores over the visible keys: slot s < ctx_len is context row ctx_lo + s,
    // the rest are the block's own 5 positions
    for (int e = tid; e < kBlock * nkeys; e += blockDim.x) {
        const int j = e / nkeys, s = e % nkeys;
        const bool is_ctx = s < ctx_len;
        const size_t krow = is_ctx ? ((size_t)b * p.S + ctx_lo + s) : (qrow0 + (s - ctx_len));
        const T* ckv = is_ctx ? ckv_ctx : ckv_blk;
        const T* kr = is_ctx ? kr_ctx : kr_blk;
        const int pos = is_ctx ? ctx_lo + s : pos0 + (s - ctx_len);
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += qa[j * D + d] * ldf(ckv, krow * D + d);
        for (int i = 0; i < pairs; ++i) {
            const float x0 = ldf(kr, krow * dr + 2 * i), x1 = ldf(kr, krow * dr + 2 * i + 1);
            const float2 cs = rope[(size_t)pos * pairs + i];
            acc += qr[j * dr + 2 * i] * (x0 * cs.x - x1 * cs.y) +
                   qr[j * dr + 2 * i + 1] * (x0 * cs.y + x1 * cs.x);
        }
        sc[j * vmax + s] = acc * p.scale;
    }
    __syncthreads();
    if (tid < kBlock) {
        float m = -INFINITY;
        for (int s = 0; s < nkeys; ++s) m = fmaxf(m, sc[tid * vmax + s]);
        float sum = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            const float w = expf(sc[tid * vmax + s] - m);
            sc[tid * vmax + s] = w;
            sum += w;
        }
        inv[tid] = 1.0f / sum;
    }
    __syncthreads();
    for (int e = tid; e < kBlock * D; e += blockDim.x) {
        const int j = e / D, d = e % D;
        float acc = 0.f;
        for (int s = 0; s < nkeys; ++s) {
            const bool is_ctx = s < ctx_len;
            const size_t krow = is_ctx ? ((size_t)b * p.S + ctx_lo + s) : (qrow0 + (s - ctx_len));
            acc += sc[j * vmax + s] * ldf(is_ctx ? ckv_ctx : ckv_blk, krow * D + d);
        }
        ol[e] = acc * inv[j];
    }
    __syncthreads();
    for (int e = tid; e < kBlock * p.dv; e += blockDim.x) {
        const int j = e / p.dv, v = e % p.dv;
        float acc = 0.f;
        for (int d = 0; d < D; ++d) acc += ldf(w_uv, ((size_t)h * p.dv + v) * D + d) * ol[j * D + d];
        stf(out, ((qrow0 + j) * p.H + h) * p.dv + v, acc);
    }
}

int generic_vmax(const Problem& p) {
    const int ctx_max = (p.W - 1 < p.S - 2) ? p.W - 1 : (p.S - 2 > 0 ? p.S - 2 : 0);
    return ctx_max + kBlock;
}

}  // namespace

size_t generic_lds_bytes(const Problem& p) {
    const size_t vmax = (size_t)generic_vmax(p);
    return sizeof(float) * ((size_t)kBlock * (2 * (size_t)p.D + p.dr + vmax) + kBlock);
}

hipError_t launch_generic(const Problem& p, bool bf16_io, const Inputs& in, const Workspace& ws,
                          hipStream_t s) {
    const dim3 grid(p.B * p.N, p.H);
    const size_t lds = generic_lds_bytes(p);
    const int vmax = generic_vmax(p);
    if (bf16_io) {
        hipLaunchKernelGGL(generic_kernel<bf16>, grid, dim3(256), lds, s, p,
                           (const bf16*)in.q_nope, (const bf16*)in.q_rope, (const bf16*)in.ckv_ctx,
                           (const bf16*)in.kr_ctx, (const bf16*)in.ckv_blk, (const bf16*)in.kr_blk,
                           (const bf16*)in.w_uk, (const bf16*)in.w_uv, (bf16*)in.out, ws.idx,
                           ws.rope, vmax);
    } else {
        hipLaunchKernelGGL(generic_kernel<float>, grid, dim3(256), lds, s, p,
                           (const float*)in.q_nope, (const float*)in.q_rope,
                           (const float*)in.ckv_ctx, (const float*)in.kr_ctx,
                           (const float*)in.ckv_blk, (const float*)in.kr_blk,
                           (const float*)in.w_uk, (const float*)in.w_uv, (float*)in.out, ws.idx,
                           ws.rope, vmax);
    }
    return hipGetLastError();
}

}  // namespace dspark
