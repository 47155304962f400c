// Absorb: q_abs[h][r] = W_UK[h]^T q^C[r, h]  (192 -> 512) for every kept
// query row r, bf16 MFMA with fp32 accumulation.
//
// Absorption is the identity q^C . (W_UK[h] c) = (W_UK[h]^T q^C) . c (design
// page §4 "MLA Projection": k^C_h = W_UK[h] c^KV), so the attention can score
// the 512 cached latent numbers directly.
//
// Output layout (consumed by the attention kernel): q_abs[h][r][512] bf16 with
// the latent dims permuted inside every 32-dim group: stored position
// 32*k + 8*g + s holds dim 32*k + 4*g + s for s < 4 and 32*k + 16 + 4*g + (s-4)
// for s >= 4.  That is exactly what one lane of a 16x16 MFMA output tile pair
// holds, and the attention kernel reads c^KV in the same order.
//
// Work split: a workgroup owns one head, one half of the 512 output dims and
// a strided range of 128-row iterations.  The 192 x 256 weight slice stays in
// LDS for the workgroup's lifetime; its transposed MFMA fragments are read
// with ds_read_b64_tr_b16.  Each wave computes 128 dims x 64 rows.
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kAbsRowGroups = 2;        // workgroups per (head, dim half)
constexpr int kAbsStride = 256 + 16;    // LDS row stride (bf16) of the weight slice
constexpr int kAbsRowsPerIter = 128;

__global__ __launch_bounds__(256) void absorb_kernel(const bf16* __restrict__ q_nope,
                                                     const bf16* __restrict__ w_uk,
                                                     const int32_t* __restrict__ kept,
                                                     const int32_t* __restrict__ status,
                                                     bf16* __restrict__ q_abs, int N, int L5,
                                                     int rows_max) {
    __shared__ __attribute__((aligned(16))) bf16 wl[kDc * kAbsStride];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int dh = lid & 1;
    const int rg = (lid >> 1) % kAbsRowGroups;
    const int h = (lid >> 1) / kAbsRowGroups;
    const int tid = threadIdx.x;

    // weight slice W_UK[h][0:192][dh*256 : dh*256+256]
    for (int e = tid; e < kDc * 32; e += 256) {
        const int c = e >> 5, ch = e & 31;
        st16(&wl[c * kAbsStride + ch * 8],
             ld16(w_uk + ((size_t)h * kDc + c) * kD + dh * 256 + ch * 8));
    }
    __syncthreads();

    const int rows = kBlock * status[kStKeptCount];
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int wd = wave & 1;      // 128-dim quarter inside the half
    const int wr = wave >> 1;     // 64-row group inside the iteration

    for (int it = rg; it * kAbsRowsPerIter < rows; it += kAbsRowGroups) {
        const int row0 = it * kAbsRowsPerIter + wr * 64;
        const bf16* qp[4];
        for (int t = 0; t < 4; ++t) {
            int r = row0 + t * 16 + l16;
            r = (r < rows) ? r : rows - 1;
            const int slot = r / kBlock, j = r % kBlock;
            const int blk = kept[slot];
            const int b = blk / N, n = blk % N;
            qp[t] = q_nope + (((size_t)b * L5 + (size_t)kBlock * n + j) * kH + h) * kDc + g * 8;
        }
        f32x4 acc[8][4];
        for (int dt = 0; dt < 8; ++dt)
            for (int t = 0; t < 4; ++t) acc[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int ks = 0; ks < kDc / 32; ++ks) {
            bf16x8 bq[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bq[t] = ld16(qp[t] + ks * 32);
            // A fragment rows: dims wd*128 + dt*16 + l16; k-values c = ks*32 + g*8 + 0..7
            const bf16* abase = wl + (ks * 32 + g * 8 + (l16 >> 2)) * kAbsStride + wd * 128 +
                                (l16 & 3) * 4;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const bf16x4 lo = lds_read_tr(abase + dt * 16);
                const bf16x4 hi = lds_read_tr(abase + 4 * kAbsStride + dt * 16);
                const bf16x8 af = cat(lo, hi);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[dt][t] = mfma_16x16x32(af, bq[t], acc[dt][t]);
            }
        }
        // lane holds dims dcol + 4g + i of tile pair (2p, 2p+1) for row row0 + 16t + l16
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = row0 + t * 16 + l16;
            if (r >= rows) continue;
            bf16* dst = q_abs + ((size_t)h * rows_max + r) * kD + dh * 256 + wd * 128 + g * 8;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                bf16x8 v;
                v[0] = (bf16)a0[0]; v[1] = (bf16)a0[1]; v[2] = (bf16)a0[2]; v[3] = (bf16)a0[3];
                v[4] = (bf16)a1[0]; v[5] = (bf16)a1[1]; v[6] = (bf16)a1[2]; v[7] = (bf16)a1[3];
                st16(dst + pp * 32, v);
            }
        }
    }
}

}  // namespace

hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, hipStream_t s) {
    const int grid = kH * 2 * kAbsRowGroups;
    hipLaunchKernelGGL(absorb_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)in.q_nope,
                       (const bf16*)in.w_uk, ws.kept, ws.status, ws.qabs, p.N, p.L5, p.rows_max);
    return hipGetLastError();
}

}  // namespace dspark
