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
// with ds_read_b64_tr_b16 one k-step ahead of their use.  Each wave computes
// 128 dims x 64 rows per iteration and keeps a whole iteration of q^C rows in
// flight.
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
                                                     int lat_rows, int slot0, int nslots) {
    __shared__ __attribute__((aligned(16))) bf16 wl[kDc * kAbsStride];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int dh = lid & 1;
    const int rg = (lid >> 1) % kAbsRowGroups;
    const int h = (lid >> 1) / kAbsRowGroups;
    const int tid = threadIdx.x;

    // weight slice W_UK[h][0:192][dh*256 : dh*256+256]
    // one 512-byte weight row per half-wave instruction, straight into LDS
    {
        const int wave = tid >> 6, lane = tid & 63;
        const int half = lane >> 5;
        for (int c0 = 2 * wave; c0 < kDc; c0 += 8) {
            const int c = c0 + half;
            if (half == 0)
                async_copy_16(w_uk + ((size_t)h * kDc + c) * kD + dh * 256 + lane * 8,
                              &wl[c0 * kAbsStride]);
            else
                async_copy_16(w_uk + ((size_t)h * kDc + c) * kD + dh * 256 + (lane - 32) * 8,
                              &wl[c0 * kAbsStride + kAbsStride - 256]);
        }
        __builtin_amdgcn_s_waitcnt(0);     // the LDS copies are counted by vmcnt
    }
    __syncthreads();

    // rows of this chunk: kept slots [slot0, slot0 + nslots); local row r is
    // query r % 5 of slot slot0 + r / 5
    const int rows = kBlock * max(0, min(nslots, status[kStKeptCount] - slot0));
    const int n_iter = (rows + kAbsRowsPerIter - 1) / kAbsRowsPerIter;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int wd = wave & 1;      // 128-dim quarter inside the half
    const int wr = wave >> 1;     // 64-row group inside the iteration
    if (rg >= n_iter) return;

    // row r of iteration `it`, tile t (clamped; rows past the end are computed
    // on a duplicate row and not stored)
    auto row_of = [&](int it, int t) {
        const int r = it * kAbsRowsPerIter + wr * 64 + t * 16 + l16;
        return (r < rows) ? r : rows - 1;
    };
    auto q_ptr = [&](int r, int blk) {
        const int j = r % kBlock;
        const int b = blk / N, n = blk % N;
        return q_nope + (((size_t)b * L5 + (size_t)kBlock * n + j) * kH + h) * kDc + g * 8;
    };
    constexpr int kKs = kDc / 32;     // 6 k-steps per iteration

    // A operand (the wave's 128 x 192 slice of W_UK[h]^T): fragment (ks, dt)
    // holds rows d = wd*128 + dt*16 + l16 and k-values c = ks*32 + g*8 + 0..7,
    // read transposed out of the [c][d] LDS slice with ds_read_b64_tr_b16.
    auto a_frag = [&](int ks, int dt) -> bf16x8 {
        const bf16* abase = wl + (ks * 32 + g * 8 + (l16 >> 2)) * kAbsStride + wd * 128 +
                            (l16 & 3) * 4 + dt * 16;
        return cat(lds_read_tr(abase), lds_read_tr(abase + 4 * kAbsStride));
    };

    // B fragments: a ring of kPf k-steps (one whole iteration); consuming
    // k-step ks frees slot ks % kPf, which is refilled with the same k-step
    // of the next iteration.
    constexpr int kPf = kKs;
    bf16x8 ring[kPf][4];
    const bf16* qp[4];
    int blk_next[4];
    for (int t = 0; t < 4; ++t) {
        const int r = row_of(rg, t);
        qp[t] = q_ptr(r, kept[slot0 + r / kBlock]);
    }
#pragma unroll
    for (int ks = 0; ks < kPf; ++ks)
#pragma unroll
        for (int t = 0; t < 4; ++t) ring[ks][t] = gld16(qp[t] + ks * 32);
    for (int t = 0; t < 4; ++t) blk_next[t] = kept[slot0 + row_of(rg + kAbsRowGroups, t) / kBlock];

    // The loop body is branch-free so that the compiler's wait counts stay
    // exact across iterations: past the last iteration the prefetches and
    // kept-list reads re-read clamped (valid) rows, and rows past the end are
    // computed on a duplicate of the last row and stored onto it (same value).
    // Results of one iteration are stored at the start of the next one, so
    // that the loop header sees the same operations in flight from both sides
    // and no wait for a prefetched row also waits for fresh stores.
    bf16x8 pend[4][4];
    bf16* pdst[4];
    auto compute = [&](int it) {
        __asm__ volatile("" ::: "memory");
        const int nxt = it + kAbsRowGroups;
        const bf16* np[4];
        for (int t = 0; t < 4; ++t) np[t] = q_ptr(row_of(nxt, t), blk_next[t]);
        for (int t = 0; t < 4; ++t) blk_next[t] = kept[slot0 + row_of(nxt + kAbsRowGroups, t) / kBlock];
        f32x4 acc[8][4];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 acur[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acur[dt] = a_frag(0, dt);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            bf16x8 bq[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bq[t] = ring[ks][t];
#pragma unroll
            for (int t = 0; t < 4; ++t) ring[ks][t] = gld16(np[t] + ks * 32);
            bf16x8 anext[8];
            if (ks + 1 < kKs) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) anext[dt] = a_frag(ks + 1, dt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[dt][t] = mfma_16x16x32(acur[dt], bq[t], acc[dt][t]);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kKs) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acur[dt] = anext[dt];
            }
        }
        // lane holds dims dcol + 4g + i of tile pair (2p, 2p+1) for row it*128 + wr*64 + 16t + l16
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = row_of(it, t);
            pdst[t] = q_abs + ((size_t)h * lat_rows + r) * kD + dh * 256 + wd * 128 + g * 8;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                bf16x8 v;
                v[0] = (bf16)a0[0]; v[1] = (bf16)a0[1]; v[2] = (bf16)a0[2]; v[3] = (bf16)a0[3];
                v[4] = (bf16)a1[0]; v[5] = (bf16)a1[1]; v[6] = (bf16)a1[2]; v[7] = (bf16)a1[3];
                pend[t][pp] = v;
            }
        }
    };
    auto flush = [&]() {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) gst16(pdst[t] + pp * 32, pend[t][pp]);
    };

    compute(rg);
    for (int it = rg + kAbsRowGroups; it < n_iter; it += kAbsRowGroups) {
        flush();
        compute(it);
    }
    flush();
}

}  // namespace

hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                         hipStream_t s) {
    const int grid = kH * 2 * kAbsRowGroups;
    hipLaunchKernelGGL(absorb_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)in.q_nope,
                       (const bf16*)in.w_uk, ws.kept, ws.status, ws.qabs, p.N, p.L5, p.lat_rows,
                       c.slot0, c.nslots);
    return hipGetLastError();
}

}  // namespace dspark
