// Absorb: q_abs[r][h] = W_UK[h]^T q^C[r, h]  (192 -> 512) for every kept
// query row r, bf16 MFMA with fp32 accumulation.
//
// Absorption is the identity q^C . (W_UK[h] c) = (W_UK[h]^T q^C) . c (design
// page §4 "MLA Projection": k^C_h = W_UK[h] c^KV), so the attention can score
// the 512 cached latent numbers directly.
//
// Output layout (consumed by the attention kernel): q_abs[r][h][512] bf16
// (block-major: the 5 rows x 64 heads of a kept block are contiguous), with
// the latent dims permuted inside every 32-dim group: stored position
// 32*k + 8*g + s holds dim 32*k + 4*g + s for s < 4 and 32*k + 16 + 4*g + (s-4)
// for s >= 4.  That is exactly what one lane of a 16x16 MFMA output tile pair
// holds, and the attention kernel reads c^KV in the same order.
//
// Work split: a workgroup owns one head, one half of the 512 output dims and
// a strided range of 128-row iterations.  The 192 x 256 weight slice stays in
// LDS for the workgroup's lifetime; its transposed MFMA fragments are read
// with ds_read_b64_tr_b16 one k-step ahead of their use.  Each wave computes
// 128 dims x 64 rows per iteration.  The q^C rows of an iteration are copied
// into LDS once per workgroup (LDS DMA, laid out as MFMA B fragments) and
// read by both waves that need them; the copy for the next iteration runs
// while the current one computes.  Results are transposed through LDS so
// that each store instruction writes 4 rows x 256 B of q_abs: with 16 rows x
// 64 B per instruction (the MFMA tile layout) the stores ran ~20% slower.
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kAbsRowGroups = 2;        // workgroups per (head, dim half)
constexpr int kAbsStride = 256 + 16;    // LDS row stride (bf16) of the weight slice
constexpr int kAbsTiles = 4;                         // 16-row tiles per wave and iteration
constexpr int kAbsRowsPerIter = 2 * 16 * kAbsTiles;  // two row groups per workgroup
constexpr int kAbsCopyTiles = 2 * kAbsTiles / 4;     // tiles each wave copies per iteration

constexpr int kAbsKs = kDc / 32;                        // 6 k-steps
constexpr int kAbsFrags = (kAbsRowsPerIter / 16) * kAbsKs;  // B fragments per iteration

__global__ __launch_bounds__(256) void absorb_kernel(const bf16* __restrict__ q_nope,
                                                     const bf16* __restrict__ w_uk,
                                                     const int32_t* __restrict__ kept,
                                                     const int32_t* __restrict__ status,
                                                     bf16* __restrict__ q_abs, int N, int L5,
                                                     int slot0, int nslots,
                                                     uint32_t q_bytes) {
    __shared__ __attribute__((aligned(16))) bf16 wl[kDc * kAbsStride];
    // B fragments of one iteration: [row tile][k-step][lane][8]
    __shared__ __attribute__((aligned(16))) bf16 qs[kAbsFrags * 512];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int dh = lid & 1;
    const int rg = (lid >> 1) % kAbsRowGroups;
    const int h = (lid >> 1) / kAbsRowGroups;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    // weight slice W_UK[h][0:192][dh*256 : dh*256+256]
    // one 512-byte weight row per half-wave instruction, straight into LDS
    {
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
    }

    // rows of this chunk: kept slots [slot0, slot0 + nslots); local row r is
    // query r % 5 of slot slot0 + r / 5
    const int rows = kBlock * max(0, min(nslots, status[kStKeptCount] - slot0));
    const int n_iter = (rows + kAbsRowsPerIter - 1) / kAbsRowsPerIter;
    const int wd = wave & 1;      // 128-dim quarter inside the half
    const int wr = wave >> 1;     // row group inside the iteration
    if (rg >= n_iter) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);   // no LDS copy left in flight
        return;
    }

    auto clamp_row = [&](int r) { return (r < rows) ? r : rows - 1; };
    auto q_ptr = [&](int r, int blk) {
        const int j = r % kBlock;
        const int b = blk / N, n = blk % N;
        return q_nope + (((size_t)b * L5 + (size_t)kBlock * n + j) * kH + h) * kDc + g * 8;
    };
    // Copy side: this wave copies row tiles kAbsCopyTiles*wave + u of an
    // iteration (all k-steps).  Rows past the end copy the last row.
    auto copy_row = [&](int it, int u) {
        return clamp_row(it * kAbsRowsPerIter + (kAbsCopyTiles * wave + u) * 16 + l16);
    };
    const __amdgpu_buffer_rsrc_t q_rsrc = buffer_rsrc(q_nope, q_bytes);
    auto stage = [&](int it, const int* blk) {
#pragma unroll
        for (int u = 0; u < kAbsCopyTiles; ++u) {
            const uint32_t off = (uint32_t)((q_ptr(copy_row(it, u), blk[u]) - q_nope) * 2);
#pragma unroll
            for (int ks = 0; ks < kAbsKs; ++ks)
                buffer_copy_16(q_rsrc, off + ks * 64,
                               &qs[((kAbsCopyTiles * wave + u) * kAbsKs + ks) * 512]);
        }
    };
    int cblk[kAbsCopyTiles];
    for (int u = 0; u < kAbsCopyTiles; ++u) cblk[u] = kept[slot0 + copy_row(rg, u) / kBlock];
    stage(rg, cblk);
    for (int u = 0; u < kAbsCopyTiles; ++u)
        cblk[u] = kept[slot0 + copy_row(rg + kAbsRowGroups, u) / kBlock];

    // A operand (the wave's 128 x 192 slice of W_UK[h]^T): fragment (ks, dt)
    // holds rows d = wd*128 + dt*16 + l16 and k-values c = ks*32 + g*8 + 0..7,
    // read transposed out of the [c][d] LDS slice with ds_read_b64_tr_b16.
    auto a_frag = [&](int ks, int dt) -> bf16x8 {
        const bf16* abase = wl + (ks * 32 + g * 8 + (l16 >> 2)) * kAbsStride + wd * 128 +
                            (l16 & 3) * 4 + dt * 16;
        return cat(lds_read_tr(abase), lds_read_tr(abase + 4 * kAbsStride));
    };

    // Per iteration: wait for this iteration's copy (issued one iteration
    // earlier), read the wave's B fragments into registers, store the
    // previous iteration's results, start the next copy, then compute.
    // Everything waited for at the top of an iteration was issued before the
    // previous iteration's MFMAs.
    //
    // Results leave through LDS while the q^C buffer is free (after the
    // B-fragment reads, before the next copy): each wave writes its rows
    // there as they sit in the MFMA tiles (16 rows per instruction), reads
    // them back as 4 rows x 256 B per instruction and stores those, so that
    // a store instruction touches 4 rows of q_abs instead of 16.
    constexpr int kEpiStride = 256 + 16;      // bytes per row (16 B pad: no bank conflicts)
    constexpr int kEpiRows = 32;              // rows per pass (two row tiles)
    static_assert(4 * kEpiRows * kEpiStride <= (int)sizeof(qs), "epilogue area");
    char* const epi = reinterpret_cast<char*>(qs) + wave * kEpiRows * kEpiStride;
    bf16x8 pend[kAbsTiles][4];
    int prow0 = 0;        // chunk-local row of the wave's first pending result
    auto flush = [&]() {
#pragma unroll
        for (int hf = 0; hf < kAbsTiles / 2; ++hf) {
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int pp = 0; pp < 4; ++pp)
                    *reinterpret_cast<bf16x8*>(epi + (t2 * 16 + l16) * kEpiStride +
                                               (pp * 4 + g) * 16) = pend[2 * hf + t2][pp];
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            bf16x8 w[kEpiRows / 4];
#pragma unroll
            for (int j = 0; j < kEpiRows / 4; ++j)
                w[j] = *reinterpret_cast<const bf16x8*>(epi + (4 * j + (lane >> 4)) * kEpiStride +
                                                        (lane & 15) * 16);
#pragma unroll
            for (int j = 0; j < kEpiRows / 4; ++j) {
                const int r = clamp_row(prow0 + hf * kEpiRows + 4 * j + (lane >> 4));
                gst16(q_abs + ((size_t)(kBlock * slot0 + r) * kH + h) * kD + dh * 256 + wd * 128 +
                          (lane & 15) * 8,
                      w[j]);
            }
        }
    };
    for (int it = rg; it < n_iter; it += kAbsRowGroups) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        bf16x8 bq[kAbsKs][kAbsTiles];
#pragma unroll
        for (int ks = 0; ks < kAbsKs; ++ks)
#pragma unroll
            for (int t = 0; t < kAbsTiles; ++t)
                bq[ks][t] = ld16(&qs[((wr * kAbsTiles + t) * kAbsKs + ks) * 512 + lane * 8]);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __syncthreads();
        if (it != rg) {
            flush();
            __syncthreads();   // every wave is done with its part of the buffer
        }
        stage(it + kAbsRowGroups, cblk);
        for (int u = 0; u < kAbsCopyTiles; ++u)
            cblk[u] = kept[slot0 + copy_row(it + 2 * kAbsRowGroups, u) / kBlock];

        f32x4 acc[8][kAbsTiles];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int t = 0; t < kAbsTiles; ++t) acc[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // A fragments of k-step ks + 1 are read in two halves, each while 16
        // MFMAs of k-step ks run, so that at most 8 LDS reads (16 counted
        // operations would overflow lgkmcnt) separate a fragment from its use.
        bf16x8 acur[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acur[dt] = a_frag(0, dt);
#pragma unroll
        for (int ks = 0; ks < kAbsKs; ++ks) {
            bf16x8 anext[8];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int dt = 4 * hf; dt < 4 * hf + 4; ++dt)
#pragma unroll
                    for (int t = 0; t < kAbsTiles; ++t)
                        acc[dt][t] = mfma_16x16x32(acur[dt], bq[ks][t], acc[dt][t]);
                __builtin_amdgcn_sched_barrier(0);
                if (ks + 1 < kAbsKs) {
#pragma unroll
                    for (int dt = 4 * hf; dt < 4 * hf + 4; ++dt) anext[dt] = a_frag(ks + 1, dt);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kAbsKs) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acur[dt] = anext[dt];
            }
        }
        // lane holds dims dcol + 4g + i of tile pair (2p, 2p+1) for row
        // it*rows_per_iter + (wr*kAbsTiles + t)*16 + l16; rows past the end
        // repeat the last row (same values, same place)
        prow0 = it * kAbsRowsPerIter + wr * kAbsTiles * 16;
#pragma unroll
        for (int t = 0; t < kAbsTiles; ++t) {
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                bf16x8 v;
                v[0] = (bf16)a0[0]; v[1] = (bf16)a0[1]; v[2] = (bf16)a0[2]; v[3] = (bf16)a0[3];
                v[4] = (bf16)a1[0]; v[5] = (bf16)a1[1]; v[6] = (bf16)a1[2]; v[7] = (bf16)a1[3];
                pend[t][pp] = v;
            }
        }
    }
    // the copy started by the last iteration is not used; it must land
    // before the buffer holds the last results
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    flush();
}

}  // namespace

hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                         hipStream_t s) {
    const int grid = kH * 2 * kAbsRowGroups;
    hipLaunchKernelGGL(absorb_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)in.q_nope,
                       (const bf16*)in.w_uk, ws.kept, ws.status, ws.qabs, p.N, p.L5,
                       c.slot0, c.nslots,
                       (uint32_t)((size_t)p.B * p.L5 * kH * kDc * sizeof(bf16)));
    return hipGetLastError();
}

}  // namespace dspark
