// W_UV up-projection: out[b, q, h, :] = W_UV[h] o_lat[r][h]  (512 -> 256) for
// every kept query row r, bf16 MFMA with fp32 accumulation.
//
// Design page §4 "MLA Projection": v_h = W_UV[h] c^KV; because the attention
// weights sum to one per row, sum_k p_k v_h(k) = W_UV[h] (sum_k p_k c^KV_k),
// so the value up-projection is applied once per (query, head) to o_lat.
//
// o_lat[r][h][512] (block-major) comes from the attention kernel with the latent dims
// permuted inside each 32-dim group (stored position 32k + 8g + s is dim
// 32k + 4g + s for s < 4, 32k + 16 + 4g + (s-4) for s >= 4); the weight
// fragments are read in the same order, two 8-byte pieces per lane.
//
// Work split: a workgroup owns one head, one half of the 256 output dims
// (a 128 x 512 weight slice resident in LDS, rows permuted) and a strided
// range of 128-row iterations; each wave computes 128 dims x 32 rows,
// transposed (dims x rows), and writes 8 consecutive output dims per lane.
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kUvRowGroups = 2;
constexpr int kUvStride = kD + 8;        // bf16 per LDS weight row (1040 B)
constexpr int kUvTiles = 2;             // 16-row tiles per wave and iteration
constexpr int kUvRowsPerIter = 4 * 16 * kUvTiles;

__global__ __launch_bounds__(256) void uv_kernel(const bf16* __restrict__ w_uv,
                                                 const bf16* __restrict__ o_lat,
                                                 const int32_t* __restrict__ kept,
                                                 const int32_t* __restrict__ status,
                                                 bf16* __restrict__ out, int N, int L5,
                                                 int slot0, int nslots) {
    __shared__ __attribute__((aligned(16))) bf16 wl[128 * kUvStride];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int vh = lid & 1;
    const int rg = (lid >> 1) % kUvRowGroups;
    const int h = (lid >> 1) / kUvRowGroups;
    const int tid = threadIdx.x;

    // LDS row R = 16 * vt + m of the slice holds output dim
    // 32 * (vt / 2) + 8 * (m / 4) + 4 * (vt % 2) + m % 4, so that after the
    // transposed MFMAs the lane with k-group g holds the 8 consecutive dims
    // 32p + 8g .. 32p + 8g + 7 of tile pair p and writes them as one 16-byte
    // store (4 lanes cover 64 contiguous bytes of a row).
    // one 1 KB weight row per wave instruction, straight into LDS
    {
        const int wave = tid >> 6, lane = tid & 63;
        for (int R = wave; R < 128; R += 4) {
            const int vt = R >> 4, m = R & 15;
            const int v = 32 * (vt >> 1) + 8 * (m >> 2) + 4 * (vt & 1) + (m & 3);
            async_copy_16(w_uv + ((size_t)h * kDv + vh * 128 + v) * kD + lane * 8,
                          &wl[R * kUvStride]);
        }
    }

    // rows of this chunk (kept slots [slot0, slot0 + nslots))
    const int rows = kBlock * max(0, min(nslots, status[kStKeptCount] - slot0));
    const int n_iter = (rows + kUvRowsPerIter - 1) / kUvRowsPerIter;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    if (rg >= n_iter) {
        __builtin_amdgcn_s_waitcnt(0);     // no LDS copy left in flight
        return;
    }

    auto row_of = [&](int it, int t) {
        const int r = it * kUvRowsPerIter + wave * 16 * kUvTiles + t * 16 + l16;
        return (r < rows) ? r : rows - 1;     // duplicate rows are computed, not stored
    };
    constexpr int kKs = kD / 32;     // 16 k-steps
    // A fragment (ks, vt): LDS rows 16 vt + l16, k-values in the permuted
    // o_lat order (dims 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3)
    auto a_frag = [&](int ks, int vt) -> bf16x8 {
        const bf16* ap = &wl[(vt * 16 + l16) * kUvStride + ks * 32 + g * 4];
        return cat(ld8(ap), ld8(ap + 16));
    };
    constexpr int kPf = 8;           // prefetch distance in k-steps (divides kKs)
    const bf16* op[kUvTiles];
    for (int t = 0; t < kUvTiles; ++t)
        op[t] = o_lat + ((size_t)(kBlock * slot0 + row_of(rg, t)) * kH + h) * kD + g * 8;
    bf16x8 ring[kPf][kUvTiles];
#pragma unroll
    for (int ks = 0; ks < kPf; ++ks)
#pragma unroll
        for (int t = 0; t < kUvTiles; ++t) ring[ks][t] = gld16(op[t] + ks * 32);
    // the weight copies and the first rows are in flight together
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Results of one iteration are stored at the start of the next one: the
    // loop then enters its header with the same kinds of memory operations in
    // flight from both sides, and the stores have the whole prefetch distance
    // to complete before any load issued after them is waited for.
    bf16x8 pend[kUvTiles][4];        // [row tile][tile pair]
    bf16* pdst[kUvTiles];
    auto compute = [&](int it) {
        __asm__ volatile("" ::: "memory");
        const int nxt = it + kUvRowGroups;
        const bf16* np[kUvTiles];
        for (int t = 0; t < kUvTiles; ++t)
            np[t] = o_lat + ((size_t)(kBlock * slot0 + row_of(nxt, t)) * kH + h) * kD + g * 8;
        int blk[kUvTiles];
        for (int t = 0; t < kUvTiles; ++t) blk[t] = kept[slot0 + row_of(it, t) / kBlock];

        f32x4 acc[8][kUvTiles];
#pragma unroll
        for (int vt = 0; vt < 8; ++vt)
#pragma unroll
            for (int t = 0; t < kUvTiles; ++t) acc[vt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // A fragments of k-step ks + 1 are read from LDS while the MFMAs of
        // k-step ks run; sched_barrier keeps the reads ahead of the MFMAs
        bf16x8 acur[8];
#pragma unroll
        for (int vt = 0; vt < 8; ++vt) acur[vt] = a_frag(0, vt);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            bf16x8 bo[kUvTiles];
#pragma unroll
            for (int t = 0; t < kUvTiles; ++t) bo[t] = ring[ks % kPf][t];
            // without a next iteration np points at the current rows: the
            // loads stay unconditional so that the wait counts stay exact
            if (ks + kPf < kKs) {
#pragma unroll
                for (int t = 0; t < kUvTiles; ++t) ring[ks % kPf][t] = gld16(op[t] + (ks + kPf) * 32);
            } else {
#pragma unroll
                for (int t = 0; t < kUvTiles; ++t) ring[ks % kPf][t] = gld16(np[t] + (ks + kPf - kKs) * 32);
            }
            bf16x8 anext[8];
            if (ks + 1 < kKs) {
#pragma unroll
                for (int vt = 0; vt < 8; ++vt) anext[vt] = a_frag(ks + 1, vt);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int vt = 0; vt < 8; ++vt)
#pragma unroll
                for (int t = 0; t < kUvTiles; ++t) acc[vt][t] = mfma_16x16x32(acur[vt], bo[t], acc[vt][t]);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kKs) {
#pragma unroll
                for (int vt = 0; vt < 8; ++vt) acur[vt] = anext[vt];
            }
        }
#pragma unroll
        for (int t = 0; t < kUvTiles; ++t) {
            // rows past the end repeat the last row (same values, same place)
            const int r = row_of(it, t);
            const int j = r % kBlock;
            const int b = blk[t] / N, n = blk[t] % N;
            pdst[t] = out + (((size_t)b * L5 + (size_t)kBlock * n + j) * kH + h) * kDv +
                      vh * 128 + g * 8;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                bf16x8 v;
                v[0] = (bf16)a0[0]; v[1] = (bf16)a0[1]; v[2] = (bf16)a0[2]; v[3] = (bf16)a0[3];
                v[4] = (bf16)a1[0]; v[5] = (bf16)a1[1]; v[6] = (bf16)a1[2]; v[7] = (bf16)a1[3];
                pend[t][pp] = v;
            }
        }
        for (int t = 0; t < kUvTiles; ++t) op[t] = np[t];
    };
    auto flush = [&]() {
#pragma unroll
        for (int t = 0; t < kUvTiles; ++t)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) gst16(pdst[t] + pp * 32, pend[t][pp]);
    };

    compute(rg);
    for (int it = rg + kUvRowGroups; it < n_iter; it += kUvRowGroups) {
        flush();
        compute(it);
    }
    flush();
}

}  // namespace

hipError_t launch_uv(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                     hipStream_t s) {
    const int grid = kH * 2 * kUvRowGroups;
    hipLaunchKernelGGL(uv_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)in.w_uv, ws.olat,
                       ws.kept, ws.status, (bf16*)in.out, p.N, p.L5, c.slot0,
                       c.nslots);
    return hipGetLastError();
}

}  // namespace dspark
