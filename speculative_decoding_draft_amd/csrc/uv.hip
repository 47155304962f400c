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
// The same kernel, with 192 output dims and 6 waves, computes the
// backward's dq^C[r][h] = W_UK[h] dq_abs[r][h] (512 -> 192): dq_abs has
// o_lat's layout and W_UK[h] W_UV[h]'s.
//
// Work split: a workgroup (8 waves, two per SIMD) owns one head and a
// strided range of 32-row iterations; wave w computes output dims
// 32w .. 32w+31, transposed (dims x rows), with its 32 x 512 slice of
// W_UV[h] resident in registers (staged through LDS at start).  One workgroup covering all 256 dims reads
// every o_lat row once: splitting the dims over two workgroups made both
// read it (the second read hits L2, but a read-only probe of this pattern
// takes 47 us with two readers against 36 with one).  The o_lat rows of an iteration
// are copied into LDS one 1 KB row per instruction (LDS DMA) through a ring
// of four slots, three iterations ahead of their use, and every wave reads
// its B fragments from there.  Results are transposed through LDS and
// stored as 4 rows x 256 B per instruction.  Reading o_lat as MFMA
// fragments straight from memory (16 rows x 64 B per instruction) and
// storing in the tile layout made this kernel ~30% slower.
#include <algorithm>

#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kUvRowGroups = 4;               // workgroups per head
constexpr int kUvRows = 32;                   // o_lat rows per iteration
constexpr int kUvLdsStride = kD * 2 + 16;     // bytes per staged o_lat row (pad: no bank conflicts)
constexpr int kUvSlot = kUvRows * kUvLdsStride;
constexpr int kUvKs = kD / 32;                // 16 k-steps

// Shape of the kernel for DOUT output dims: one wave per 32 dims.  A wave
// issues kCopies o_lat row copies and kStores output stores (two rows each)
// per iteration; where the waves do not divide the 32 rows (or 16 stores)
// evenly, the last indices repeat the last row: the same bytes to the same
// place.
template <int DOUT>
struct UvCfg {
    static constexpr int kWaves = DOUT / 32;
    static constexpr int kCopies = (kUvRows + kWaves - 1) / kWaves;
    static constexpr int kStores = (kUvRows / 2 + kWaves - 1) / kWaves;
    static constexpr int kEpiStride = DOUT * 2 + 16;    // bytes per row of the output transpose
    static constexpr int kHalf = DOUT / 2;              // weight rows staged per half
    static_assert(DOUT % 64 == 0 && kHalf <= 4 * kUvRows && kHalf % kWaves == 0, "uv shape");
};

template <int DOUT>
__global__ __launch_bounds__(DOUT / 32 * 64) void uv_kernel(const bf16* __restrict__ w_uv,
                                                 const bf16* __restrict__ o_lat,
                                                 const int32_t* __restrict__ kept,
                                                 const int32_t* __restrict__ status,
                                                 bf16* __restrict__ out, int N, int L5,
                                                 int slot0, int nslots,
                                                 const int32_t* __restrict__ anchors,
                                                 const uint8_t* __restrict__ keep, int S,
                                                 int total_blocks, int n_fill) {
    using C = UvCfg<DOUT>;
    // the last n_fill workgroups (dispatched after the others, so they run in
    // the launch's tail) write the rows of padding / invalid-anchor blocks
    const int n_work = (int)gridDim.x - n_fill;
    if ((int)blockIdx.x >= n_work) {
        for (int blk = (int)blockIdx.x - n_work; blk < total_blocks; blk += n_fill)
            fill_block(blk, S, N, L5, kH, DOUT, anchors, keep, out);
        return;
    }
    constexpr int kUvWaves = C::kWaves, kUvCopies = C::kCopies, kUvStores = C::kStores;
    constexpr int kUvEpiStride = C::kEpiStride;
    // the ring slots are separate arrays so that the compiler sees that a
    // copy into one slot does not touch the slot being read
    __shared__ __attribute__((aligned(16))) char s0[kUvSlot];
    __shared__ __attribute__((aligned(16))) char s1[kUvSlot];
    __shared__ __attribute__((aligned(16))) char s2[kUvSlot];
    __shared__ __attribute__((aligned(16))) char s3[kUvSlot];
    __shared__ __attribute__((aligned(16))) char epi[kUvRows * kUvEpiStride];
    const int lid = xcd_remap(blockIdx.x, n_work);
    const int rg = lid % kUvRowGroups;
    const int h = lid / kUvRowGroups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    // rows of this chunk (kept slots [slot0, slot0 + nslots)); local row r is
    // query r % 5 of slot slot0 + r / 5
    const int rows = kBlock * max(0, min(nslots, status[kStKeptCount] - slot0));
    const int n_iter = (rows + kUvRows - 1) / kUvRows;
    if (rg >= n_iter) return;
    const int n_mine = (n_iter - rg + kUvRowGroups - 1) / kUvRowGroups;   // iterations here

    // A fragments: tile vt, row m = l16 is output dim
    // 32*wave + 8*(m/4) + 4*vt + m%4, so that after the transposed
    // MFMAs the lane with k-group g holds the 8 consecutive dims
    // 32*wave + 8g .. 32*wave + 8g + 7; k-values follow the permuted o_lat
    // order (dims 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3).
    // W_UV[h] reaches them through the ring slots (idle until the first
    // o_lat copy) in two halves of DOUT / 2 output dims: one 1 KB weight row
    // per wave instruction, row r of a half at slot r / 32, row r % 32 (the
    // ring's own row stride); the waves whose dims a half holds then read
    // their fragments out of LDS.  Loading the fragments straight from
    // memory (8 bytes a lane from 16 rows per instruction) made a 64-block
    // call ~6 us slower.
    auto slot_of = [&](int k) -> char* { return k == 0 ? s0 : k == 1 ? s1 : k == 2 ? s2 : s3; };
    bf16x8 a[kUvKs][2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int i = 0; i < C::kHalf / kUvWaves; ++i) {
            const int r = wave * (C::kHalf / kUvWaves) + i;     // uniform per wave
            async_copy_16(w_uv + ((size_t)h * DOUT + C::kHalf * half + r) * kD + lane * 8,
                          slot_of(r / 32) + (r % 32) * kUvLdsStride);
        }
        __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
        __syncthreads();
        if (wave / (kUvWaves / 2) == half) {
            const char* base = slot_of(wave % (kUvWaves / 2));
#pragma unroll
            for (int vt = 0; vt < 2; ++vt) {
                const bf16* row = reinterpret_cast<const bf16*>(
                    base + (8 * (l16 >> 2) + 4 * vt + (l16 & 3)) * kUvLdsStride);
#pragma unroll
                for (int ks = 0; ks < kUvKs; ++ks)
                    a[ks][vt] = cat(ld8(row + 32 * ks + 4 * g), ld8(row + 32 * ks + 16 + 4 * g));
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __syncthreads();
    }

    // Copy of the workgroup's k-th iteration into `dst`: wave w copies rows
    // kCopies w .. kCopies w + kCopies - 1 (at most 31), one o_lat row (1 KB)
    // per instruction; rows past the end copy the last row.  Iterations past the last one are still issued (so
    // that every iteration issues the same memory operations) but read
    // nothing: their offsets fall outside the buffer resource, and such
    // reads return zeros without touching memory.
    auto stage = [&](int k, char* dst) {
        const int r0 = (rg + k * kUvRowGroups) * kUvRows;
        const i32x4 rs = rsrc_words(o_lat + ((size_t)kBlock * slot0 + r0) * kH * kD,
                                    (uint32_t)(kUvRows * kH * kD * sizeof(bf16)));
#pragma unroll
        for (int q = 0; q < kUvCopies; ++q) {
            const int lr = min(kUvCopies * wave + q, kUvRows - 1);
            const int r = min(r0 + lr, rows - 1) - r0;      // negative past the end
            const uint32_t off = (r >= 0) ? (uint32_t)((r * kH + h) * kD * sizeof(bf16) + lane * 16)
                                          : 0xFFFFFFF0u;
            copy_16_untracked(rs, off, dst + lr * kUvLdsStride);
        }
    };

    // B fragment (t, ks): row 16t + l16 of the staged tile, stored o_lat
    // positions 32ks + 8g .. 32ks + 8g + 7
    auto b_frag = [&](const char* src, int t, int ks) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(src + (16 * t + l16) * kUvLdsStride + ks * 64 +
                                                g * 16);
    };

    // Output transpose: every wave writes its 64 B of each of the 32 rows,
    // then wave w stores rows 2 kStores w .. (at most 31) as 2 rows x
    // DOUT x 2 B per instruction.  Rows past the end repeat the last row
    // (same values, same place).  The kept blocks of those rows (at most 2
    // slots: 6 consecutive rows span at most two blocks of 5) are read with
    // scalar loads.
    bf16x8 pend[2];
    int pk[2];            // kept[] of the 2 slots from pslot on
    int pslot = 0, prow0 = 0;
    auto out_row = [&](int j) { return 2 * min(kUvStores * wave + j, kUvRows / 2 - 1) + (lane >> 5); };
    auto flush = [&]() {
#pragma unroll
        for (int t = 0; t < 2; ++t)
            *reinterpret_cast<bf16x8*>(&epi[(16 * t + l16) * kUvEpiStride + 64 * wave + 16 * g]) =
                pend[t];
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int j = 0; j < kUvStores; ++j) {
            // lanes past the row's DOUT / 8 chunks read its last chunk and store nothing
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(
                &epi[out_row(j) * kUvEpiStride + min(lane & 31, DOUT / 8 - 1) * 16]);
            const int r = min(prow0 + out_row(j), rows - 1);
            const int blk = (r / kBlock == pslot) ? pk[0] : pk[1];
            const int b = blk / N, n = blk % N;
            bf16* dst = out + (((size_t)b * L5 + (size_t)kBlock * n + r % kBlock) * kH + h) * DOUT +
                        (lane & 31) * 8;
            // non-temporal when no wave repeats another's row pair (a repeated
            // store would then reach HBM twice instead of merging in L2)
            if ((lane & 31) < DOUT / 8) {
                if constexpr (kUvStores * kUvWaves == kUvRows / 2) gst16_nt(dst, v);
                else gst16(dst, v);
            }
        }
    };

    // Iteration k: wait for its copy (issued three iterations earlier), start
    // the copy three iterations ahead into the slot freed by iteration k-1,
    // store iteration k-1's results, compute.  vmcnt retires in issue order,
    // stores included; the operations issued after the copy of iteration k
    // are the copies of k+1 and k+2 (kUvCopies each) and the stores of
    // iterations k-4 .. k-2 (none before the first iteration).
    auto iteration = [&](int k, const char* cur, char* ahead) {
        if (k >= 4) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kUvCopies + 3 * kUvStores));
        else if (k == 3) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kUvCopies + 2 * kUvStores));
        else if (k == 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kUvCopies + kUvStores));
        else __builtin_amdgcn_s_waitcnt(wait_vm(2 * kUvCopies));
        __asm__ volatile("s_barrier" ::: "memory");
        stage(k + 3, ahead);
        if (k > 0) flush();

        f32x4 acc[2][2];
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[vt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B fragments of k-step ks + 1 are read while the MFMAs of ks run
        bf16x8 bcur[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) bcur[t] = b_frag(cur, t, 0);
#pragma unroll
        for (int ks = 0; ks < kUvKs; ++ks) {
            bf16x8 bnext[2];
            if (ks + 1 < kUvKs) {
#pragma unroll
                for (int t = 0; t < 2; ++t) bnext[t] = b_frag(cur, t, ks + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[vt][t] = mfma_16x16x32(a[ks][vt], bcur[t], acc[vt][t]);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kUvKs) {
#pragma unroll
                for (int t = 0; t < 2; ++t) bcur[t] = bnext[t];
            }
        }
        prow0 = (rg + k * kUvRowGroups) * kUvRows;
        pslot = min(prow0 + 2 * min(kUvStores * wave, kUvRows / 2 - 1), rows - 1) / kBlock;
#pragma unroll
        for (int i = 0; i < 2; ++i) pk[i] = kept[slot0 + min(pslot + i, (rows - 1) / kBlock)];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = (bf16)acc[0][t][i];
                v[4 + i] = (bf16)acc[1][t][i];
            }
            pend[t] = v;
        }
    };

    stage(0, s0);
    stage(1, s1);
    stage(2, s2);
    for (int k = 0; k < n_mine; k += 4) {
        iteration(k, s0, s3);
        if (k + 1 < n_mine) iteration(k + 1, s1, s0);
        if (k + 2 < n_mine) iteration(k + 2, s2, s1);
        if (k + 3 < n_mine) iteration(k + 3, s3, s2);
    }
    // every wave is done with the transpose area of the previous store
    __asm__ volatile("s_barrier" ::: "memory");
    flush();
    // copies issued past the last iteration must land before the
    // workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

}  // namespace

hipError_t launch_uv(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                     hipStream_t s, const int32_t* anchors, const uint8_t* keep) {
    const int grid = kH * kUvRowGroups;
    const int total = p.B * p.N;
    const int n_fill = anchors ? std::min(256, total) : 0;
    hipLaunchKernelGGL(uv_kernel<kDv>, dim3(grid + n_fill), dim3(UvCfg<kDv>::kWaves * 64), 0, s,
                       (const bf16*)in.w_uv, ws.olat, ws.kept, ws.status, (bf16*)in.out, p.N,
                       p.L5, c.slot0, c.nslots, anchors, keep, p.S, total, n_fill);
    return hipGetLastError();
}

hipError_t launch_uv_dqc(const Problem& p, const void* w_uk, const bf16* dqabs,
                         const Workspace& ws, void* dq_nope, hipStream_t s) {
    const int grid = kH * kUvRowGroups;
    hipLaunchKernelGGL(uv_kernel<kDc>, dim3(grid), dim3(UvCfg<kDc>::kWaves * 64), 0, s,
                       (const bf16*)w_uk, dqabs, ws.kept, ws.status, (bf16*)dq_nope, p.N, p.L5,
                       0, p.B * p.N, nullptr, nullptr, p.S, 0, 0);
    return hipGetLastError();
}

}  // namespace dspark
