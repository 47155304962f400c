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
// Work split: a workgroup (8 waves, two per SIMD) owns one head and a
// strided range of 64-row iterations; wave w computes output dims
// 64w .. 64w+63, transposed (dims x rows), with its 64 x 192 slice of
// W_UK[h]^T in registers.  One workgroup covering all 512 dims copies every
// q^C row into LDS once (splitting the dims over two workgroups made both
// copy it).  W_UK[h] is staged through LDS at start, in two halves of 256
// dims, and read transposed with ds_read_b64_tr_b16.  The q^C rows of an
// iteration are copied into LDS already laid out as MFMA B fragments (LDS
// DMA, double buffered: the copy for the next iteration overlaps the
// current MFMAs) and read by all eight waves.  Results are transposed
// through LDS (the weight staging area, free after start) and stored one
// 1 KB q_abs row per instruction: in the MFMA tile layout (16 rows x 64 B
// per instruction) the stores ran ~20% slower.
#include "index.hpp"

namespace dspark {

namespace {

constexpr int kAbsWaves = 8;                            // 64 output dims each
constexpr int kAbsRowGroups = 4;                        // workgroups per head
constexpr int kAbsRowsPerIter = 64;
constexpr int kAbsTiles = kAbsRowsPerIter / 16;         // row tiles per iteration
constexpr int kAbsDt = 4;                               // 16-dim tiles per wave
constexpr int kAbsEpiStride = kD * 2 + 16;              // bytes per row of the output transpose
constexpr int kAbsStoreRows = kAbsRowsPerIter / kAbsWaves;   // q_abs rows each wave stores

// KD: input dims per row (d_c = 192 for q_abs; the backward runs the same
// kernel with d_v = 256 for W_UV^T dout).  The weight slice is staged
// through LDS in PARTS column parts (2 for 192 rows, 4 for 256, to fit LDS).
template <int KD, int PARTS>
struct AbsCfg {
    static constexpr int Ks = KD / 32;                              // k-steps
    static constexpr int Frags = kAbsTiles * Ks;                    // 1 KB B fragments per iteration
    static constexpr int Copies = Frags / kAbsWaves;                // copy instructions per wave
    static constexpr int PartCols = kD / PARTS;                     // weight columns per part
    static constexpr int Stride = PartCols + 16;                    // weight staging row (bf16)
    static constexpr int WavesPerPart = kAbsWaves / PARTS;
    static constexpr int Shared = (KD * Stride * 2 > kAbsRowsPerIter * kAbsEpiStride)
                                      ? KD * Stride * 2 : kAbsRowsPerIter * kAbsEpiStride;
    static_assert(Copies * kAbsWaves == Frags && Ks % Copies == 0,
                  "each wave copies k-steps of one row tile");
    static_assert(WavesPerPart * 64 == PartCols, "a part holds whole waves' dims");
};

// acc / acc_n4 (the backward's W_UV^T dout, KD = d_v): the workgroups first
// clear the fp32 dc^KV accumulator (acc_n4 float4) when the slots' anchors
// do not ascend (status[kStUnsorted]): the atomic sums need it zeroed.
// SELF_INDEX (one round of at most kSelfIndexMax blocks): every workgroup
// builds the index itself while its first weight part is in flight and
// keeps the slot table in LDS; workgroup 0 also writes the index records and
// status words for the launches after it, so no launch has to precede this
// one.
template <int KD, int PARTS, bool SELF_INDEX = false>
__global__ __launch_bounds__(kAbsWaves * 64) void absorb_kernel(
    const bf16* __restrict__ q_nope, const bf16* __restrict__ w_uk,
    const int32_t* __restrict__ kept, const int32_t* __restrict__ status,
    bf16* __restrict__ q_abs, int N, int L5, int slot0, int nslots, uint32_t q_bytes,
    float4* __restrict__ acc, size_t acc_n4, SelfIndexArgs si) {
    using C = AbsCfg<KD, PARTS>;
    if constexpr (KD == kDv) {
        if (status[kStUnsorted] != 0) {
            for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < acc_n4;
                 e += (size_t)gridDim.x * blockDim.x)
                acc[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    constexpr int kAbsKs = C::Ks, kAbsFrags = C::Frags, kAbsCopies = C::Copies;
    constexpr int kAbsStride = C::Stride, kAbsShared = C::Shared;
    // weight staging at start, then the output transpose
    __shared__ __attribute__((aligned(16))) char shared_area[kAbsShared];
    // the two q^C buffers are separate arrays: the compiler then sees that a
    // copy into one does not touch the other
    __shared__ __attribute__((aligned(16))) char qa_s[kAbsFrags * 1024];
    __shared__ __attribute__((aligned(16))) char qb_s[kAbsFrags * 1024];
    // the slot table when this launch builds the index
    __shared__ int kept_l[SELF_INDEX ? kSelfIndexMax : 1];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int rg = lid % kAbsRowGroups;
    const int h = lid / kAbsRowGroups;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    // rows of this chunk: kept slots [slot0, slot0 + nslots); local row r is
    // query r % 5 of slot slot0 + r / 5
    int rows = 0, n_iter = 0;
    auto set_rows = [&](int n_kept) {
        rows = kBlock * max(0, min(nslots, n_kept - slot0));
        n_iter = (rows + kAbsRowsPerIter - 1) / kAbsRowsPerIter;
    };
    auto kept_at = [&](int slot) -> int {
        if constexpr (SELF_INDEX) return kept_l[slot];
        else return kept[slot];
    };
    if constexpr (!SELF_INDEX) {
        set_rows(status[kStKeptCount]);
        if (rg >= n_iter) return;
    }

    // ---- q^C copies: fragment f = T * 6 + ks of an iteration holds rows
    // 16T + l16 and k-values 32ks + 8g .. +7 (16 rows x 64 B); wave w copies
    // fragments 3w .. 3w+2, all of row tile w / 2.  Rows past the end copy
    // the last row.  The copies are issued from inline asm (waited for at the
    // top of every iteration) so that the compiler adds no waits of its own.
    auto clamp_row = [&](int r) { return (r < rows) ? r : rows - 1; };
    const int copy_tile = (kAbsCopies * wave) / kAbsKs;
    auto copy_row = [&](int it) { return clamp_row(it * kAbsRowsPerIter + 16 * copy_tile + l16); };
    const i32x4 q_rs = rsrc_words(q_nope, q_bytes);
    auto stage = [&](int it, int blk, char* dst) {
        const int r = copy_row(it);
        const int b = blk / N, n = blk % N;
        const uint32_t off = (uint32_t)(
            ((((size_t)b * L5 + (size_t)kBlock * n + r % kBlock) * kH + h) * KD + g * 8) *
            sizeof(bf16));
#pragma unroll
        for (int j = 0; j < kAbsCopies; ++j) {
            const int f = kAbsCopies * wave + j;
            copy_16_untracked(q_rs, off + (f % kAbsKs) * 64, dst + f * 1024);
        }
    };

    // ---- A operand: fragment (ks, dt) holds output dims 64w + 16dt + l16
    // and k-values c = 32ks + 8g .. +7, read transposed out of the [c][d]
    // staging copy of one column part of the weight (the waves whose dims it
    // holds read it).
    bf16x8 a[kAbsKs][kAbsDt];
    {
        bf16* wl = reinterpret_cast<bf16*>(shared_area);
        const int hl = lane >> 5;
#pragma unroll
        for (int part = 0; part < PARTS; ++part) {
            if constexpr (PARTS == 2) {
                // one 512-byte weight row per half-wave instruction
                for (int c0 = 2 * wave; c0 < KD; c0 += 2 * kAbsWaves) {
                    const int c = c0 + hl;
                    if (hl == 0)
                        async_copy_16(w_uk + ((size_t)h * KD + c) * kD + part * 256 + lane * 8,
                                      &wl[c0 * kAbsStride]);
                    else
                        async_copy_16(w_uk + ((size_t)h * KD + c) * kD + part * 256 +
                                          (lane - 32) * 8,
                                      &wl[c0 * kAbsStride + kAbsStride - 256]);
                }
            } else {
                // full-wave copies that fill the padded layout contiguously, 1 KB
                // each: lane l's 16 bytes land at byte 1024 i + 16 l, i.e. row
                // (1024 i + 16 l) / (2 * stride); lanes that land in a row's
                // padding fetch any element of that row
                constexpr int kRowBytes = 2 * kAbsStride;
                constexpr int kCopies = KD * kRowBytes / 1024;
                static_assert(KD * kRowBytes % 1024 == 0 && kRowBytes % 16 == 0, "whole copies");
                for (int i = wave; i < kCopies; i += kAbsWaves) {
                    const int off = 1024 * i + 16 * lane;
                    const int row = off / kRowBytes, cb = off % kRowBytes;
                    const int col = (cb < 2 * C::PartCols) ? cb / 2 : 0;
                    async_copy_16(w_uk + ((size_t)h * KD + row) * kD + part * C::PartCols + col,
                                  shared_area + 1024 * i);
                }
            }
            if constexpr (SELF_INDEX) {
                if (part == 0) {
                    __shared__ IndexScratch<kAbsWaves * 64> sc;
                    set_rows(build_index<kAbsWaves * 64>(
                        si.total, si.S, si.W, N, si.anchors, si.keep, sc, kept_l,
                        blockIdx.x == 0, si.idx, si.kept, si.srec, si.status, nullptr, nullptr,
                        0, si.path_tag));
                }
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
            __syncthreads();
            // the first iteration's q^C copy goes out once the rows are known
            // (the index, built during part 0), so it overlaps the next part
            if (part == 0 && rg < n_iter) stage(rg, kept_at(slot0 + copy_row(rg) / kBlock), qa_s);
            if (wave / C::WavesPerPart == part) {
                const int wd = wave % C::WavesPerPart;
#pragma unroll
                for (int ks = 0; ks < kAbsKs; ++ks)
#pragma unroll
                    for (int dt = 0; dt < kAbsDt; ++dt) {
                        const bf16* ab = wl + (ks * 32 + g * 8 + (l16 >> 2)) * kAbsStride + wd * 64 +
                                         (l16 & 3) * 4 + dt * 16;
                        a[ks][dt] = cat(lds_read_tr(ab), lds_read_tr(ab + 4 * kAbsStride));
                    }
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __syncthreads();
        }
    }

    // a workgroup with no rows leaves once its weight copies have landed
    if constexpr (SELF_INDEX) {
        if (rg >= n_iter) return;
    }

    // ---- output transpose: every wave writes its 64 dims (128 B) of each of
    // the 64 rows, then wave w stores rows 8w .. 8w+7, one 1 KB row per
    // instruction.  Rows past the end repeat the last row (same values, same
    // place).
    char* const epi = shared_area;
    bf16x8 pend[kAbsTiles][2];       // [row tile][dim-tile pair]
    int pit = 0;                     // iteration of the pending results
    auto flush = [&]() {
#pragma unroll
        for (int t = 0; t < kAbsTiles; ++t)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
                *reinterpret_cast<bf16x8*>(epi + (16 * t + l16) * kAbsEpiStride + 128 * wave +
                                           (4 * pp + g) * 16) = pend[t][pp];
        __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int j = 0; j < kAbsStoreRows; ++j) {
            const int lr = kAbsStoreRows * wave + j;
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(epi + lr * kAbsEpiStride + lane * 16);
            const int r = clamp_row(pit * kAbsRowsPerIter + lr);
            gst16(q_abs + ((size_t)(kBlock * slot0 + r) * kH + h) * kD + lane * 8, v);
        }
    };

    // Iteration: wait for its copy (issued one iteration earlier) and the
    // block index of the next copy, start that copy into the other buffer,
    // store the previous iteration's results, compute.
    int cblk = kept_at(slot0 + copy_row(rg + kAbsRowGroups) / kBlock);
    auto iteration = [&](int it, const char* cur, char* other) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        stage(it + kAbsRowGroups, cblk, other);
        cblk = kept_at(slot0 + copy_row(it + 2 * kAbsRowGroups) / kBlock);
        if (it != rg) flush();

        f32x4 acc[kAbsDt][kAbsTiles];
#pragma unroll
        for (int dt = 0; dt < kAbsDt; ++dt)
#pragma unroll
            for (int t = 0; t < kAbsTiles; ++t) acc[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        // B fragments of k-step ks + 1 are read while the MFMAs of ks run
        auto b_frag = [&](int t, int ks) {
            return *reinterpret_cast<const bf16x8*>(cur + (t * kAbsKs + ks) * 1024 + lane * 16);
        };
        bf16x8 bcur[kAbsTiles];
#pragma unroll
        for (int t = 0; t < kAbsTiles; ++t) bcur[t] = b_frag(t, 0);
#pragma unroll
        for (int ks = 0; ks < kAbsKs; ++ks) {
            bf16x8 bnext[kAbsTiles];
            if (ks + 1 < kAbsKs) {
#pragma unroll
                for (int t = 0; t < kAbsTiles; ++t) bnext[t] = b_frag(t, ks + 1);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int dt = 0; dt < kAbsDt; ++dt)
#pragma unroll
                for (int t = 0; t < kAbsTiles; ++t)
                    acc[dt][t] = mfma_16x16x32(a[ks][dt], bcur[t], acc[dt][t]);
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < kAbsKs) {
#pragma unroll
                for (int t = 0; t < kAbsTiles; ++t) bcur[t] = bnext[t];
            }
        }
        // lane holds dims 32pp + 4g + i (tile 2pp) and 32pp + 16 + 4g + i
        // (tile 2pp + 1) of the wave's 64, row 16t + l16: stored positions
        // 32pp + 8g .. +7 of the permuted layout
        pit = it;
#pragma unroll
        for (int t = 0; t < kAbsTiles; ++t)
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                bf16x8 v;
                v[0] = (bf16)a0[0]; v[1] = (bf16)a0[1]; v[2] = (bf16)a0[2]; v[3] = (bf16)a0[3];
                v[4] = (bf16)a1[0]; v[5] = (bf16)a1[1]; v[6] = (bf16)a1[2]; v[7] = (bf16)a1[3];
                pend[t][pp] = v;
            }
    };
    for (int it = rg; it < n_iter; it += 2 * kAbsRowGroups) {
        iteration(it, qa_s, qb_s);
        if (it + kAbsRowGroups < n_iter) iteration(it + kAbsRowGroups, qb_s, qa_s);
    }
    // every wave is done with the transpose area of the previous store
    __syncthreads();
    flush();
    // the copy started by the last iteration is not used; let it land before
    // the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

}  // namespace

hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                         hipStream_t s, const int32_t* anchors, const uint8_t* keep,
                         int32_t path_tag) {
    const int grid = kH * kAbsRowGroups;
    const bool self_index = anchors != nullptr;
    if (self_index && (p.B * p.N > kSelfIndexMax || c.slot0 != 0 || c.nslots < p.B * p.N))
        return hipErrorInvalidValue;
    const SelfIndexArgs si{anchors, keep, p.B * p.N, p.S, p.W, path_tag,
                           ws.idx, ws.kept, ws.srec, ws.status};
    auto* kernel = self_index ? absorb_kernel<kDc, 2, true> : absorb_kernel<kDc, 2, false>;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kAbsWaves * 64), 0, s,
                       (const bf16*)in.q_nope, (const bf16*)in.w_uk, ws.kept, ws.status, ws.qabs,
                       p.N, p.L5, c.slot0, c.nslots,
                       (uint32_t)((size_t)p.B * p.L5 * kH * kDc * sizeof(bf16)), nullptr,
                       (size_t)0, si);
    return hipGetLastError();
}

hipError_t launch_absorb_dv(const Problem& p, const void* dout, const void* w_uv,
                            const Workspace& ws, bf16* dolat, float* acc, size_t n,
                            hipStream_t s) {
    const int grid = kH * kAbsRowGroups;
    hipLaunchKernelGGL((absorb_kernel<kDv, 4>), dim3(grid), dim3(kAbsWaves * 64), 0, s,
                       (const bf16*)dout, (const bf16*)w_uv, ws.kept, ws.status, dolat, p.N, p.L5,
                       0, p.B * p.N, (uint32_t)((size_t)p.B * p.L5 * kH * kDv * sizeof(bf16)),
                       reinterpret_cast<float4*>(acc), n / 4, SelfIndexArgs{});
    return hipGetLastError();
}

}  // namespace dspark
