// The anchor/window index of a forward, as a device function that any
// workgroup of T threads can run (the preparation launch runs it with 1024
// threads; the absorb launch of a one-round forward runs it in every
// workgroup, so that no launch has to precede it).
//
// GLM 5.2 DSpark training-design page, §3 "attention mask": a kept block with
// anchor A sees the context columns [max(0, A-W+1), A) -- at most W-1 of
// them, A excluded, the same for its 5 queries -- plus its own 5 draft
// columns; a padding block (keep = 0) sees nothing and its anchor is never
// read.  A kept anchor must lie in [0, S-2] (§2 "Anchor sampling").
#pragma once

#include <climits>

#include "kernels.hpp"

namespace dspark {

// LDS the index build works in.
template <int T>
struct IndexScratch {
    int wave_count[T / 64];
    // the chunk's kept blocks in slot order (block index, anchor), and the
    // last kept block before the chunk, for the anchor-order check
    int2 chunk_kept[T];
    int2 prev_kept;
    int unsorted;
    int first_bad;
};

// Scans all `total` blocks in (b, n) order with T threads, so the kept slots
// are the ranks of the kept blocks in that order.  Returns the number of kept
// blocks (the same value in every thread).
//   kept_lds != nullptr: kept_lds[slot] = block for every kept slot (LDS,
//                        room for `total` entries).
//   write_global:        also the records idx[block] = {ctx_lo, ctx_len, A,
//                        slot or -1 (padding) or -2 (bad anchor)},
//                        kept[slot], srec[slot] = {ctx_lo, ctx_len, A, block},
//                        idx_copy[block] (if given), ctl zeroed, and the
//                        status words (kept count, first bad block, anchor
//                        order, path tag, cleared fault words).
template <int T>
__device__ inline int build_index(int total, int S, int W, int N,
                                  const int32_t* __restrict__ anchors,
                                  const uint8_t* __restrict__ keep, IndexScratch<T>& sc,
                                  int* kept_lds, bool write_global, int4* __restrict__ idx,
                                  int32_t* __restrict__ kept, int4* __restrict__ srec,
                                  int32_t* __restrict__ status, int4* __restrict__ idx_copy,
                                  int32_t* __restrict__ ctl, int ctl_words, int32_t path_tag) {
    const int tid = threadIdx.x;
    if (write_global) {
        for (int i = tid; i < ctl_words; i += T) ctl[i] = 0;
        if (tid == 0) {
            status[kStPipeFault] = 0;
            status[kStPathTag] = path_tag;
            status[kStReuseBad] = 0;
        }
    }
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid == 0) {
        sc.first_bad = INT_MAX;
        sc.prev_kept = make_int2(-1, 0);
        sc.unsorted = 0;
    }
    int carry = 0;        // kept blocks before this chunk (same value in every thread)
    int first_bad = INT_MAX;
    __syncthreads();
    for (int base = 0; base < total; base += T) {
        const int i = base + tid;
        int state = 0;    // 0 padding / out of range, 1 kept, 2 kept with a bad anchor
        int4 rec = make_int4(0, 0, 0, -1);
        if (i < total && keep[i] != 0) {
            const int A = anchors[i];
            if (A >= 0 && A <= S - 2) {
                const int lo = (A - W + 1 > 0) ? (A - W + 1) : 0;
                rec = make_int4(lo, A - lo, A, 0);
                state = 1;
            } else {
                rec = make_int4(0, 0, 0, -2);
                state = 2;
                first_bad = min(first_bad, i);
            }
        }
        const unsigned long long ballot = __ballot(state == 1);
        const int before_in_wave = __popcll(ballot & ((1ull << lane) - 1ull));
        if (lane == 0) sc.wave_count[wave] = __popcll(ballot);
        __syncthreads();
        int before = carry;
        int chunk = 0;
        for (int w = 0; w < T / 64; ++w) {
            const int c = sc.wave_count[w];
            if (w < wave) before += c;
            chunk += c;
        }
        if (state == 1) {
            rec.w = before + before_in_wave;
            if (write_global) {
                kept[rec.w] = i;
                srec[rec.w] = make_int4(rec.x, rec.y, rec.z, i);
            }
            if (kept_lds) kept_lds[rec.w] = i;
            sc.chunk_kept[rec.w - carry] = make_int2(i, rec.z);
        }
        if (write_global && i < total) {
            idx[i] = rec;
            if (idx_copy) idx_copy[i] = rec;
        }
        __syncthreads();
        // anchors descend between two consecutive kept slots of one sample
        if (state == 1) {
            const int r = rec.w - carry;
            const int2 prev = r > 0 ? sc.chunk_kept[r - 1] : sc.prev_kept;
            if (prev.x >= 0 && prev.x / N == i / N && rec.z < prev.y) sc.unsorted = 1;
        }
        __syncthreads();   // wave_count, chunk_kept and prev_kept are rewritten next
        if (tid == 0 && chunk > 0) sc.prev_kept = sc.chunk_kept[chunk - 1];
        carry += chunk;
    }
    if (first_bad != INT_MAX) atomicMin(&sc.first_bad, first_bad);
    __syncthreads();
    if (write_global && tid == 0) {
        status[kStKeptCount] = carry;
        status[kStFirstBad] = (sc.first_bad == INT_MAX) ? -1 : sc.first_bad;
        status[kStUnsorted] = sc.unsorted;
    }
    return carry;
}

}  // namespace dspark
