// Preparation pass, one launch: the anchor/window index, the RoPE table and
// the rows of blocks that are not computed (padding, invalid anchors).
//
// Index (GLM 5.2 DSpark training-design page, §3 "attention mask"): a kept
// block with anchor A sees the context columns [max(0, A-W+1), A) -- at most
// W-1 of them, A excluded, the same for its 5 queries -- plus its own 5
// draft columns; a padding block (keep = 0) sees nothing and its anchor is
// never read.  A kept anchor must lie in [0, S-2] (§2 "Anchor sampling").
//
// RoPE (§4 "RoPE"): interleaved adjacent pairs; pair i of a vector at
// position p rotates by p * theta_i with theta_i = base^(-2i/d_r).  The
// table covers every position the forward uses: context 0..S-1 and block
// positions A..A+4 <= S+2.
//
// Padding rows (§3 "Padding block"): no output is defined for them; they are
// written as 0.  Rows of a kept block whose anchor lies outside [0, S-2] are
// written as NaN (the status area records the first such block).
//
// Workgroup 0 builds the index; the next ones fill the RoPE table, the rest
// fill rows, so the three parts run side by side.
#include <algorithm>
#include <climits>

#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kIndexThreads = kPrepThreads;

// One workgroup: scans all B*N blocks in order, so the kept slots are the
// ranks of the kept blocks in (b, n) order.
__device__ void build_index(int total, int S, int W, const int32_t* __restrict__ anchors,
                            const uint8_t* __restrict__ keep, int4* __restrict__ idx,
                            int32_t* __restrict__ kept, int4* __restrict__ srec,
                            int32_t* __restrict__ status, int4* __restrict__ idx_copy) {
    __shared__ int wave_count[kIndexThreads / 64];
    __shared__ int first_bad_sh;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid == 0) first_bad_sh = INT_MAX;
    int carry = 0;        // kept blocks before this chunk (same value in every thread)
    int first_bad = INT_MAX;
    __syncthreads();
    for (int base = 0; base < total; base += kIndexThreads) {
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
        if (lane == 0) wave_count[wave] = __popcll(ballot);
        __syncthreads();
        int before = carry;
        int chunk = 0;
        for (int w = 0; w < kIndexThreads / 64; ++w) {
            const int c = wave_count[w];
            if (w < wave) before += c;
            chunk += c;
        }
        if (state == 1) {
            rec.w = before + before_in_wave;
            kept[rec.w] = i;
            srec[rec.w] = make_int4(rec.x, rec.y, rec.z, i);
        }
        if (i < total) {
            idx[i] = rec;
            if (idx_copy) idx_copy[i] = rec;
        }
        carry += chunk;
        __syncthreads();   // wave_count is rewritten by the next chunk
    }
    if (first_bad != INT_MAX) atomicMin(&first_bad_sh, first_bad);
    __syncthreads();
    if (tid == 0) {
        status[kStKeptCount] = carry;
        status[kStFirstBad] = (first_bad_sh == INT_MAX) ? -1 : first_bad_sh;
    }
}

// table[p][i] = (cos, sin)(p * theta_i).  The angle is formed and reduced to
// [-pi, pi] in fp64 (two-term 2*pi), then evaluated in fp32: an fp32 angle
// at p ~ 1.3e5 would carry an absolute error of up to ~4e-3 rad.
__device__ void rope_entry(long long e, int pairs, const RopeTheta& th,
                           float2* __restrict__ table) {
    const int p = (int)(e / pairs);
    const int i = (int)(e % pairs);
    const double two_pi_hi = 6.283185307179586232;
    const double two_pi_lo = 2.449293598294706e-16;
    const double a = (double)p * th.t[i];
    const double k = rint(a / two_pi_hi);
    double r = fma(-k, two_pi_hi, a);
    r = fma(-k, two_pi_lo, r);
    float s, c;
    sincosf((float)r, &s, &c);
    table[e] = make_float2(c, s);
}

// Rows of one block that the attention path does not compute: the block's
// 5 rows of H * dv outputs are contiguous.
__device__ void fill_block(int blk, int S, int N, int L5, int H, int dv,
                           const int32_t* __restrict__ anchors, const uint8_t* __restrict__ keep,
                           bf16* __restrict__ out) {
    bf16 fill;
    if (keep[blk] == 0) {
        fill = (bf16)0.0f;
    } else {
        const int A = anchors[blk];
        if (A >= 0 && A <= S - 2) return;
        fill = (bf16)__builtin_nanf("");
    }
    bf16x8 fv;
    for (int e = 0; e < 8; ++e) fv[e] = fill;
    const int b = blk / N, n = blk % N;
    bf16* base = out + ((size_t)b * L5 + (size_t)kBlock * n) * H * dv;
    const int chunks = kBlock * H * dv / 8;
    for (int e = threadIdx.x; e < chunks; e += kPrepThreads) gst16(base + (size_t)e * 8, fv);
}

// grid = 1 + rope_wgs + fill_wgs; out == nullptr (fill_wgs = 0) skips the fill.
// The RoPE and fill parts loop with a grid stride, so a few hundred
// workgroups cover any problem size.
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    int total, int S, int W, const int32_t* __restrict__ anchors,
    const uint8_t* __restrict__ keep, int4* __restrict__ idx, int32_t* __restrict__ kept,
    int4* __restrict__ srec, int32_t* __restrict__ status, int4* __restrict__ idx_copy,
    long long rope_n, int pairs,
    RopeTheta th, float2* __restrict__ table, int rope_wgs, bf16* __restrict__ out, int N,
    int L5, int H, int dv) {
    if (blockIdx.x == 0) {
        build_index(total, S, W, anchors, keep, idx, kept, srec, status, idx_copy);
        return;
    }
    const int r = blockIdx.x - 1;
    if (r < rope_wgs) {
        for (long long e = (long long)r * kPrepThreads + threadIdx.x; e < rope_n;
             e += (long long)rope_wgs * kPrepThreads)
            rope_entry(e, pairs, th, table);
        return;
    }
    // fill workgroups visit every block; kept blocks with valid anchors are
    // skipped (the test is uniform per block)
    const int fill_wgs = gridDim.x - 1 - rope_wgs;
    for (int blk = r - rope_wgs; blk < total; blk += fill_wgs)
        fill_block(blk, S, N, L5, H, dv, anchors, keep, out);
}

}  // namespace

hipError_t launch_prep(const Problem& p, const int32_t* anchors, const uint8_t* keep,
                       const Workspace& ws, int32_t* index_copy, int rope_rows,
                       const RopeTheta* th, void* out, hipStream_t s) {
    const int pairs = p.dr / 2;
    const long long rope_n = (th && pairs > 0) ? (long long)rope_rows * pairs : 0;
    constexpr long long kRopeWgs = 128, kFillWgs = 256;
    const int rope_wgs = (int)std::min(kRopeWgs, (rope_n + kPrepThreads - 1) / kPrepThreads);
    const int fill_wgs = out ? (int)std::min<long long>(kFillWgs, (long long)p.B * p.N) : 0;
    RopeTheta none{};
    hipLaunchKernelGGL(prep_kernel, dim3(1 + rope_wgs + fill_wgs), dim3(kPrepThreads), 0, s,
                       p.B * p.N, p.S, p.W, anchors, keep, ws.idx, ws.kept, ws.srec, ws.status,
                       reinterpret_cast<int4*>(index_copy), rope_n, pairs > 0 ? pairs : 1,
                       th ? *th : none, ws.rope, rope_wgs, static_cast<bf16*>(out), p.N, p.L5,
                       p.H, p.dv);
    return hipGetLastError();
}

}  // namespace dspark
