// Anchor/window index builder and RoPE table.
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
#include <climits>

#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kIndexThreads = 1024;

// One workgroup: scans all B*N blocks in order, so the kept slots are the
// ranks of the kept blocks in (b, n) order.
__global__ __launch_bounds__(kIndexThreads) void index_kernel(
    int total, int S, int W, const int32_t* __restrict__ anchors,
    const uint8_t* __restrict__ keep, int4* __restrict__ idx, int32_t* __restrict__ kept,
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
__global__ __launch_bounds__(256) void rope_table_kernel(int rows, int pairs, RopeTheta th,
                                                         float2* __restrict__ table) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (long long)rows * pairs) return;
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

}  // namespace

hipError_t launch_index(const Problem& p, const int32_t* anchors, const uint8_t* keep,
                        const Workspace& ws, int32_t* index_copy, hipStream_t s) {
    hipLaunchKernelGGL(index_kernel, dim3(1), dim3(kIndexThreads), 0, s, p.B * p.N, p.S, p.W,
                       anchors, keep, ws.idx, ws.kept, ws.status,
                       reinterpret_cast<int4*>(index_copy));
    return hipGetLastError();
}

hipError_t launch_rope_table(const Problem& p, int rope_rows, const RopeTheta& th,
                             const Workspace& ws, hipStream_t s) {
    const int pairs = p.dr / 2;
    if (pairs == 0) return hipSuccess;
    const long long n = (long long)rope_rows * pairs;
    const int blocks = (int)((n + 255) / 256);
    hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, rope_rows, pairs, th,
                       ws.rope);
    return hipGetLastError();
}

}  // namespace dspark
