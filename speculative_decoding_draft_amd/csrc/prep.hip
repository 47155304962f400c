// Preparation pass, one launch: the anchor/window index, the RoPE table and
// the rows of blocks that are not computed (padding, invalid anchors).
//
// Index: build_index (index.hpp), run by one 1024-thread workgroup.
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

#include "index.hpp"

namespace dspark {

namespace {

constexpr int kPrepThreads = 1024;
constexpr int kIndexThreads = kPrepThreads;

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

// grid = 1 + rope_wgs + fill_wgs; out == nullptr (fill_wgs = 0) skips the fill.
// The RoPE and fill parts loop with a grid stride, so a few hundred
// workgroups cover any problem size.
__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    int total, int S, int W, const int32_t* __restrict__ anchors,
    const uint8_t* __restrict__ keep, int4* __restrict__ idx, int32_t* __restrict__ kept,
    int4* __restrict__ srec, int32_t* __restrict__ status, int4* __restrict__ idx_copy,
    int32_t* __restrict__ ctl, int ctl_words, int32_t path_tag, long long rope_n, int pairs,
    RopeTheta th, float2* __restrict__ table, int rope_wgs, bf16* __restrict__ out, int N,
    int L5, int H, int dv) {
    if (blockIdx.x == 0) {
        __shared__ IndexScratch<kIndexThreads> sc;
        build_index<kIndexThreads>(total, S, W, N, anchors, keep, sc, nullptr, true, idx, kept,
                                   srec, status, idx_copy, ctl, ctl_words, path_tag);
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
                       const RopeTheta* th, void* out, hipStream_t s, int32_t path_tag) {
    const int pairs = p.dr / 2;
    const long long rope_n = (th && pairs > 0) ? (long long)rope_rows * pairs : 0;
    constexpr long long kRopeWgs = 128, kFillWgs = 256;
    const int rope_wgs = (int)std::min(kRopeWgs, (rope_n + kPrepThreads - 1) / kPrepThreads);
    const int fill_wgs = out ? (int)std::min<long long>(kFillWgs, (long long)p.B * p.N) : 0;
    RopeTheta none{};
    hipLaunchKernelGGL(prep_kernel, dim3(1 + rope_wgs + fill_wgs), dim3(kPrepThreads), 0, s,
                       p.B * p.N, p.S, p.W, anchors, keep, ws.idx, ws.kept, ws.srec, ws.status,
                       reinterpret_cast<int4*>(index_copy), ws.ctl,
                       ws.ctl ? kFusedCtlWords : 0, path_tag, rope_n, pairs > 0 ? pairs : 1,
                       th ? *th : none, ws.rope, rope_wgs, static_cast<bf16*>(out), p.N, p.L5,
                       p.H, p.dv);
    return hipGetLastError();
}

}  // namespace dspark
