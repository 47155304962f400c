// W_UV up-projection: out[b, q, h, :] = W_UV[h] o_lat[h][r]  (512 -> 256) for
// every kept query row r, bf16 MFMA with fp32 accumulation.
//
// Design page §4 "MLA Projection": v_h = W_UV[h] c^KV; because the attention
// weights sum to one per row, sum_k p_k v_h(k) = W_UV[h] (sum_k p_k c^KV_k),
// so the value up-projection is applied once per (query, head) to o_lat.
//
// o_lat[h][r][512] comes from the attention kernel with the latent dims
// permuted inside each 32-dim group (stored position 32k + 8g + s is dim
// 32k + 4g + s for s < 4, 32k + 16 + 4g + (s-4) for s >= 4); the weight
// fragments are read in the same order, two 8-byte pieces per lane.
//
// Work split: a workgroup owns one head, one half of the 256 output dims
// (a 128 x 512 weight slice resident in LDS) and a strided range of 256-row
// iterations; each wave computes 128 dims x 64 rows, transposed (dims x rows),
// and writes 4 consecutive output dims per lane.
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kUvRowGroups = 2;
constexpr int kUvStride = kD + 8;        // bf16 per LDS weight row (1040 B)
constexpr int kUvRowsPerIter = 256;

__global__ __launch_bounds__(256) void uv_kernel(const bf16* __restrict__ w_uv,
                                                 const bf16* __restrict__ o_lat,
                                                 const int32_t* __restrict__ kept,
                                                 const int32_t* __restrict__ status,
                                                 bf16* __restrict__ out, int N, int L5,
                                                 int rows_max) {
    __shared__ __attribute__((aligned(16))) bf16 wl[128 * kUvStride];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int vh = lid & 1;
    const int rg = (lid >> 1) % kUvRowGroups;
    const int h = (lid >> 1) / kUvRowGroups;
    const int tid = threadIdx.x;

    for (int e = tid; e < 128 * (kD / 8); e += 256) {
        const int v = e / (kD / 8), ch = e % (kD / 8);
        st16(&wl[v * kUvStride + ch * 8],
             ld16(w_uv + ((size_t)h * kDv + vh * 128 + v) * kD + ch * 8));
    }
    __syncthreads();

    const int rows = kBlock * status[kStKeptCount];
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    for (int it = rg; it * kUvRowsPerIter < rows; it += kUvRowGroups) {
        const int row0 = it * kUvRowsPerIter + wave * 64;
        if (row0 >= rows) continue;
        const bf16* op[4];
        for (int t = 0; t < 4; ++t) {
            int r = row0 + t * 16 + l16;
            r = (r < rows) ? r : rows - 1;
            op[t] = o_lat + ((size_t)h * rows_max + r) * kD + g * 8;
        }
        f32x4 acc[8][4];
        for (int vt = 0; vt < 8; ++vt)
            for (int t = 0; t < 4; ++t) acc[vt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int ks = 0; ks < kD / 32; ++ks) {
            bf16x8 bo[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) bo[t] = ld16(op[t] + ks * 32);
#pragma unroll
            for (int vt = 0; vt < 8; ++vt) {
                const bf16* ap = &wl[(vt * 16 + l16) * kUvStride + ks * 32 + g * 4];
                const bf16x8 af = cat(ld8(ap), ld8(ap + 16));
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[vt][t] = mfma_16x16x32(af, bo[t], acc[vt][t]);
            }
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = row0 + t * 16 + l16;
            if (r >= rows) continue;
            const int slot = r / kBlock, j = r % kBlock;
            const int blk = kept[slot];
            const int b = blk / N, n = blk % N;
            bf16* dst = out + (((size_t)b * L5 + (size_t)kBlock * n + j) * kH + h) * kDv +
                        vh * 128 + g * 4;
#pragma unroll
            for (int vt = 0; vt < 8; ++vt) {
                const f32x4 a = acc[vt][t];
                st8(dst + vt * 16, bf16x4{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3]});
            }
        }
    }
}

}  // namespace

hipError_t launch_uv(const Problem& p, const Inputs& in, const Workspace& ws, hipStream_t s) {
    const int grid = kH * 2 * kUvRowGroups;
    hipLaunchKernelGGL(uv_kernel, dim3(grid), dim3(256), 0, s, (const bf16*)in.w_uv, ws.olat,
                       ws.kept, ws.status, (bf16*)in.out, p.N, p.L5, p.rows_max);
    return hipGetLastError();
}

}  // namespace dspark
