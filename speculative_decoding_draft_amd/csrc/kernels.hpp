// Launch wrappers of the gfx950 kernels (internal to libdspark_attn.so).
#pragma once

#include "common.hpp"

namespace dspark {

// Per-call problem constants handed to every kernel.
struct Problem {
    int B, S, N, W, H, D, dc, dr, dv;
    int L5;          // 5 * N queries per sample
    float scale;     // softmax scale
};

struct Inputs {
    const void* q_nope;
    const void* q_rope;
    const void* ckv_ctx;
    const void* kr_ctx;
    const void* ckv_blk;
    const void* kr_blk;
    const void* w_uk;
    const void* w_uv;
    void* out;
};

struct Workspace {
    int4* idx;
    int32_t* kept;
    int4* srec;
    int32_t* status;
    float2* rope;
    bf16* qabs;
    bf16* olat;
    int32_t* ctl = nullptr;     // fused path
    bf16* qring = nullptr;
    bf16* oring = nullptr;
};

// Index build, and optionally (th != nullptr) the RoPE table and (out !=
// nullptr) the rows of padding / invalid-anchor blocks, in one launch.
// ws.ctl != nullptr: the fused path's control words are zeroed as well.
// path_tag goes to status[kStPathTag] (0: the index is for no forward that
// a backward may reuse).
hipError_t launch_prep(const Problem& p, const int32_t* anchors, const uint8_t* keep,
                       const Workspace& ws, int32_t* index_copy, int rope_rows,
                       const RopeTheta* th, void* out, hipStream_t s, int32_t path_tag = 0);
hipError_t launch_generic(const Problem& p, bool bf16_io, const Inputs& in,
                          const Workspace& ws, hipStream_t s);
size_t generic_lds_bytes(const Problem& p);
// A chunk is the range [slot0, slot0 + nslots) of kept-block slots; its
// latent rows are 5 * (slot - slot0) + j in the latent buffers.
struct Chunk {
    int slot0;
    int nslots;
};

// Largest B*N for which the absorb launch builds the index itself (its
// slot table lives in LDS).
constexpr int kSelfIndexMax = 1024;

// The inputs and outputs of the index build, for an absorb launch that runs
// it itself.
struct SelfIndexArgs {
    const int32_t* anchors;
    const uint8_t* keep;
    int total, S, W;
    int32_t path_tag;
    int4* idx;
    int32_t* kept;
    int4* srec;
    int32_t* status;
};

// anchors / keep != nullptr: the launch also builds the index (as
// launch_prep without RoPE table and fill, path_tag to the status area), so
// no preparation launch precedes it; only for one round (c covers every
// block) of at most kSelfIndexMax blocks (hipErrorInvalidValue otherwise).
hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                         hipStream_t s, const int32_t* anchors = nullptr,
                         const uint8_t* keep = nullptr, int32_t path_tag = 0);
// pmat: nullptr, or where the normalised probabilities go as well (bf16,
// [slot][5 H][kKeySlots]) for a backward that reuses them.
hipError_t launch_attn(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                       const RopeTheta& th, hipStream_t s, bf16* pmat = nullptr);
// anchors / keep != nullptr: also write the rows of padding (0) and
// invalid-anchor (NaN) blocks, with extra workgroups that run in the
// launch's tail.
hipError_t launch_uv(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                     hipStream_t s, const int32_t* anchors = nullptr,
                     const uint8_t* keep = nullptr);

// The 5 output rows of block blk (H * dv values each, contiguous) when the
// attention path does not compute them: 0 for a padding block, NaN for a
// kept block whose anchor is outside [0, S-2]; nothing otherwise.  All
// threads of the workgroup take part.
__device__ inline void fill_block(int blk, int S, int N, int L5, int H, int dv,
                                  const int32_t* __restrict__ anchors,
                                  const uint8_t* __restrict__ keep, bf16* __restrict__ out) {
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
    for (int e = threadIdx.x; e < chunks; e += blockDim.x) gst16_nt(base + (size_t)e * 8, fv);
}
// The whole forward after the preparation launch as one persistent launch
// of kFusedCus workgroups (GLM dims; the control words must be zero).
hipError_t launch_fused(const Problem& p, const Inputs& in, const Workspace& ws,
                        const RopeTheta& th, hipStream_t s);
// LDS bytes and threads of the fused kernel (for the host-side residency check)
int fused_threads();
const void* fused_kernel_fn();

}  // namespace dspark
