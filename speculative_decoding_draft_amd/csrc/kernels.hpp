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
};

// Index build, and optionally (th != nullptr) the RoPE table and (out !=
// nullptr) the rows of padding / invalid-anchor blocks, in one launch.
hipError_t launch_prep(const Problem& p, const int32_t* anchors, const uint8_t* keep,
                       const Workspace& ws, int32_t* index_copy, int rope_rows,
                       const RopeTheta* th, void* out, hipStream_t s);
hipError_t launch_generic(const Problem& p, bool bf16_io, const Inputs& in,
                          const Workspace& ws, hipStream_t s);
size_t generic_lds_bytes(const Problem& p);
// A chunk is the range [slot0, slot0 + nslots) of kept-block slots; its
// latent rows are 5 * (slot - slot0) + j in the latent buffers.
struct Chunk {
    int slot0;
    int nslots;
};

hipError_t launch_absorb(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                         hipStream_t s);
hipError_t launch_attn(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                       const RopeTheta& th, hipStream_t s);
hipError_t launch_uv(const Problem& p, const Inputs& in, const Workspace& ws, Chunk c,
                     hipStream_t s);

}  // namespace dspark
