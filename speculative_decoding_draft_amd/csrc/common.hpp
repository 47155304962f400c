// Internal definitions shared by the host API and the gfx950 kernels of
// libdspark_attn.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark_attn.h"

namespace dspark {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 5;          // draft block length (design page, §2)
constexpr int kMaxRopePairs = 128; // d_rope <= 256

// GLM-5.2 DSpark draft attention dims served by the MFMA kernels.
constexpr int kH = 64, kD = 512, kDc = 192, kDr = 64, kDv = 256;
constexpr int kMaxWindow = 128;    // W <= 128: at most 127 context + 5 block keys
constexpr int kMaxKeys = kMaxWindow - 1 + kBlock;   // 132
constexpr int kKeySlots = (kMaxKeys + 15) / 16 * 16;   // 144: a block's keys in 16-key tiles

// Status area of the workspace (int32 words), written by the index builder
// except where noted.  kStUnsorted: nonzero when some sample's kept anchors
// do not ascend in slot order (the backward then sums block partials with
// atomics).  kStPipeFault: a stalled fused pipeline.  kStPathTag: what the
// last index build on this workspace was for (a hash of the descriptor and
// the forward path; 0 when nothing may reuse it).  kStReuseBad: set by a
// backward with reuse_forward whose workspace does not hold that tag.
enum StatusWord {
    kStKeptCount = 0, kStFirstBad = 1, kStUnsorted = 2, kStPipeFault = 3, kStPathTag = 4,
    kStReuseBad = 5, kStWords = 16
};
static_assert(kStWords * 4 == DSPARK_STATUS_BYTES, "status area size");

// Fused forward (GLM dims on a 256-CU, 8-XCD gfx950).  Each XCD owns 8 of
// the 64 heads; the query latents and attention outputs of its heads travel
// between its compute units through two rings of kFusedRing kept blocks in
// that XCD's L2, coordinated by int32 counters (kFusedCtlStride words per
// XCD, zeroed by the preparation launch).
constexpr int kFusedXcds = 8;
constexpr int kFusedCus = 256;
constexpr int kFusedRing = 32;
constexpr int kFusedHeads = kH / kFusedXcds;
constexpr size_t kFusedSlotElems = (size_t)kBlock * kFusedHeads * kD;   // bf16 per ring slot
constexpr int kFusedCtlStride = 576;   // 320 control words, then 8 timing words per unit
constexpr int kFusedCtlWords = kFusedXcds * kFusedCtlStride;

// RoPE angles theta_i = base^(-2i/d_r), computed on the host in fp64.
struct RopeTheta {
    double t[kMaxRopePairs];
};

// The status area is always at offset 0 so that it can be found from the
// workspace pointer alone.
struct WsLayout {
    size_t status = 0;   // int32 [kStWords]
    size_t idx = 0;      // int4 [B*N]       {ctx_lo, ctx_len, pos0, slot}
    size_t kept = 0;     // int32 [B*N]      slot -> b*N + n
    size_t srec = 0;     // int4 [B*N]       slot -> {ctx_lo, ctx_len, pos0, b*N + n}
    size_t rope = 0;     // float2 [S + 8][d_r/2]  (cos, sin)
    size_t qabs = 0;     // bf16 [5*B*N][H][D]  (MFMA path; row = 5*slot + query,
                         // the same rows whatever the round size)
    size_t olat = 0;     // bf16 [5*B*N][H][D]  (MFMA path)
    size_t ctl = 0;      // int32 [kFusedCtlWords]                 (fused path)
    size_t qring = 0;    // bf16 [8 XCDs][kFusedRing][5][8][D]     (fused path)
    size_t oring = 0;    // bf16 [8 XCDs][kFusedRing][5][8][D]     (fused path)
    size_t total = 0;
    int rope_rows = 0;   // S + 8
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// mfma: the three-kernel MFMA path (materialised q_abs / o_lat); fused: the
// one-launch pipeline (control words and rings instead of the RoPE table and
// the latent buffers); neither: the generic path (RoPE table).
inline WsLayout ws_layout(const dspark_attn_desc& d, bool mfma, bool fused = false) {
    WsLayout w;
    const size_t blocks = size_t(d.B) * size_t(d.N);
    size_t off = 0;
    w.status = off; off = align256(off + kStWords * 4);
    w.idx = off;    off = align256(off + blocks * 16);
    w.kept = off;   off = align256(off + blocks * 4);
    w.srec = off;   off = align256(off + blocks * 16);
    if (fused) {
        const size_t ring = (size_t)kFusedXcds * kFusedRing * kFusedSlotElems * 2;
        w.rope = off;   // no table
        w.ctl = off;    off = align256(off + (size_t)kFusedCtlWords * 4);
        w.qring = off;  off = align256(off + ring);
        w.oring = off;  off = align256(off + ring);
        w.total = off;
        return w;
    }
    w.rope_rows = d.S + 8;
    w.rope = off;   off = align256(off + size_t(w.rope_rows) * size_t(d.d_rope / 2) * 8);
    if (mfma) {
        const size_t lat = size_t(d.n_heads) * kBlock * blocks * size_t(d.d_latent) * 2;
        w.qabs = off; off = align256(off + lat);
        w.olat = off; off = align256(off + lat);
    }
    w.total = off;
    return w;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (id % 8).  Give each
// XCD a contiguous range of logical ids so that neighbouring work items (for
// example blocks with overlapping windows) share that XCD's L2.
__device__ inline int xcd_remap(int id, int grid) {
    if (grid % 8 != 0) return id;
    return (id % 8) * (grid / 8) + id / 8;
}

// The same for a grid of which only the first n_live logical ids have work
// (the count is known on the device only): each XCD gets an equal share of
// the live ids, again as a contiguous range.  Returns -1 for ids without
// work.  Requires grid % 8 == 0 and n_live <= grid.
__device__ inline int xcd_balance(int id, int n_live) {
    const int share = (n_live + 7) / 8;
    const int x = id % 8, k = id / 8;
    if (k >= share) return -1;
    const int lid = x * share + k;
    return lid < n_live ? lid : -1;
}

// Global-memory accesses go through address-space-1 pointers so that they
// compile to global_load/global_store: a generic (flat) access also counts
// against lgkmcnt and turns every LDS wait into a wait for memory as well.
typedef __attribute__((address_space(1))) bf16x8 gbf16x8;
typedef __attribute__((address_space(1))) bf16x4 gbf16x4;
__device__ inline bf16x8 gld16(const bf16* p) { return *(const gbf16x8*)(p); }
__device__ inline bf16x4 gld8(const bf16* p) { return *(const gbf16x4*)(p); }
__device__ inline void gst16(bf16* p, bf16x8 v) { *(gbf16x8*)(p) = v; }
__device__ inline void gst8(bf16* p, bf16x4 v) { *(gbf16x4*)(p) = v; }
// Non-temporal store (the line is not kept dirty in L2), for whole rows that
// no later launch of the call reads (the forward's output): the launch's end
// then has fewer dirty L2 lines to write back before the next launch starts.
// Rows a later launch reads are stored normally, so that they are read from
// the Infinity Cache; stores of partial lines (64-byte pieces) are also
// slower this way.
__device__ inline void gst16_nt(bf16* p, bf16x8 v) { __builtin_nontemporal_store(v, (gbf16x8*)(p)); }

// LDS accesses (pointers into __shared__ arrays)
__device__ inline bf16x8 ld16(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline void st16(bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ inline bf16x4 ld8(const bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }
__device__ inline void st8(bf16* p, bf16x4 v) { *reinterpret_cast<bf16x4*>(p) = v; }

__device__ inline bf16x8 cat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// D(16x16, f32) += A(16x32) * B(32x16), bf16 operands.  Lane l supplies row
// l%16 of A and column l%16 of B, each with 8 k-values (k-group l/16); lane l
// receives D[4*(l/16) + i][l%16], i = 0..3.
__device__ inline f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same with K = 16: 4 k-values per lane (k-group l/16).
__device__ inline f32x4 mfma_16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                     __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (gfx950
// global_load_lds_dwordx4): lane i's 16 bytes land at lds_base + 16 * i, so
// one wave moves 1 KB into a contiguous LDS range.  lds_base must be the same
// for every lane of the wave.  Completion is tracked by vmcnt.
__device__ inline void async_copy_16(const void* gsrc, void* lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)(lds_base),
                                     16, 0, 0);
}

// Buffer resource over a whole tensor (raw, untyped access; reads past
// num_bytes return 0) and a 16-byte copy through it into LDS.  Unlike the
// global form, the buffer form is counted by vmcnt only, so LDS reads issued
// after it keep exact lgkmcnt waits.  Offsets are 32-bit: tensors below 4 GiB.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_bytes,
                                             0x00020000);
}
__device__ inline void buffer_copy_16(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset,
                                      void* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(lds_base), 16, (int)byte_offset, 0, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); the counters not named are left unconstrained.
constexpr int kWaitVm0 = 0x0F70;     // vmcnt(0): this wave's global loads, stores, LDS DMA
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0): this wave's LDS operations
constexpr int kWaitVm0Lgkm0 = 0x0070;   // vmcnt(0) and lgkmcnt(0)

// s_waitcnt vmcnt(n), other counters unconstrained (gfx9 encoding)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Words of a raw buffer resource over num_bytes from base (the fields
// buffer_rsrc() sets), made wave-uniform so that they live in SGPRs.
__device__ inline i32x4 rsrc_words(const void* base, uint32_t num_bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF)), (int)num_bytes,
                 0x00020000};
}

// 16-byte-per-lane LDS DMA (lane i's bytes land at lds + 16 i) issued from
// inline asm.  The compiler does not see it, so it adds no waits of its own
// for it (its alias tracking would otherwise make every LDS read wait for
// all copies in flight); the caller waits with vmcnt before the destination
// is read.  `lds` must be the same for every lane.
// M0 is reserved by the compiler, which sets it itself before every use; the
// clobber tells it that the value does not survive this statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void copy_16_untracked(i32x4 rsrc, uint32_t byte_offset, const char* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(lds));
    __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0), "v"(byte_offset), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// RoPE (cos, sin) of pair i at position pos (design page §4 "RoPE": angle
// pos * theta_i).  The angle is formed in fp64 as turns, pos * theta_i / 2pi
// (turns[i] = theta_i / 2pi, in LDS), reduced to [-1/2, 1/2] and evaluated
// with the hardware sin/cos, which take turns (absolute error ~1e-7, far
// below bf16 resolution).  An fp32 angle at position ~1e5 would be off by up
// to ~4e-3 rad.
__device__ inline float2 rope_cs(const double* turns, int pos, int i) {
    const double a = (double)pos * turns[i];
    const float f = (float)(a - __builtin_rint(a));
    return make_float2(__builtin_amdgcn_cosf(f), __builtin_amdgcn_sinf(f));
}

// One RoPE pair rotation, (x0, x1) by the angle whose (cos, sin) is cs, with
// the multiply-adds spelled out, so that every kernel that rotates a key or
// query row (the forward's and the backward's attention) rounds it the same
// way whatever the compiler would otherwise contract.
__device__ inline float2 rope_rot(float x0, float x1, float2 cs) {
    return make_float2(__builtin_fmaf(x0, cs.x, -(x1 * cs.y)), __builtin_fmaf(x0, cs.y, x1 * cs.x));
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane r*4 + c points at 4 consecutive 16-bit elements of "row" r
// (r = 0..3); lane j of the group receives element j%4 of the chunk held by
// lane (row e)*4 + j/4, for e = 0..3, i.e. column j of the 4 x 16 tile.
__device__ inline bf16x4 lds_read_tr(const bf16* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

}  // namespace dspark
