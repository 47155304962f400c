// The masked latent attention forward for the GLM dims as one persistent
// launch: absorb, attention and the W_UV projection run side by side on
// different compute units, and the query latents (q_abs) and attention
// outputs (o_lat) pass between them through the L2 cache instead of HBM.
//
// What is computed is the absorbed form of the GLM 5.2 DSpark design page
// (§4 "MLA Projection", the appendix equation, the §3 mask):
//   q_abs[r, h] = W_UK[h]^T q^C[r, h]                                (absorb)
//   s = scale (q_abs . c^KV + RoPE(q^R) . RoPE(k^R)) over the block's keys
//   o_lat = softmax(s) . c^KV ,  out[r, h] = W_UV[h] o_lat           (W_UV)
// where a block's keys are the context window [ctx_lo, A) and its own 5
// draft positions.
//
// Layout of the work.  Workgroup i runs on XCD i % 8 (the hardware XCC id is
// read, not assumed); each XCD owns 8 of the 64 heads, so the W_UK and W_UV
// slices of its heads (3.7 MB) live in the registers of its compute units
// and never move again.  The 32 workgroups of an XCD take roles by arrival:
//   * 8 absorb units, one head each: W_UK[h] in registers, q^C rows staged
//     in LDS by DMA, q_abs of every kept row written into the XCD's q ring;
//   * 8 W_UV units, one head each: W_UV[h] in registers, o_lat rows staged
//     in LDS by DMA from the o ring, out written to HBM;
//   * 16 attention units taking kept blocks from a queue: the block's keys
//     (c^KV rows) staged in LDS, the block's q_abs for the 8 heads (40
//     columns = 5 queries x 8 heads) held in registers, scores and P.c^KV on
//     MFMA, o_lat written into the o ring.
// The rings hold kFusedRing kept blocks (40 KB per block per ring) and are
// read back through the XCD's 4 MB L2; int32 counters in the same L2
// (atomics without the agent-scope bit, read with scalar loads that bypass
// the scalar cache) say which ring slots are full and which are free again.
// The L2 is write-back and the other streams evict ring lines before their
// slots are rewritten, so the ring writes still reach HBM (measured: 625 MB
// written per headline call, of which 126 MB is the output).  Every wait is
// bounded in time: a stalled pipeline (never expected: each wait's producer
// is always able to progress) aborts the XCD's units and is reported in the
// status area instead of hanging.
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kFT = 256;                    // 4 waves, one per SIMD
constexpr int kHx = kFusedHeads;            // 8 heads per XCD
constexpr int kNA = kHx, kNU = kHx;         // absorb and W_UV units per XCD
constexpr int kRanks = 32;                  // compute units per XCD
constexpr int kR = kFusedRing;

// control words of one XCD (int32, all in that XCD's L2)
constexpr int kCtTicket = 0, kCtQueue = 16, kCtAbort = 32;
constexpr int kCtQReady = 64, kCtQFree = 128, kCtOReady = 192, kCtOFree = 256;
constexpr int kCtTiming = 320;              // per unit: role, busy, waiting, items, 4 phases
static_assert(kCtOFree + kR <= kCtTiming && kCtTiming + 8 * 32 <= kFusedCtlStride,
              "control words fit");
// counter increments per block and generation of a ring slot
constexpr int kQReadyPer = kNA * 4;         // every absorb wave
constexpr int kQFreePer = 4;                // the attention unit's waves
constexpr int kOReadyPer = 4;
constexpr int kOFreePer = kNU * 4;          // every W_UV wave
constexpr uint64_t kSpinTicks = 20000000ull;    // 0.2 s of the 100 MHz real-time clock

constexpr float kLog2e = 1.4426950408889634f;

struct FusedArgs {
    const bf16* q_nope;
    const bf16* q_rope;
    const bf16* ckv_ctx;
    const bf16* kr_ctx;
    const bf16* ckv_blk;
    const bf16* kr_blk;
    const bf16* w_uk;
    const bf16* w_uv;
    const int32_t* kept;
    const int4* srec;
    int32_t* status;
    int32_t* ctl;
    bf16* q_ring;
    bf16* o_ring;
    bf16* out;
    int S, N, L5;
    float scale;
    uint32_t ctx_bytes, blk_bytes, q_bytes;
    RopeTheta turns;                        // theta_i / 2pi
};

// ---------------------------------------------------------------------------
// coordination
// ---------------------------------------------------------------------------

// XCC id of the executing wave (hardware register HW_REG_XCC_ID, bits 3:0).
__device__ inline int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7); }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Current value of a control word: a scalar load that misses the scalar
// cache and reads the XCD's L2, where the counters are updated.  p must be
// wave-uniform.  The load is waited for in the same statement.
__device__ inline int ctl_read(const int32_t* p) {
    int v;
    __asm__ volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p)
                     : "memory");
    return v;
}

typedef int i32x16 __attribute__((ext_vector_type(16)));
// Sixteen consecutive control words (64-byte aligned), like ctl_read.
__device__ inline i32x16 ctl_read16(const int32_t* p) {
    i32x16 v;
    __asm__ volatile("s_load_dwordx16 %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v)
                     : "s"(p) : "memory");
    return v;
}

// Four consecutive read-only words (a uniform address) through the scalar
// cache, waited for in the same statement.
__device__ inline i32x4 sld4(const int32_t* p) {
    i32x4 v;
    __asm__ volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p)
                     : "memory");
    return v;
}

// 16-byte-per-lane LDS DMA like copy_16_untracked, non-temporal: such a
// load does not return a line this compute unit's L1 still holds from an
// earlier use of the ring slot (plain and sc0 loads do), and is served by
// the XCD's L2, where another unit wrote the slot.
__device__ inline void copy_ring_16(i32x4 rsrc, uint32_t byte_offset, const char* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(
        (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(lds));
    __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     :: "s"(m0), "v"(byte_offset), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait (in hardware) until this wave's vector memory operations have
// completed, except the n most recent; also a compiler barrier.
#define VM_WAIT(n) __asm__ volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

// Ring load (16 B per lane), non-temporal for the same reason as copy_ring_16.
__device__ inline bf16x8 ring_ld16(__amdgpu_buffer_rsrc_t rsrc, uint32_t byte_offset) {
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    const i32x4v v = __builtin_bit_cast(
        i32x4v, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)byte_offset, 0, 2));
    return __builtin_bit_cast(bf16x8, v);
}

// Counter update in the XCD's L2 (no agent-scope bit: every reader is on
// the same XCD), one per wave (called wave-uniformly; lane 0 issues it).
// Callers make their data stores complete first.
__device__ inline void ctl_add(int32_t* p, int v) {
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Spin (whole wave, uniform) until *p >= target.  Returns false once this
// XCD's pipeline is aborted or the wait exceeds its time bound (which
// aborts it and records the fault).
__device__ bool wait_ge(const int32_t* p, int target, int32_t* xctl, int32_t* status,
                        uint64_t* waited = nullptr) {
    if (ctl_read(p) >= target) return true;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        __builtin_amdgcn_s_sleep(2);
        if (ctl_read(p) >= target) {
            if (waited) *waited += __builtin_amdgcn_s_memrealtime() - t0;
            return true;
        }
        if (ctl_read(xctl + kCtAbort) != 0) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
            if ((threadIdx.x & 63) == 0) {
                __hip_atomic_store(xctl + kCtAbort, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_store(status + kStPipeFault, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            return false;
        }
    }
}

// Phase timer (10 ns ticks of the real-time clock) for the timing words.
struct PhaseClock {
    uint64_t last;
    uint32_t* acc;
    __device__ void start() { last = __builtin_amdgcn_s_memrealtime(); }
    __device__ void lap(int i) {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        acc[i] += (uint32_t)(t - last);
        last = t;
    }
};

// A wave's copy of 32 consecutive counters (lane i holds counter i), read
// again only when a check against it fails: a counter only grows, so a
// check that once passed stays true.
struct CtlView {
    const int32_t* base;     // 64-byte aligned
    int v;
    __device__ void refresh() {
        const i32x16 a = ctl_read16(base), b = ctl_read16(base + 16);
        const int lane = threadIdx.x & 63;
        int w = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            w = (lane == i) ? a[i] : w;
            w = (lane == 16 + i) ? b[i] : w;
        }
        v = w;
    }
    __device__ int get(int s) const { return __builtin_amdgcn_readlane(v, s); }
};

// view[s] >= target, refreshing the view while it is not; false on abort or
// when the wait exceeds its time bound (as wait_ge).
__device__ bool view_wait(CtlView& view, int s, int target, int32_t* xctl, int32_t* status,
                          uint64_t* waited) {
    if (view.get(s) >= target) return true;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        view.refresh();
        if (view.get(s) >= target) {
            *waited += __builtin_amdgcn_s_memrealtime() - t0;
            return true;
        }
        if (ctl_read(xctl + kCtAbort) != 0) return false;
        if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) {
            if ((threadIdx.x & 63) == 0) {
                __hip_atomic_store(xctl + kCtAbort, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_store(status + kStPipeFault, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
}

// ---------------------------------------------------------------------------
// attention unit
// ---------------------------------------------------------------------------

constexpr int kTStride = kD + 8;                     // bf16 per staged c^KV row
constexpr int kTCols = kBlock * kHx;                 // 40 columns: col = 8 j + a
constexpr int kTLdsCkv = 0;
constexpr int kTLdsP = kTLdsCkv + kMaxKeys * kTStride * 2;   // P fragments [kk][ct][lane] 16 B
constexpr int kTLdsRed = kTLdsP + 5 * 3 * 1024;              // [max | sum][4 waves][48]
constexpr int kTLdsTurns = kTLdsRed + 2 * 4 * 48 * 4;
constexpr int kTLdsK = kTLdsTurns + (kDr / 2) * 8;
constexpr int kTLds = kTLdsK + 16;

// One block at a time: the block's keys (c^KV rows, ~137 KB) in LDS; the
// 40 columns (query j, head a) as three 16-column tiles, with the block's
// whole q (576 numbers per column, rope part rotated) in registers.  Scores
// are computed transposed (keys x columns): wave w owns key tiles w and
// w + 4 for all three column tiles, and waves 1..3 the ninth key tile
// (keys 128..143) for column tile w - 1, so every A fragment read from LDS
// serves three MFMAs.  The softmax maxima and sums are combined across the
// waves in LDS, the probabilities go to LDS in the B-fragment layout of
// P . c^KV, and for that product wave w owns latent dims 128w .. 128w+127.
__device__ __forceinline__ void role_attn(const FusedArgs& P, int x, char* lds, int32_t* xctl,
                                          uint64_t* waited, int* items, uint32_t* ph) {
    bf16* ckv_l = reinterpret_cast<bf16*>(lds + kTLdsCkv);
    char* p_l = lds + kTLdsP;
    float* red = reinterpret_cast<float*>(lds + kTLdsRed);
    double* turns = reinterpret_cast<double*>(lds + kTLdsTurns);
    int* k_sh = reinterpret_cast<int*>(lds + kTLdsK);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int K = __builtin_amdgcn_readfirstlane(P.status[kStKeptCount]);
    for (int i = tid; i < kDr / 2; i += kFT) turns[i] = P.turns.t[i];

    // this lane's column in each column tile (40..47 are padding and read
    // column 39; their results are never stored)
    int cj[3], ca[3];
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) {
        const int col = min(16 * ct + l16, kTCols - 1);
        cj[ct] = col >> 3;
        ca[ct] = col & 7;
    }
    const size_t ring_elems = (size_t)kR * kFusedSlotElems;
    bf16* oring = P.o_ring + (size_t)x * ring_elems;
    const __amdgpu_buffer_rsrc_t q_rsrc =
        buffer_rsrc(P.q_ring + (size_t)x * ring_elems, (uint32_t)(ring_elems * 2));
    const __amdgpu_buffer_rsrc_t ctx_rsrc = buffer_rsrc(P.ckv_ctx, P.ctx_bytes);
    const __amdgpu_buffer_rsrc_t blk_rsrc = buffer_rsrc(P.ckv_blk, P.blk_bytes);
    const int kt0 = wave, kt1 = wave + 4;
    const int ct8 = wave - 1;                 // column tile of key tile 8 (none for wave 0)
    const float c2 = P.scale * kLog2e;
    const int tr_row = g * 4 + (l16 >> 2);    // transpose-read row inside a 16-key group
    const int tr_col = (l16 & 3) * 4;
    __syncthreads();
    PhaseClock clk{0, ph};
    clk.start();
    // the next block index is fetched one block ahead; the o_lat of a block
    // is announced once the next block's first full wait has completed its
    // stores (or after the loop)
    int k_next = 0;
    if (tid == 0)
        k_next = __hip_atomic_fetch_add(xctl + kCtQueue, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_WORKGROUP);
    int prev_slot = -1;

    for (;;) {
        if (tid == 0) *k_sh = k_next;
        __syncthreads();
        const int k = __builtin_amdgcn_readfirstlane(*k_sh);
        if (k >= K) break;
        ++*items;
        if (tid == 0)
            k_next = __hip_atomic_fetch_add(xctl + kCtQueue, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
        const int slot = k % kR, gen = k / kR;
        const int4 rec = P.srec[k];
        const int blk = rec.w, b = blk / P.N, n = blk % P.N;
        const int ctx_lo = rec.x, ctx_len = rec.y, pos0 = rec.z;
        const int nkeys = ctx_len + kBlock, nkt = (nkeys + 15) >> 4;
        const size_t qrow0 = (size_t)b * P.L5 + (size_t)kBlock * n;

        // ---- keys: slot t < ctx_len is context row ctx_lo + t, then the
        // block's own 5 rows; one 1 KB c^KV row per wave instruction
#pragma unroll
        for (int i = 0; i < (kMaxKeys + 3) / 4; ++i) {
            const int t = wave + 4 * i;
            if (t < nkeys) {
                const bool is_ctx = t < ctx_len;
                const uint32_t row = is_ctx ? (uint32_t)(b * P.S + ctx_lo + t)
                                            : (uint32_t)(qrow0 + (t - ctx_len));
                buffer_copy_16(is_ctx ? ctx_rsrc : blk_rsrc, (row * kD + lane * 8) * 2,
                               &ckv_l[t * kTStride]);
            }
        }
        // k^R A fragments of this wave's key tiles (rope k-steps), rotated
        // in registers: key 16 kt + l16, rope dims 32 r + 8 g .. +7
        auto key_pos = [&](int kt) {
            const int t = min(16 * kt + l16, nkeys - 1);
            return t < ctx_len ? ctx_lo + t : pos0 + (t - ctx_len);
        };
        auto kr_src = [&](int kt) -> const bf16* {
            const int t = min(16 * kt + l16, nkeys - 1);
            return t < ctx_len ? P.kr_ctx + ((size_t)b * P.S + ctx_lo + t) * kDr
                               : P.kr_blk + (qrow0 + (t - ctx_len)) * kDr;
        };
        bf16x8 kra[3][2];
        {
            const bf16* s0 = kr_src(kt0);
            const bf16* s1 = kr_src(kt1);
            const bf16* s8 = kr_src(8);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                kra[0][r] = gld16(s0 + r * 32 + g * 8);
                kra[1][r] = gld16(s1 + r * 32 + g * 8);
                kra[2][r] = gld16(s8 + r * 32 + g * 8);
            }
        }

        // ---- the block's q_abs must be in the ring
        if (!wait_ge(xctl + kCtQReady + slot, kQReadyPer * (gen + 1), xctl, P.status, waited)) return;
        clk.lap(0);
        bf16x8 qf[3][18];
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            const uint32_t qo =
                (uint32_t)(((((size_t)slot * kBlock + cj[ct]) * kHx + ca[ct]) * kD + g * 8) * 2);
#pragma unroll
            for (int ks = 0; ks < kD / 32; ++ks) qf[ct][ks] = ring_ld16(q_rsrc, qo + ks * 64);
            const bf16* qr = P.q_rope + ((qrow0 + cj[ct]) * kH + kHx * x + ca[ct]) * kDr + g * 8;
            qf[ct][16] = gld16(qr);
            qf[ct][17] = gld16(qr + 32);
        }
        VM_WAIT(0);
        ctl_add(xctl + kCtQFree + slot, 1);       // the ring slot's q_abs is no longer needed
        if (prev_slot >= 0) ctl_add(xctl + kCtOReady + prev_slot, 1);   // its stores completed
        // rotate q^R (position pos0 + j) and k^R in registers
        auto rotate = [&](bf16x8& v, int pos, int r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 cs = rope_cs(turns, pos, r * 16 + g * 4 + q);
                const float x0 = (float)v[2 * q], x1 = (float)v[2 * q + 1];
                v[2 * q] = (bf16)(x0 * cs.x - x1 * cs.y);
                v[2 * q + 1] = (bf16)(x0 * cs.y + x1 * cs.x);
            }
        };
#pragma unroll
        for (int r = 0; r < 2; ++r) {
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) rotate(qf[ct][16 + r], pos0 + cj[ct], r);
            rotate(kra[0][r], key_pos(kt0), r);
            rotate(kra[1][r], key_pos(kt1), r);
            rotate(kra[2][r], key_pos(8), r);
        }
        __syncthreads();                          // the keys are in LDS
        clk.lap(1);

        // ---- scores (transposed): st[i][ct] = keys of tile kt_i x column tile ct
        const bool act0 = kt0 < nkt, act1 = kt1 < nkt, act8 = (wave >= 1) && (nkt > 8);
        const int krow0 = min(16 * kt0 + l16, nkeys - 1);
        const int krow1 = min(16 * kt1 + l16, nkeys - 1);
        const int krow8 = min(128 + l16, nkeys - 1);
        // latent k-steps read c^KV in the permuted order q_abs is stored in
        auto afrag = [&](int krow, int ks) -> bf16x8 {
            const bf16* ap = &ckv_l[krow * kTStride + ks * 32 + g * 4];
            return cat(ld8(ap), ld8(ap + 16));
        };
        f32x4 st[2][3], st8 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) st[i][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            bf16x8 a0, a1, a8;
            if (ks < 16) {
                a0 = afrag(krow0, ks);
                a1 = afrag(krow1, ks);
                a8 = afrag(krow8, ks);
            } else {
                a0 = kra[0][ks - 16];
                a1 = kra[1][ks - 16];
                a8 = kra[2][ks - 16];
            }
            const bf16x8 q8 = (ct8 == 0) ? qf[0][ks] : (ct8 == 1) ? qf[1][ks] : qf[2][ks];
            if (act0) {
#pragma unroll
                for (int ct = 0; ct < 3; ++ct) st[0][ct] = mfma_16x16x32(a0, qf[ct][ks], st[0][ct]);
            }
            if (act1) {
#pragma unroll
                for (int ct = 0; ct < 3; ++ct) st[1][ct] = mfma_16x16x32(a1, qf[ct][ks], st[1][ct]);
            }
            if (act8) st8 = mfma_16x16x32(a8, q8, st8);
        }

        clk.lap(2);
        // ---- softmax over the block's keys, columns combined across waves.
        // Keys past nkeys (and tiles not computed) are -inf.
        const float ninf = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool v0 = act0 && (16 * kt0 + 4 * g + i < nkeys);
            const bool v1 = act1 && (16 * kt1 + 4 * g + i < nkeys);
            const bool v8 = act8 && (128 + 4 * g + i < nkeys);
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) {
                st[0][ct][i] = v0 ? st[0][ct][i] : ninf;
                st[1][ct][i] = v1 ? st[1][ct][i] : ninf;
            }
            st8[i] = v8 ? st8[i] : ninf;
        }
        float mcol[3];
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            float m = ninf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                m = fmaxf(m, fmaxf(st[0][ct][i], st[1][ct][i]));
                if (ct8 == ct) m = fmaxf(m, st8[i]);
            }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (g == 0) red[wave * 48 + 16 * ct + l16] = m;
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            float m = red[16 * ct + l16];
#pragma unroll
            for (int w = 1; w < 4; ++w) m = fmaxf(m, red[w * 48 + 16 * ct + l16]);
            mcol[ct] = m * c2;
        }
        auto put_p = [&](int kt, int ct, const f32x4& s, float& sum) {
            bf16x4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -mcol[ct]));
                pv[i] = (bf16)p;
                sum += p;
            }
            *reinterpret_cast<bf16x4*>(p_l + (((kt >> 1) * 3 + ct) * 64 + lane) * 16 +
                                       (kt & 1) * 8) = pv;
        };
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            float sum = 0.f;
            put_p(kt0, ct, st[0][ct], sum);
            put_p(kt1, ct, st[1][ct], sum);
            if (ct8 == ct) put_p(8, ct, st8, sum);
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            if (g == 0) red[4 * 48 + wave * 48 + 16 * ct + l16] = sum;
        }
        __syncthreads();
        float inv[3];
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            float sm = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) sm += red[4 * 48 + w * 48 + 16 * ct + l16];
            inv[ct] = __builtin_amdgcn_rcpf(sm);     // sm >= 1 (the maximum contributes 1)
        }

        // ---- o_lat^T = c^KV^T P^T for latent dims 128 wave .. +127: lane
        // holds dims 128 wave + 16 mt + 4 g + i of column 16 ct + l16
        const int nkk = (nkt + 1) >> 1;
        f32x4 o[8][3];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) o[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 5; ++kk) {
            if (kk < nkk) {
                const int r0 = min(32 * kk + tr_row, nkeys - 1);
                const int r1 = min(32 * kk + 16 + tr_row, nkeys - 1);
                bf16x8 pb[3];
#pragma unroll
                for (int ct = 0; ct < 3; ++ct)
                    pb[ct] = *reinterpret_cast<const bf16x8*>(p_l + ((kk * 3 + ct) * 64 + lane) * 16);
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const int col = 128 * wave + 16 * mt + tr_col;
                    const bf16x4 lo = lds_read_tr(&ckv_l[r0 * kTStride + col]);
                    if (kk < 4) {
                        const bf16x8 v = cat(lo, lds_read_tr(&ckv_l[r1 * kTStride + col]));
#pragma unroll
                        for (int ct = 0; ct < 3; ++ct) o[mt][ct] = mfma_16x16x32(v, pb[ct], o[mt][ct]);
                    } else {
#pragma unroll
                        for (int ct = 0; ct < 3; ++ct)
                            o[mt][ct] = mfma_16x16x16(
                                lo, __builtin_shufflevector(pb[ct], pb[ct], 0, 1, 2, 3), o[mt][ct]);
                    }
                }
            }
        }

        clk.lap(2);
        // ---- o_lat into the o ring once the W_UV units have read the
        // slot's previous block
        if (!wait_ge(xctl + kCtOFree + slot, kOFreePer * gen, xctl, P.status, waited)) return;
#pragma unroll
        for (int ct = 0; ct < 3; ++ct) {
            const int col = 16 * ct + l16;
            if (col < kTCols) {
                bf16* dst = oring + (((size_t)slot * kBlock + (col >> 3)) * kHx + (col & 7)) * kD +
                            128 * wave + g * 8;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    bf16x8 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = (bf16)(o[2 * pp][ct][i] * inv[ct]);
                        v[4 + i] = (bf16)(o[2 * pp + 1][ct][i] * inv[ct]);
                    }
                    gst16(dst + 32 * pp, v);
                }
            }
        }
        prev_slot = slot;
        clk.lap(3);
    }
    VM_WAIT(0);
    if (prev_slot >= 0) ctl_add(xctl + kCtOReady + prev_slot, 1);
}

// ---------------------------------------------------------------------------
// absorb unit: q_abs[r][h] = W_UK[h]^T q^C[r][h] for every kept row r
// ---------------------------------------------------------------------------

constexpr int kARows = 64;                 // rows per iteration
constexpr int kATiles = kARows / 16;
constexpr int kAKs = kDc / 32;             // 6 k-steps
constexpr int kADt = 8;                    // 16-dim output tiles per wave (128 dims)
constexpr int kAWStride = 256 + 16;        // bf16 per staged weight row (one 256-dim part)
constexpr int kABuf = kATiles * kAKs * 1024;
constexpr int kALds = (kDc * kAWStride * 2 > 2 * kABuf) ? kDc * kAWStride * 2 : 2 * kABuf;

// Wave w computes output dims 128w .. 128w+127 transposed (dims x rows) with
// its 128 x 192 slice of W_UK[h]^T resident in registers (staged through LDS
// at start and read transposed).  Per 64-row iteration the q^C rows are
// copied into LDS already in the B-fragment layout (wave w copies row tile
// w), double buffered; results go to the q ring as 16 bytes per lane (the
// permuted order the attention unit reads).
__device__ __forceinline__ void role_absorb(const FusedArgs& P, int x, int a, char* lds,
                                            int32_t* xctl, uint64_t* waited, int* items,
                                            uint32_t* ph) {
    const int h = kHx * x + a;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    bf16x8 aw[kAKs][kADt];
    {
        bf16* wl = reinterpret_cast<bf16*>(lds);
        // full-wave copies that fill the padded [c][272] layout contiguously:
        // lane l's 16 bytes land at byte 1024 i + 16 l, i.e. row (1024 i +
        // 16 l) / 544; lanes that land in a row's padding fetch any element
        // of that row.  (Every copy has one LDS base for the whole wave.)
        constexpr int kRowBytes = 2 * kAWStride;
        constexpr int kCopies = kDc * kRowBytes / 1024;
        static_assert(kDc * kRowBytes % 1024 == 0, "whole copies");
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            for (int i = wave; i < kCopies; i += 4) {
                const int off = 1024 * i + 16 * lane;
                const int c = off / kRowBytes, cb = off % kRowBytes;
                const int col = (cb < 512) ? cb / 2 : 0;
                async_copy_16(P.w_uk + ((size_t)h * kDc + c) * kD + part * 256 + col,
                              lds + 1024 * i);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm0Lgkm0);
            __syncthreads();
            if ((wave >> 1) == part) {
                const int wd = wave & 1;
#pragma unroll
                for (int ks = 0; ks < kAKs; ++ks)
#pragma unroll
                    for (int dt = 0; dt < kADt; ++dt) {
                        const bf16* ab = wl + (ks * 32 + g * 8 + (l16 >> 2)) * kAWStride +
                                         wd * 128 + (l16 & 3) * 4 + dt * 16;
                        aw[ks][dt] = cat(lds_read_tr(ab), lds_read_tr(ab + 4 * kAWStride));
                    }
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __syncthreads();
        }
    }

    const int K = __builtin_amdgcn_readfirstlane(P.status[kStKeptCount]);
    const int rows = kBlock * K;
    const int n_iter = (rows + kARows - 1) / kARows;
    bf16* qring = P.q_ring + (size_t)x * kR * kFusedSlotElems;
    const i32x4 q_rs = rsrc_words(P.q_nope, P.q_bytes);
    char* const buf0 = lds;
    char* const buf1 = lds + kABuf;

    // copy of iteration it: wave w copies row tile w (rows past the end
    // repeat the last row); the tile's 16 rows span at most 4 kept blocks
    auto stage = [&](int it, char* dst) {
        const int rfirst = min(it * kARows + 16 * wave, rows - 1);
        const int kb = rfirst / kBlock;
        const i32x4 kv = sld4(P.kept + kb);
        const int r = min(it * kARows + 16 * wave + l16, rows - 1);
        const int d = r / kBlock - kb;
        const int blk = d == 0 ? kv[0] : d == 1 ? kv[1] : d == 2 ? kv[2] : kv[3];
        const int b = blk / P.N, n = blk % P.N;
        const uint32_t off = (uint32_t)(
            ((((size_t)b * P.L5 + (size_t)kBlock * n + r % kBlock) * kH + h) * kDc + g * 8) * 2);
#pragma unroll
        for (int ks = 0; ks < kAKs; ++ks)
            copy_16_untracked(q_rs, off + ks * 64, dst + (wave * kAKs + ks) * 1024);
    };

    *items = n_iter;
    CtlView qfree_view{xctl + kCtQFree, 0};
    PhaseClock clk{0, ph};
    clk.start();
    if (n_iter > 0) stage(0, buf0);
    int sig = 0;                       // kept blocks whose q_abs this wave has announced
    for (int it = 0; it < n_iter; ++it) {
        char* const cur = (it & 1) ? buf1 : buf0;
        char* const nxt = (it & 1) ? buf0 : buf1;
        // this iteration's copy has landed (the stores of iteration it-1, at
        // most 16, may still be in flight; everything older has completed)
        if (it == 0) VM_WAIT(0); else VM_WAIT(16);
        __syncthreads();
        clk.lap(0);
        if (it >= 2) {
            const int done = min((it - 1) * kARows, rows) / kBlock;
            for (; sig < done; ++sig) ctl_add(xctl + kCtQReady + sig % kR, 1);
        }
        if (it + 1 < n_iter) stage(it + 1, nxt);
        clk.lap(1);

        f32x4 acc[kADt][kATiles];
#pragma unroll
        for (int dt = 0; dt < kADt; ++dt)
#pragma unroll
            for (int t = 0; t < kATiles; ++t) acc[dt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kAKs; ++ks) {
            bf16x8 bq[kATiles];
#pragma unroll
            for (int t = 0; t < kATiles; ++t)
                bq[t] = *reinterpret_cast<const bf16x8*>(cur + (t * kAKs + ks) * 1024 + lane * 16);
#pragma unroll
            for (int dt = 0; dt < kADt; ++dt)
#pragma unroll
                for (int t = 0; t < kATiles; ++t) acc[dt][t] = mfma_16x16x32(aw[ks][dt], bq[t], acc[dt][t]);
        }

        clk.lap(2);
        // the ring slots of this iteration's blocks must have been consumed
        // in their previous use
        const int kb0 = (it * kARows) / kBlock;
        const int kb1 = min((it * kARows + kARows - 1) / kBlock, K - 1);
        for (int kk = kb0; kk <= kb1; ++kk)
            if (!view_wait(qfree_view, kk % kR, kQFreePer * (kk / kR), xctl, P.status, waited))
                return;
        // lane holds dims 128 wave + 16 dt + 4 g + i of row 16 t + l16; dims
        // 32pp + 4g + i (tile 2pp) and 32pp + 16 + 4g + i (tile 2pp + 1) go to
        // stored positions 32pp + 8g .. +7
#pragma unroll
        for (int t = 0; t < kATiles; ++t) {
            const int r = it * kARows + 16 * t + l16;
            if (r < rows) {
                const int s = (r / kBlock) % kR;
                bf16* dst = qring + (((size_t)s * kBlock + r % kBlock) * kHx + a) * kD + 128 * wave +
                            g * 8;
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const f32x4 a0 = acc[2 * pp][t], a1 = acc[2 * pp + 1][t];
                    bf16x8 v;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[i] = (bf16)a0[i];
                        v[4 + i] = (bf16)a1[i];
                    }
                    gst16(dst + 32 * pp, v);
                }
            }
        }
        clk.lap(3);
    }
    VM_WAIT(0);
    for (; sig < K; ++sig) ctl_add(xctl + kCtQReady + sig % kR, 1);
}

// ---------------------------------------------------------------------------
// W_UV unit: out[b, q, h, :] = W_UV[h] o_lat[r][h] for every kept row r
// ---------------------------------------------------------------------------

constexpr int kURows = 32;                 // rows per iteration
constexpr int kUSlots = 3;                 // LDS ring of staged iterations
constexpr int kUStride = kD * 2 + 16;      // bytes per staged o_lat row
constexpr int kUSlotBytes = kURows * kUStride;
constexpr int kULds = kUSlots * kUSlotBytes;
constexpr int kUCopies = kURows / 4;       // copies per wave and iteration

// Wave w computes output dims 64w .. 64w+63 transposed with its 64 x 512
// slice of W_UV[h] resident in registers (rows permuted so that each lane
// ends up with 8 consecutive output dims).  o_lat rows are copied from the o
// ring into LDS (one 1 KB row per instruction) two iterations ahead.
__device__ __forceinline__ void role_uv(const FusedArgs& P, int x, int a, char* lds,
                                        int32_t* xctl, uint64_t* waited, int* items,
                                        uint32_t* ph) {
    const int h = kHx * x + a;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;

    // A fragment (ks, q), q = 2 q2 + vt: row m = l16 is output dim
    // 64 wave + 32 q2 + 8 (m / 4) + 4 vt + m % 4; k-values follow the
    // permuted o_lat order (dims 32ks + 4g + 0..3 and 32ks + 16 + 4g + 0..3)
    bf16x8 aw[kD / 32][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bf16* wrow = P.w_uv + ((size_t)h * kDv + 64 * wave + 32 * (q >> 1) + 8 * (l16 >> 2) +
                                     4 * (q & 1) + (l16 & 3)) * kD + 4 * g;
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) aw[ks][q] = cat(gld8(wrow + 32 * ks), gld8(wrow + 32 * ks + 16));
    }
    VM_WAIT(0);                        // before any copy is in flight

    const int K = __builtin_amdgcn_readfirstlane(P.status[kStKeptCount]);
    const int rows = kBlock * K;
    const int n_iter = (rows + kURows - 1) / kURows;
    const size_t ring_elems = (size_t)kR * kFusedSlotElems;
    const i32x4 o_rs = rsrc_words(P.o_ring + (size_t)x * ring_elems, (uint32_t)(ring_elems * 2));

    CtlView oready_view{xctl + kCtOReady, 0};
    // wave w copies rows 8w .. 8w+7 of the iteration, after the attention
    // units have written them; rows past the end read nothing (offsets
    // outside the buffer resource) so that every iteration issues the same
    // number of copies
    auto stage = [&](int it) -> bool {
        const int r_lo = it * kURows + kUCopies * wave;
        const int r_hi = min(r_lo + kUCopies, rows) - 1;
        for (int kb = r_lo / kBlock; kb <= r_hi / kBlock && r_lo <= r_hi; ++kb)
            if (!view_wait(oready_view, kb % kR, kOReadyPer * (kb / kR + 1), xctl, P.status,
                           waited))
                return false;
        char* dst = lds + (it % kUSlots) * kUSlotBytes;
#pragma unroll
        for (int q = 0; q < kUCopies; ++q) {
            const int lr = kUCopies * wave + q;
            const int r = it * kURows + lr;
            const uint32_t off =
                (r < rows) ? (uint32_t)((((size_t)((r / kBlock) % kR) * kBlock + r % kBlock) * kHx + a) *
                                            kD * 2 + lane * 16)
                           : 0xFFFFFFF0u;
            copy_ring_16(o_rs, off, dst + lr * kUStride);
        }
        return true;
    };

    *items = n_iter;
    PhaseClock clk{0, ph};
    clk.start();
    if (n_iter > 0 && !stage(0)) return;
    if (n_iter > 1 && !stage(1)) return;
    int sig = 0;                       // kept blocks whose o_lat rows this wave has released
    for (int it = 0; it < n_iter; ++it) {
        // this iteration's copy has landed: after it were issued at most the
        // next iteration's copies and the previous iteration's stores
        if (it == 0) {
            if (n_iter > 1) VM_WAIT(8); else VM_WAIT(0);
        } else if (it + 1 < n_iter) {
            VM_WAIT(12);
        } else {
            VM_WAIT(4);            // no copy was issued after this one's successor
        }
        __syncthreads();
        clk.lap(0);
        {
            const int done = min((it + 1) * kURows, rows) / kBlock;
            for (; sig < done; ++sig) ctl_add(xctl + kCtOFree + sig % kR, 1);
        }
        if (it + 2 < n_iter && !stage(it + 2)) return;
        clk.lap(1);

        const char* cur = lds + (it % kUSlots) * kUSlotBytes;
        f32x4 acc[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[q][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < kD / 32; ++ks) {
            bf16x8 bv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                bv[t] = *reinterpret_cast<const bf16x8*>(cur + (16 * t + l16) * kUStride + ks * 64 + g * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int t = 0; t < 2; ++t) acc[q][t] = mfma_16x16x32(aw[ks][q], bv[t], acc[q][t]);
        }
        clk.lap(2);
        // lane holds output dims 64 wave + 32 q2 + 8 g .. +7 of row 16 t + l16
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r0 = it * kURows + 16 * t;
            if (r0 < rows) {
                const int kb = r0 / kBlock;
                const i32x4 kv = sld4(P.kept + kb);
                const int r = it * kURows + 16 * t + l16;
                if (r < rows) {
                    const int d = r / kBlock - kb;
                    const int blk = d == 0 ? kv[0] : d == 1 ? kv[1] : d == 2 ? kv[2] : kv[3];
                    const int b = blk / P.N, n = blk % P.N;
                    bf16* dst = P.out + (((size_t)b * P.L5 + (size_t)kBlock * n + r % kBlock) * kH + h) * kDv +
                                64 * wave + 8 * g;
#pragma unroll
                    for (int q2 = 0; q2 < 2; ++q2) {
                        bf16x8 v;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            v[i] = (bf16)acc[2 * q2][t][i];
                            v[4 + i] = (bf16)acc[2 * q2 + 1][t][i];
                        }
                        gst16(dst + 32 * q2, v);
                    }
                }
            }
        }
        clk.lap(3);
    }
    VM_WAIT(0);
}

constexpr int kFusedLds = (kTLds > kALds ? (kTLds > kULds ? kTLds : kULds)
                                         : (kALds > kULds ? kALds : kULds));

__global__ __launch_bounds__(kFT) void fused_kernel(FusedArgs P) {
    __shared__ __attribute__((aligned(16))) char lds[kFusedLds];
    __shared__ int rank_sh;
    const int x = xcc_id();
    int32_t* xctl = P.ctl + x * kFusedCtlStride;
    if (threadIdx.x == 0)
        rank_sh = __hip_atomic_fetch_add(xctl + kCtTicket, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    const int r = rank_sh;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint64_t waited = 0;
    int items = 0;
    uint32_t ph[4] = {0, 0, 0, 0};
    if (r < kNA)
        role_absorb(P, x, r, lds, xctl, &waited, &items, ph);
    else if (r < kNA + kNU)
        role_uv(P, x, r - kNA, lds, xctl, &waited, &items, ph);
    else if (r < kRanks)
        role_attn(P, x, lds, xctl, &waited, &items, ph);
    // timing words of this unit (wave 0): role, busy and waiting 10 ns ticks,
    // work items, and the ticks of four phases of the unit's loop
    if (threadIdx.x == 0 && r < kRanks) {
        int32_t* tw = xctl + kCtTiming + 8 * r;
        tw[0] = r < kNA ? 1 : (r < kNA + kNU ? 2 : 3);
        tw[1] = (int32_t)(__builtin_amdgcn_s_memrealtime() - t0);
        tw[2] = (int32_t)waited;
        tw[3] = items;
        for (int i = 0; i < 4; ++i) tw[4 + i] = (int32_t)ph[i];
    }
}

}  // namespace

int fused_threads() { return kFT; }
const void* fused_kernel_fn() { return reinterpret_cast<const void*>(&fused_kernel); }

hipError_t launch_fused(const Problem& p, const Inputs& in, const Workspace& ws,
                        const RopeTheta& th, hipStream_t s) {
    FusedArgs a;
    a.q_nope = (const bf16*)in.q_nope;
    a.q_rope = (const bf16*)in.q_rope;
    a.ckv_ctx = (const bf16*)in.ckv_ctx;
    a.kr_ctx = (const bf16*)in.kr_ctx;
    a.ckv_blk = (const bf16*)in.ckv_blk;
    a.kr_blk = (const bf16*)in.kr_blk;
    a.w_uk = (const bf16*)in.w_uk;
    a.w_uv = (const bf16*)in.w_uv;
    a.kept = ws.kept;
    a.srec = ws.srec;
    a.status = ws.status;
    a.ctl = ws.ctl;
    a.q_ring = ws.qring;
    a.o_ring = ws.oring;
    a.out = (bf16*)in.out;
    a.S = p.S;
    a.N = p.N;
    a.L5 = p.L5;
    a.scale = p.scale;
    a.ctx_bytes = (uint32_t)((size_t)p.B * p.S * kD * sizeof(bf16));
    a.blk_bytes = (uint32_t)((size_t)p.B * p.L5 * kD * sizeof(bf16));
    a.q_bytes = (uint32_t)((size_t)p.B * p.L5 * kH * kDc * sizeof(bf16));
    a.turns = RopeTheta{};
    for (int k = 0; k < kDr / 2; ++k) a.turns.t[k] = th.t[k] * 0.15915494309189533577;   // 1 / 2pi
    hipLaunchKernelGGL(fused_kernel, dim3(kFusedCus), dim3(kFT), 0, s, a);
    return hipGetLastError();
}

}  // namespace dspark
