// extern "C" entry points of libdspark_attn.so: argument validation,
// workspace layout, kernel launches.  See include/dspark_attn.h.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "bwd.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

thread_local std::string g_last_error;

dspark_status fail(dspark_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

dspark_status ok() {
    g_last_error.clear();
    return DSPARK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The MFMA path addresses q^C and c^KV through buffer resources with 32-bit
// byte offsets, so each must stay below 4 GiB (B * 5N <= 174762 query rows,
// B * S < 4M context rows).
bool is_fast_path(const dspark_attn_desc& d) {
    const size_t q_bytes = (size_t)d.B * kBlock * d.N * kH * kDc * 2;
    const size_t ctx_bytes = (size_t)d.B * d.S * kD * 2;
    return d.dtype == DSPARK_BF16 && d.n_heads == kH && d.d_latent == kD && d.d_nope == kDc &&
           d.d_rope == kDr && d.d_v == kDv && d.window <= kMaxWindow &&
           q_bytes < (1ull << 32) && ctx_bytes < (1ull << 32);
}

// Validates the descriptor; `empty` is set when there is nothing to compute.
dspark_status check_desc(const dspark_attn_desc* d, bool* empty) {
    if (!d) return fail(DSPARK_EINVAL, "desc is NULL");
    if (d->block != kBlock)
        return fail(DSPARK_EUNSUPPORTED, "block must be 5 (got %d)", d->block);
    if (d->B < 0 || d->N < 0) return fail(DSPARK_EINVAL, "B and N must be >= 0");
    if (d->S < 1) return fail(DSPARK_EINVAL, "S must be >= 1 (got %d)", d->S);
    if (d->window < 1) return fail(DSPARK_EINVAL, "window must be >= 1 (got %d)", d->window);
    if (d->n_heads < 1 || d->d_latent < 1 || d->d_nope < 1 || d->d_v < 1 || d->d_rope < 0)
        return fail(DSPARK_EINVAL, "n_heads, d_latent, d_nope, d_v must be >= 1, d_rope >= 0");
    if (d->d_rope % 2 != 0) return fail(DSPARK_EINVAL, "d_rope must be even (got %d)", d->d_rope);
    if (d->d_rope / 2 > kMaxRopePairs)
        return fail(DSPARK_EUNSUPPORTED, "d_rope must be <= %d", 2 * kMaxRopePairs);
    if (d->dtype != DSPARK_F32 && d->dtype != DSPARK_BF16)
        return fail(DSPARK_EINVAL, "dtype must be DSPARK_F32 or DSPARK_BF16 (got %d)", d->dtype);
    if (!(d->rope_base > 0.0) || !std::isfinite(d->rope_base))
        return fail(DSPARK_EINVAL, "rope_base must be a finite positive number");
    if (!std::isfinite(d->softmax_scale))
        return fail(DSPARK_EINVAL, "softmax_scale must be finite");
    const long long blocks = (long long)d->B * d->N;
    if (blocks > (1LL << 26))
        return fail(DSPARK_EUNSUPPORTED, "B*N = %lld exceeds 2^26 blocks", blocks);
    if ((long long)d->S + 8 > (1LL << 30)) return fail(DSPARK_EUNSUPPORTED, "S too large");
    if (d->n_heads > 65535) return fail(DSPARK_EUNSUPPORTED, "n_heads must be <= 65535");
    *empty = blocks == 0;
    return DSPARK_OK;
}

// Kept blocks per kernel round.  By default one round covers every block:
// each kernel's grid is sized for the whole problem, and smaller rounds
// (which would keep a round's q_abs / o_lat, 640 KiB per block, inside the
// 256 MB Infinity Cache) leave the 256 CUs under-filled and pay each
// launch's weight staging again, which costs more than the cache saves.
int chunk_blocks(const dspark_attn_desc& d, const dspark_attn_opts* opts) {
    const int blocks = d.B * d.N;
    const int c = (opts && opts->chunk_blocks > 0) ? opts->chunk_blocks : blocks;
    return c < blocks ? c : blocks;
}

Problem make_problem(const dspark_attn_desc& d) {
    Problem p;
    p.B = d.B; p.S = d.S; p.N = d.N; p.W = d.window; p.H = d.n_heads;
    p.D = d.d_latent; p.dc = d.d_nope; p.dr = d.d_rope; p.dv = d.d_v;
    p.L5 = kBlock * d.N;
    p.scale = (float)(d.softmax_scale > 0.0 ? d.softmax_scale
                                            : 1.0 / std::sqrt((double)(d.d_nope + d.d_rope)));
    return p;
}

Workspace carve(void* base, const WsLayout& L) {
    char* c = static_cast<char*>(base);
    Workspace w;
    w.idx = reinterpret_cast<int4*>(c + L.idx);
    w.kept = reinterpret_cast<int32_t*>(c + L.kept);
    w.srec = reinterpret_cast<int4*>(c + L.srec);
    w.status = reinterpret_cast<int32_t*>(c + L.status);
    w.rope = reinterpret_cast<float2*>(c + L.rope);
    w.qabs = L.qabs ? reinterpret_cast<bf16*>(c + L.qabs) : nullptr;
    w.olat = L.olat ? reinterpret_cast<bf16*>(c + L.olat) : nullptr;
    w.ctl = L.ctl ? reinterpret_cast<int32_t*>(c + L.ctl) : nullptr;
    w.qring = L.qring ? reinterpret_cast<bf16*>(c + L.qring) : nullptr;
    w.oring = L.oring ? reinterpret_cast<bf16*>(c + L.oring) : nullptr;
    return w;
}

dspark_status check_workspace(const void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return fail(DSPARK_EWORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
        return fail(DSPARK_EWORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace too small: %zu bytes given, %zu needed",
                    ws_bytes, need);
    return DSPARK_OK;
}

dspark_status hip_fail(hipError_t e, const char* what) {
    return fail(DSPARK_EHIP, "%s: %s", what, hipGetErrorString(e));
}

BwdWork carve_bwd(void* base, const BwdLayout& L) {
    char* c = static_cast<char*>(base);
    BwdWork w;
    w.fwd = carve(base, L.fwd);
    auto at = [&](size_t off) { return off ? c + off : nullptr; };
    w.dolat = reinterpret_cast<bf16*>(at(L.dolat));
    w.dqabs = reinterpret_cast<bf16*>(at(L.dqabs));
    w.qrot = reinterpret_cast<bf16*>(at(L.qrot));
    w.pmat = reinterpret_cast<bf16*>(at(L.pmat));
    w.dsmat = reinterpret_cast<bf16*>(at(L.dsmat));
    w.part = reinterpret_cast<float*>(at(L.part));
    w.acc = reinterpret_cast<float*>(c + L.acc);
    w.wacc = reinterpret_cast<float*>(at(L.wacc));
    return w;
}

// launches of dspark_attn_bwd_ex: index, anchor-order check, accumulator
// clear (a no-op unless the anchors are unsorted), absorb, d_olat,
// attention, dc^KV, dq^C, dW, final (MFMA path); index + RoPE table, clear,
// generic kernel, final (generic path)
constexpr int kBwdLaunchesFast = 10, kBwdLaunchesGeneric = 4;

RopeTheta make_theta(const dspark_attn_desc& d) {
    RopeTheta th;
    std::memset(&th, 0, sizeof(th));
    for (int i = 0; i < d.d_rope / 2; ++i)
        th.t[i] = std::pow(d.rope_base, -2.0 * i / (double)d.d_rope);
    return th;
}

// Forward paths: the generic fp32 kernels (any shape), the three MFMA
// kernels with q_abs / o_lat materialised in the workspace, and the fused
// one-launch pipeline (GLM dims, 256 compute units).
enum class FwdPath { kGeneric, kMaterialised, kFused };

// The fused launch needs every one of its 256 workgroups resident at once
// (one per compute unit) on an 8-XCD device.  Answered once per device.
bool fused_device_ok() {
    static std::atomic<int8_t> known[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
    if (dev < 64) {
        const int8_t k = known[dev].load(std::memory_order_relaxed);
        if (k != 0) return k == 1;
    }
    int cus = 0, nb = 0;
    bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                  hipSuccess &&
              cus == kFusedCus &&
              hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fused_kernel_fn(),
                                                           fused_threads(), 0) == hipSuccess &&
              nb >= 1;
    (void)hipGetLastError();
    if (dev < 64) known[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

FwdPath pick_path(const dspark_attn_desc& d, const dspark_attn_opts* o, bool check_device) {
    if (!is_fast_path(d) || (o && o->force_generic)) return FwdPath::kGeneric;
    if (!o || !o->one_launch || o->chunk_blocks > 0 || o->aux_stream)
        return FwdPath::kMaterialised;
    if (check_device && !fused_device_ok()) return FwdPath::kMaterialised;
    return FwdPath::kFused;
}

// status[kStPathTag] written by a forward on the given path: a hash of the
// descriptor with the path in its low three bits (never 0); with_p: the
// forward also left its softmax probabilities for the backward.  A backward
// with reuse_forward expects the tag of the path it takes.
int32_t forward_tag(const dspark_attn_desc& d, FwdPath path, bool with_p = false) {
    uint32_t h = 2166136261u;
    auto mix = [&](const void* v, size_t n) {
        const unsigned char* c = static_cast<const unsigned char*>(v);
        for (size_t i = 0; i < n; ++i) h = (h ^ c[i]) * 16777619u;
    };
    const int32_t f[] = {d.B, d.S, d.N, d.window, d.n_heads, d.d_latent, d.d_nope, d.d_rope,
                         d.d_v, d.dtype};
    mix(f, sizeof(f));
    mix(&d.rope_base, sizeof(d.rope_base));
    mix(&d.softmax_scale, sizeof(d.softmax_scale));
    const uint32_t code = path == FwdPath::kMaterialised ? (with_p ? 4u : 1u)
                          : path == FwdPath::kGeneric    ? 2u
                                                         : 3u;
    return (int32_t)((h & ~7u) | code);
}

WsLayout path_layout(const dspark_attn_desc& d, FwdPath path) {
    return ws_layout(d, path == FwdPath::kMaterialised, path == FwdPath::kFused);
}


// ---------------------------------------------------------------------------
// the allocation-free forward: a fixed scratch array on every device
// ---------------------------------------------------------------------------

constexpr size_t kFixedScratchBytes = DSPARK_NOALLOC_SCRATCH_BYTES;
static_assert(kFixedScratchBytes % 256 == 0, "scratch size must be a multiple of 256");

// Held by every device the library runs on until the process ends.  In host
// code this name is only a stand-in for the symbol: kernels are given the
// address scratch_address() looked up for the current device.
static __device__ __align__(256) unsigned char scratch[kFixedScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
dspark_status scratch_address(void** out) {
    static std::mutex mu;
    static void* addr[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(DSPARK_EUNSUPPORTED, "device ordinal %d >= 64", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
        if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0)
            return fail(DSPARK_EHIP, "scratch array address %p is not 256-byte aligned", ptr);
        addr[dev] = ptr;
    }
    *out = addr[dev];
    return DSPARK_OK;
}

// Per-block bytes of q_abs plus o_lat on the MFMA path (5 query rows x H x D
// bf16, twice).
size_t latent_bytes_per_block(const dspark_attn_desc& d) {
    return 2 * (size_t)kBlock * d.n_heads * d.d_latent * 2;
}

// Layout of the fixed scratch: the index for every block as in the
// caller-workspace layout, then on the MFMA path the q_abs / o_lat rows of
// one round of *round_blocks kept blocks (as many as fit; no RoPE table,
// which that path does not read), on the generic path the RoPE table.  A
// total above kFixedScratchBytes means the shape does not fit.
WsLayout fixed_layout(const dspark_attn_desc& d, bool mfma, int* round_blocks) {
    WsLayout L = ws_layout(d, false);
    *round_blocks = 0;
    if (!mfma) return L;
    const size_t per = latent_bytes_per_block(d);
    const size_t index_end = L.rope;
    const size_t room = kFixedScratchBytes > index_end + 512 ? kFixedScratchBytes - index_end - 512
                                                             : 0;
    const long long blocks = (long long)d.B * d.N;
    long long r = (long long)(room / per);
    if (r > blocks) r = blocks;
    if (r < 1) r = 1;   // one block: the total then tells whether it fits
    *round_blocks = (int)r;
    const size_t lat = (size_t)r * per / 2;
    L.rope_rows = 0;
    L.qabs = index_end;
    L.olat = align256(L.qabs + lat);
    L.total = align256(L.olat + lat);
    return L;
}

// The workspace a round of kept slots [slot0, ...) sees when its latent rows
// start at the beginning of the latent area: the kernels address row
// 5 * slot + query, so the bases move back by slot0 blocks.  The shifted
// bases are only ever offset forward again by at least slot0 blocks.
Workspace round_latents(Workspace w, const Problem& p, int slot0) {
    const uintptr_t back = (uintptr_t)slot0 * kBlock * p.H * p.D * sizeof(bf16);
    w.qabs = reinterpret_cast<bf16*>(reinterpret_cast<uintptr_t>(w.qabs) - back);
    w.olat = reinterpret_cast<bf16*>(reinterpret_cast<uintptr_t>(w.olat) - back);
    return w;
}

// The forward behind dspark_attn_fwd_ex and dspark_attn_fwd_noalloc.  With
// `fixed` set, the workspace is the library's per-device scratch array: the
// MFMA path then runs in rounds whose q_abs / o_lat rows start at the array's
// latent area (rows are addressed relative to the round), one round after
// another on `stream`.
struct FixedScratch {
    void* base;         // device address of the array on the current device
    int32_t* status;    // the caller's status words, or NULL
};

dspark_status forward_impl(const dspark_attn_desc* desc, const void* q_nope, const void* q_rope,
                           const void* ckv_ctx, const void* kr_ctx, const void* ckv_blk,
                           const void* kr_blk, const void* w_uk, const void* w_uv,
                           const int32_t* anchors, const uint8_t* keep, void* out,
                           void* workspace, size_t ws_bytes, void* stream,
                           const dspark_attn_opts* opts, const FixedScratch* fixed) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    if (empty) return ok();
    const dspark_attn_desc& d = *desc;
    const void* ptrs[] = {q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                          anchors, keep, out};
    const char* names[] = {"q_nope", "q_rope", "ckv_ctx", "kr_ctx", "ckv_blk", "kr_blk",
                           "w_uk", "w_uv", "anchors", "keep", "out"};
    for (int i = 0; i < 11; ++i) {
        const bool may_be_null = (i == 1 || i == 3 || i == 5) && d.d_rope == 0;
        if (!ptrs[i] && !may_be_null) return fail(DSPARK_EINVAL, "%s is NULL", names[i]);
        if (ptrs[i] && i != 9 && !aligned16(ptrs[i]))
            return fail(DSPARK_EINVAL, "%s must be 16-byte aligned", names[i]);
    }
    const FwdPath path = pick_path(d, opts, true);
    const bool fast = path != FwdPath::kGeneric;
    // reuse_forward on a forward: the workspace is a backward's, and the MFMA
    // path also leaves its probabilities there for that backward
    const bool for_bwd = !fixed && opts && opts->reuse_forward;
    if (for_bwd && path == FwdPath::kFused)
        return fail(DSPARK_EINVAL,
                    "reuse_forward needs the three-kernel forward (the one-launch forward leaves "
                    "no latents)");
    const bool keep_p = for_bwd && path == FwdPath::kMaterialised;
    int round_blocks = 0;
    const WsLayout L = fixed ? fixed_layout(d, fast, &round_blocks) : path_layout(d, path);
    if (fixed) {
        if (L.total > kFixedScratchBytes)
            return fail(DSPARK_EUNSUPPORTED,
                        "this shape needs %zu bytes of scratch; the fixed scratch array holds %zu",
                        L.total, kFixedScratchBytes);
        workspace = fixed->base;
        ws_bytes = kFixedScratchBytes;
    }
    st = check_workspace(workspace, ws_bytes, keep_p ? bwd_layout(d, true).total : L.total);
    if (st != DSPARK_OK) return st;
    bf16* pmat = keep_p
                     ? reinterpret_cast<bf16*>(static_cast<char*>(workspace) + bwd_layout(d, true).pmat)
                     : nullptr;

    const Problem p = make_problem(d);
    if (!fast) {
        if (generic_lds_bytes(p) > 64 * 1024)
            return fail(DSPARK_EUNSUPPORTED,
                        "shape needs %zu bytes of LDS in the generic kernel (max 65536)",
                        generic_lds_bytes(p));
    }
    Workspace ws = carve(workspace, L);
    if (fixed && fixed->status) ws.status = fixed->status;
    const Inputs in{q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv, out};
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* const* ev = (opts && opts->stage_events) ? opts->stage_events : nullptr;
    auto mark = [&](int k) -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k]), s) : hipSuccess;
    };

    const bool fused = path == FwdPath::kFused;
    const int chunk = fixed ? round_blocks : chunk_blocks(d, opts);
    const int n_chunks = (fast && !fused) ? (d.B * d.N + chunk - 1) / chunk : 0;
    const int n_events = (fast && !fused) ? 2 + 4 * n_chunks : 3;
    if (ev && opts->n_stage_events < n_events)
        return fail(DSPARK_EINVAL, "this call records %d stage events; n_stage_events is %d",
                    n_events, opts->n_stage_events);
    hipStream_t aux = (opts && fast && n_chunks > 1) ? static_cast<hipStream_t>(opts->aux_stream)
                                                     : nullptr;
    if (aux) {
        if (aux == s) return fail(DSPARK_EINVAL, "aux_stream must differ from stream");
        if (!opts->aux_events[0] || !opts->aux_events[1])
            return fail(DSPARK_EINVAL, "aux_stream needs two events in aux_events");
    }
    auto mark_on = [&](int k, hipStream_t st) -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k]), st) : hipSuccess;
    };

    hipError_t e;
    if ((e = mark(0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    const RopeTheta theta = make_theta(d);
    if (fused) {
        // index, padding rows and the pipeline's control words, then the
        // whole forward in one launch
        if ((e = launch_prep(p, anchors, keep, ws, nullptr, 0, nullptr, out, s,
                             forward_tag(d, path))) != hipSuccess)
            return hip_fail(e, "index / fill launch");
        if ((e = mark(1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        if ((e = launch_fused(p, in, ws, theta, s)) != hipSuccess)
            return hip_fail(e, "fused forward launch");
        if ((e = mark(2)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        return ok();
    }
    // the MFMA path evaluates RoPE inside the attention kernel; only the
    // generic path reads the table
    // the fixed scratch is never handed to a backward: no tag
    // the MFMA path writes the rows of padding blocks in the last W_UV
    // launch's tail instead of here
    const int32_t tag = fixed ? 0 : forward_tag(d, path, keep_p);
    // one round of at most kSelfIndexMax blocks: the absorb launch builds the
    // index itself and no preparation launch runs (stage event [1] then
    // follows [0] directly)
    const bool self_index = fast && n_chunks == 1 && d.B * d.N <= kSelfIndexMax;
    if (!self_index) {
        if ((e = launch_prep(p, anchors, keep, ws, nullptr, L.rope_rows,
                             fast ? nullptr : &theta, nullptr, s, tag)) != hipSuccess)
            return hip_fail(e, "index / RoPE table / fill launch");
    }
    if ((e = mark(1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if (fast) {
        hipEvent_t fork = aux ? static_cast<hipEvent_t>(opts->aux_events[0]) : nullptr;
        hipEvent_t join = aux ? static_cast<hipEvent_t>(opts->aux_events[1]) : nullptr;
        if (aux) {
            if ((e = hipEventRecord(fork, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            if ((e = hipStreamWaitEvent(aux, fork, 0)) != hipSuccess)
                return hip_fail(e, "hipStreamWaitEvent");
        }
        for (int c = 0; c < n_chunks; ++c) {
            // rounds write disjoint latent rows (row = 5 * slot + query), so
            // rounds on different streams do not interfere
            hipStream_t st = (aux && (c & 1)) ? aux : s;
            const Chunk ch{c * chunk, chunk};
            if ((e = mark_on(2 + 4 * c, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            const Workspace wr = fixed ? round_latents(ws, p, ch.slot0) : ws;
            if ((e = launch_absorb(p, in, wr, ch, st, self_index ? anchors : nullptr,
                                   self_index ? keep : nullptr, tag)) != hipSuccess)
                return hip_fail(e, "absorb launch");
            if ((e = mark_on(3 + 4 * c, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            if ((e = launch_attn(p, in, wr, ch, theta, st, pmat)) != hipSuccess)
                return hip_fail(e, "attention launch");
            if ((e = mark_on(4 + 4 * c, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            const bool last = c == n_chunks - 1;
            if ((e = launch_uv(p, in, wr, ch, st, last ? anchors : nullptr,
                               last ? keep : nullptr)) != hipSuccess)
                return hip_fail(e, "W_UV launch");
            if ((e = mark_on(5 + 4 * c, st)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        }
        if (aux) {
            if ((e = hipEventRecord(join, aux)) != hipSuccess) return hip_fail(e, "hipEventRecord");
            if ((e = hipStreamWaitEvent(s, join, 0)) != hipSuccess)
                return hip_fail(e, "hipStreamWaitEvent");
        }
    } else {
        if ((e = launch_generic(p, d.dtype == DSPARK_BF16, in, ws, s)) != hipSuccess)
            return hip_fail(e, "generic kernel launch");
        if ((e = mark(2)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    return ok();
}

}  // namespace

void set_last_error(const char* msg) { g_last_error = msg; }

}  // namespace dspark

using namespace dspark;

extern "C" {

int32_t dspark_abi_version(void) { return DSPARK_ABI_VERSION; }

const char* dspark_last_error(void) { return g_last_error.c_str(); }

size_t dspark_attn_workspace_size(const dspark_attn_desc* desc) {
    bool empty = false;
    if (check_desc(desc, &empty) != DSPARK_OK) return 0;
    g_last_error.clear();
    const size_t any = ws_layout(*desc, is_fast_path(*desc)).total;
    const size_t fused = is_fast_path(*desc) ? ws_layout(*desc, false, true).total : 0;
    return any > fused ? any : fused;
}

size_t dspark_attn_workspace_size_ex(const dspark_attn_desc* desc, const dspark_attn_opts* opts) {
    bool empty = false;
    if (check_desc(desc, &empty) != DSPARK_OK) return 0;
    g_last_error.clear();
    const FwdPath path = pick_path(*desc, opts, false);
    // reuse_forward: a backward's workspace (the MFMA path writes into it)
    if (opts && opts->reuse_forward && path == FwdPath::kMaterialised)
        return bwd_layout(*desc, true).total;
    return path_layout(*desc, path).total;
}

dspark_status dspark_attn_fwd_ex(const dspark_attn_desc* desc, const void* q_nope,
                                 const void* q_rope, const void* ckv_ctx, const void* kr_ctx,
                                 const void* ckv_blk, const void* kr_blk, const void* w_uk,
                                 const void* w_uv, const int32_t* anchors, const uint8_t* keep,
                                 void* out, void* workspace, size_t ws_bytes, void* stream,
                                 const dspark_attn_opts* opts) {
    return forward_impl(desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                        anchors, keep, out, workspace, ws_bytes, stream, opts, nullptr);
}

dspark_status dspark_attn_fwd_noalloc(const dspark_attn_desc* desc, const void* q_nope,
                                      const void* q_rope, const void* ckv_ctx,
                                      const void* kr_ctx, const void* ckv_blk,
                                      const void* kr_blk, const void* w_uk, const void* w_uv,
                                      const int32_t* anchors, const uint8_t* keep, void* out,
                                      int32_t* status, void* stream) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    if (empty) return ok();
    if (status && (reinterpret_cast<uintptr_t>(status) & 3u) != 0)
        return fail(DSPARK_EINVAL, "status must be 4-byte aligned");
    // the size check needs no device: reject what does not fit first
    int round_blocks = 0;
    const WsLayout L = fixed_layout(*desc, is_fast_path(*desc), &round_blocks);
    if (L.total > kFixedScratchBytes)
        return fail(DSPARK_EUNSUPPORTED,
                    "this shape needs %zu bytes of scratch; the fixed scratch array holds %zu",
                    L.total, kFixedScratchBytes);
    FixedScratch fx{nullptr, status};
    st = scratch_address(&fx.base);
    if (st != DSPARK_OK) return st;
    return forward_impl(desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                        anchors, keep, out, nullptr, 0, stream, nullptr, &fx);
}

dspark_status dspark_attn_plan(const dspark_attn_desc* desc, const dspark_attn_opts* opts,
                               int32_t* n_chunks, int32_t* chunk_out, int32_t* n_events) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    // the one-launch forward counts as one round over every block
    const FwdPath path = empty ? FwdPath::kGeneric : pick_path(*desc, opts, true);
    const bool fast = path == FwdPath::kMaterialised;
    const bool fused = path == FwdPath::kFused;
    const int chunk = empty ? 0 : chunk_blocks(*desc, opts);
    const int nc = fast ? (desc->B * desc->N + chunk - 1) / chunk : (fused ? 1 : 0);
    if (n_chunks) *n_chunks = nc;
    if (chunk_out) *chunk_out = fast ? chunk : (fused ? desc->B * desc->N : 0);
    if (n_events) *n_events = empty ? 0 : (fast ? 2 + 4 * nc : 3);
    return ok();
}

dspark_status dspark_attn_fwd(const dspark_attn_desc* desc, const void* q_nope,
                              const void* q_rope, const void* ckv_ctx, const void* kr_ctx,
                              const void* ckv_blk, const void* kr_blk, const void* w_uk,
                              const void* w_uv, const int32_t* anchors, const uint8_t* keep,
                              void* out, void* workspace, size_t ws_bytes, void* stream) {
    return dspark_attn_fwd_ex(desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                              anchors, keep, out, workspace, ws_bytes, stream, nullptr);
}

dspark_status dspark_build_index(const dspark_attn_desc* desc, const int32_t* anchors,
                                 const uint8_t* keep, int32_t* index_out, void* workspace,
                                 size_t ws_bytes, void* stream) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    if (empty) return ok();
    if (!anchors || !keep || !index_out)
        return fail(DSPARK_EINVAL, "anchors, keep and index_out must be non-NULL");
    if (!aligned16(anchors) || !aligned16(index_out))
        return fail(DSPARK_EINVAL, "anchors and index_out must be 16-byte aligned");
    const WsLayout L = ws_layout(*desc, is_fast_path(*desc));
    // the index build touches only the status, index, kept-list and slot
    // record areas
    st = check_workspace(workspace, ws_bytes, L.rope);
    if (st != DSPARK_OK) return st;
    const Problem p = make_problem(*desc);
    const Workspace ws = carve(workspace, L);
    hipError_t e = launch_prep(p, anchors, keep, ws, index_out, 0, nullptr, nullptr,
                               static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "index kernel launch");
    return ok();
}

size_t dspark_attn_bwd_workspace_size(const dspark_attn_desc* desc) {
    bool empty = false;
    if (check_desc(desc, &empty) != DSPARK_OK) return 0;
    g_last_error.clear();
    // enough for either path, so that opts->force_generic needs no other size
    const size_t generic = bwd_layout(*desc, false).total;
    const size_t fast = is_fast_path(*desc) ? bwd_layout(*desc, true).total : 0;
    return generic > fast ? generic : fast;
}

dspark_status dspark_attn_bwd_plan(const dspark_attn_desc* desc, const dspark_attn_opts* opts,
                                   int32_t* n_events) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    const bool fast = is_fast_path(*desc) && !(opts && opts->force_generic);
    if (n_events) *n_events = empty ? 0 : 1 + (fast ? kBwdLaunchesFast : kBwdLaunchesGeneric);
    return ok();
}

dspark_status dspark_attn_bwd_ex(const dspark_attn_desc* desc, const void* q_nope,
                                 const void* q_rope, const void* ckv_ctx, const void* kr_ctx,
                                 const void* ckv_blk, const void* kr_blk, const void* w_uk,
                                 const void* w_uv, const int32_t* anchors, const uint8_t* keep,
                                 const void* dout, void* dq_nope, void* dq_rope, void* dckv_ctx,
                                 void* dkr_ctx, void* dckv_blk, void* dkr_blk, void* dw_uk,
                                 void* dw_uv, void* workspace, size_t ws_bytes, void* stream,
                                 const dspark_attn_opts* opts) {
    bool empty = false;
    dspark_status st = check_desc(desc, &empty);
    if (st != DSPARK_OK) return st;
    if (empty) return ok();
    const dspark_attn_desc& d = *desc;
    const void* ptrs[] = {q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                          anchors, keep, dout, dq_nope, dq_rope, dckv_ctx, dkr_ctx,
                          dckv_blk, dkr_blk, dw_uk, dw_uv};
    const char* names[] = {"q_nope", "q_rope", "ckv_ctx", "kr_ctx", "ckv_blk", "kr_blk",
                           "w_uk", "w_uv", "anchors", "keep", "dout", "dq_nope", "dq_rope",
                           "dckv_ctx", "dkr_ctx", "dckv_blk", "dkr_blk", "dw_uk", "dw_uv"};
    for (int i = 0; i < 19; ++i) {
        const bool rope_arg = i == 1 || i == 3 || i == 5 || i == 12 || i == 14 || i == 16;
        const bool may_be_null = rope_arg && d.d_rope == 0;
        if (!ptrs[i] && !may_be_null) return fail(DSPARK_EINVAL, "%s is NULL", names[i]);
        if (ptrs[i] && i != 9 && !aligned16(ptrs[i]))
            return fail(DSPARK_EINVAL, "%s must be 16-byte aligned", names[i]);
    }
    const bool fast = is_fast_path(d) && !(opts && opts->force_generic);
    const BwdLayout L = bwd_layout(d, fast);
    st = check_workspace(workspace, ws_bytes, L.total);
    if (st != DSPARK_OK) return st;
    const Problem p = make_problem(d);
    if (!fast && bwd_generic_lds_bytes(p) > 64 * 1024)
        return fail(DSPARK_EUNSUPPORTED,
                    "shape needs %zu bytes of LDS in the generic backward kernel (max 65536)",
                    bwd_generic_lds_bytes(p));
    const int n_events = 1 + (fast ? kBwdLaunchesFast : kBwdLaunchesGeneric);
    void* const* ev = (opts && opts->stage_events) ? opts->stage_events : nullptr;
    if (ev && opts->n_stage_events < n_events)
        return fail(DSPARK_EINVAL, "this call records %d stage events; n_stage_events is %d",
                    n_events, opts->n_stage_events);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int k_ev = 0;
    auto mark = [&]() -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k_ev++]), s) : hipSuccess;
    };
    const BwdWork w = carve_bwd(workspace, L);
    const Inputs in{q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv, nullptr};
    const BwdGrads g{dout, dq_nope, dq_rope, dckv_ctx, dkr_ctx, dckv_blk, dkr_blk, dw_uk, dw_uv};
    const RopeTheta theta = make_theta(d);
    hipError_t e;
#define DSPARK_STEP(call, what)                                   \
    do {                                                          \
        if ((e = (call)) != hipSuccess) return hip_fail(e, what); \
        if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord"); \
    } while (0)
    if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    size_t zero_n = L.acc_rows * size_t(d.d_latent + d.d_rope);
    if (!fast) zero_n = (L.total - L.acc) / 4;     // accumulators, then the weight ones
    // reuse_forward: the forward on this workspace left the index (and, on the
    // MFMA path, q_abs) in the same places; those launches are skipped (their
    // stage events are still recorded)
    // reuse_forward is checked on the device: a workspace whose last index
    // build was not for this descriptor and path gets an all-padding index
    // here and NaN gradients at the end (dspark_read_device_status reports
    // it); the backward's own index build leaves the same tag, since its
    // launches also leave the index and the latents a forward would
    // reuse_forward 2 on the MFMA path: the forward also left P (its tag
    // says so) and the attention backward reads it instead of recomputing
    // the scores; 1 accepts a forward with or without P
    const bool reuse = opts && opts->reuse_forward;
    const bool load_p = reuse && fast && opts->reuse_forward == 2;
    const int32_t tag = forward_tag(d, fast ? FwdPath::kMaterialised : FwdPath::kGeneric);
    const int32_t tag_p = forward_tag(d, FwdPath::kMaterialised, true);
    // at most kSelfIndexMax blocks on the MFMA path: the q_abs launch builds
    // the index itself (the index stage event follows event [0] directly)
    const bool self_index = fast && !reuse && d.B * d.N <= kSelfIndexMax;
    if (reuse) {
        DSPARK_STEP(launch_bwd_reuse_check(p, w, load_p ? tag_p : tag,
                                           (fast && !load_p) ? tag_p : 0, s),
                    "reuse check launch");
    } else if (self_index) {
        if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    } else {
        DSPARK_STEP(launch_prep(p, anchors, keep, w.fwd, nullptr, L.fwd.rope_rows,
                                fast ? nullptr : &theta, nullptr, s, tag),
                    "index launch");
    }
    // the MFMA path's anchor-order check is part of the index build, and the
    // accumulator clear (needed only when the anchors do not ascend) part of
    // the W_UV^T dout launch; their stage events are still recorded
    if (fast) {
        if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
        if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
    } else {
        DSPARK_STEP(launch_bwd_zero(w.acc, zero_n, nullptr, s), "accumulator clear launch");
    }
    if (fast) {
        if (reuse) {
            if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
        } else {
            DSPARK_STEP(launch_absorb(p, in, w.fwd, Chunk{0, d.B * d.N}, s,
                                      self_index ? anchors : nullptr,
                                      self_index ? keep : nullptr, tag),
                        "absorb launch");
        }
        DSPARK_STEP(launch_absorb_dv(p, dout, w_uv, w.fwd, w.dolat, w.acc, zero_n, s),
                    "W_UV^T dout launch");
        DSPARK_STEP(launch_bwd_attn(p, in, g, w, theta, s, !reuse, load_p),
                    "backward attention launch");
        DSPARK_STEP(launch_bwd_dkv(p, w, s), "dc^KV launch");
        DSPARK_STEP(launch_uv_dqc(p, in.w_uk, w.dqabs, w.fwd, g.dq_nope, s), "dq^C launch");
        DSPARK_STEP(launch_bwd_dw(p, in, g, w, s), "weight-gradient launch");
    } else {
        DSPARK_STEP(launch_bwd_generic(p, d.dtype == DSPARK_BF16, in, g, w, s),
                    "generic backward launch");
    }
    e = fast ? launch_bwd_gather(p, g, w, theta, s)
             : launch_bwd_finalize(p, d.dtype == DSPARK_BF16, g, w, w.fwd.idx, w.fwd.rope, theta,
                                   true, s);
    if (e != hipSuccess) return hip_fail(e, "final backward launch");
    if (reuse) {
        const int elem = (fast || d.dtype == DSPARK_BF16) ? 2 : 4;
        if ((e = launch_bwd_reuse_fill(p, g, w, elem, s)) != hipSuccess)
            return hip_fail(e, "reuse fill launch");
    }
    if ((e = mark()) != hipSuccess) return hip_fail(e, "hipEventRecord");
#undef DSPARK_STEP
    return ok();
}

dspark_status dspark_attn_bwd(const dspark_attn_desc* desc, const void* q_nope,
                              const void* q_rope, const void* ckv_ctx, const void* kr_ctx,
                              const void* ckv_blk, const void* kr_blk, const void* w_uk,
                              const void* w_uv, const int32_t* anchors, const uint8_t* keep,
                              const void* dout, void* dq_nope, void* dq_rope, void* dckv_ctx,
                              void* dkr_ctx, void* dckv_blk, void* dkr_blk, void* dw_uk,
                              void* dw_uv, void* workspace, size_t ws_bytes, void* stream) {
    return dspark_attn_bwd_ex(desc, q_nope, q_rope, ckv_ctx, kr_ctx, ckv_blk, kr_blk, w_uk, w_uv,
                              anchors, keep, dout, dq_nope, dq_rope, dckv_ctx, dkr_ctx, dckv_blk,
                              dkr_blk, dw_uk, dw_uv, workspace, ws_bytes, stream, nullptr);
}

dspark_status dspark_read_device_status(const void* workspace, void* stream,
                                        int32_t* first_bad_block) {
    if (first_bad_block) *first_bad_block = -1;
    if (!workspace) return fail(DSPARK_EWORKSPACE, "workspace is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int32_t words[kStWords];
    e = hipMemcpy(words, workspace, sizeof(words), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy of the status area");
    if (first_bad_block) *first_bad_block = words[kStFirstBad];
    if (words[kStFirstBad] >= 0)
        return fail(DSPARK_EANCHOR, "kept block %d has an anchor outside [0, S-2]",
                    words[kStFirstBad]);
    if (words[kStReuseBad] != 0)
        return fail(DSPARK_EINVAL,
                    "reuse_forward: the workspace's last index build was not a forward of this "
                    "descriptor on the path this backward takes; the gradients are NaN");
    if (words[kStPipeFault] != 0)
        return fail(DSPARK_EHIP,
                    "the one-launch forward stalled (a unit waited past its time bound); "
                    "its output is incomplete");
    return ok();
}

}  // extern "C"
