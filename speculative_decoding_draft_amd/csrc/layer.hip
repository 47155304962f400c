// The MLA block of one DSpark draft layer around the attention (GLM 5.2
// DSpark training-design page, §4 "MLA Projection"):
//   h    = RMSNorm(H)                          input_layernorm
//   c^Q  = RMSNorm(h W_qa^T)                   q_a_proj, q_a_layernorm
//   q    = c^Q W_qb^T -> per head (q^C, q^R)   q_b_proj
//   [c^KV ; k^R] = [H^ctx ; h] W_kva^T         kv_a_proj_with_mqa
//   c^KV <- RMSNorm(c^KV)                      kv_a_layernorm
//   o    = the masked attention (attn.hip ...) with W_UK / W_UV (kv_b_proj)
//   out  = H + o W_o^T                         o_proj into the residual
// The projections are plain GEMMs and run on rocBLAS (bf16 or fp32 operands,
// fp32 accumulation); the RMSNorms and the c^KV / k^R split are kernels
// here; q^R and k^R go to the attention unrotated (it rotates them while
// loading).  RMSNorm is x / sqrt(mean(x^2) + eps) * g; the page names the
// op without a formula or epsilon, so eps is a descriptor field.
#include <cstdio>
#include <cstring>

#include "blas.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

template <typename T> __device__ inline float ldf(const T* p, size_t i);
template <> __device__ inline float ldf<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ inline float ldf<bf16>(const bf16* p, size_t i) { return (float)p[i]; }
template <typename T> __device__ inline void stf(T* p, size_t i, float v);
template <> __device__ inline void stf<float>(float* p, size_t i, float v) { p[i] = v; }
template <> __device__ inline void stf<bf16>(bf16* p, size_t i, float v) { p[i] = (bf16)v; }

constexpr int kNormThreads = 256;

// Row r of a compacted operand (5 rows per kept-block slot) is row
// 5 * slot_blk[r / 5] + r % 5 of the [B * 5N] layout; -1 when the slot is
// empty.  slot_blk = nullptr: the identity.
__device__ inline long long full_row(const int32_t* __restrict__ slot_blk, long long r) {
    if (!slot_blk) return r;
    const int blk = slot_blk[r / kBlock];
    return blk < 0 ? -1 : (long long)blk * kBlock + r % kBlock;
}

// Sum over the workgroup (kNormThreads) of v.
__device__ inline float block_sum(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();                          // red is reused across rows
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kNormThreads / 64; ++i) s += red[i];
    return s;
}

// y[r, :n] = RMSNorm(x[r, :n]) * g for every row; when tail_out is given,
// x[r, n : n + n_tail] is copied to tail_out[r, :n_tail] (the k^R split).
// in_map / out_map (slot lists or nullptr): x's or y's (and tail_out's) row
// for row r is full_row(map, r); an empty input slot gives a zero row, an
// empty output slot is skipped.  One workgroup per row (grid-stride).
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const T* __restrict__ x, size_t ldx, const T* __restrict__ g, T* __restrict__ y, size_t ldy,
    T* __restrict__ tail_out, int n_tail, size_t rows, int n, float eps,
    const int32_t* __restrict__ in_map, const int32_t* __restrict__ out_map) {
    __shared__ float red[kNormThreads / 64];
    for (size_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const long long ri = full_row(in_map, (long long)r), ro = full_row(out_map, (long long)r);
        if (ro < 0) continue;
        T* yr = y + (size_t)ro * ldy;
        if (ri < 0) {
            for (int i = threadIdx.x; i < n; i += kNormThreads) stf(yr, i, 0.f);
            if (tail_out)
                for (int i = threadIdx.x; i < n_tail; i += kNormThreads)
                    stf(tail_out + (size_t)ro * n_tail, i, 0.f);
            continue;
        }
        const T* xr = x + (size_t)ri * ldx;
        float ss = 0.f;
        for (int i = threadIdx.x; i < n; i += kNormThreads) {
            const float v = ldf(xr, i);
            ss += v * v;
        }
        const float inv = rsqrtf(block_sum(ss, red) / (float)n + eps);
        for (int i = threadIdx.x; i < n; i += kNormThreads)
            stf(yr, i, ldf(xr, i) * inv * ldf(g, i));
        if (tail_out)
            for (int i = threadIdx.x; i < n_tail; i += kNormThreads)
                stf(tail_out + (size_t)ro * n_tail, i, ldf(xr, n + i));
    }
}

// bf16 rows with n % 512 == 0 (n <= 512 * kMaxChunks) and 16-byte aligned
// rows: one wave per row, the row held in registers (n / 512 chunks of 8
// per lane), reductions by shuffles only.
constexpr int kMaxChunks = 16;
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_wave_kernel(
    const bf16* __restrict__ x, size_t ldx, const bf16* __restrict__ g, bf16* __restrict__ y,
    size_t ldy, bf16* __restrict__ tail_out, int n_tail, size_t rows, float eps,
    const int32_t* __restrict__ in_map, const int32_t* __restrict__ out_map) {
    const int lane = threadIdx.x & 63;
    constexpr int n = 512 * CH;
    for (size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows;
         r += (size_t)gridDim.x * 4) {
        const long long ri = full_row(in_map, (long long)r), ro = full_row(out_map, (long long)r);
        if (ro < 0) continue;
        bf16* yr = y + (size_t)ro * ldy;
        if (ri < 0) {
            bf16x8 z;
#pragma unroll
            for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
#pragma unroll
            for (int c = 0; c < CH; ++c) gst16(yr + 8 * (lane + 64 * c), z);
            if (tail_out)
                for (int i = lane; i < n_tail; i += 64) tail_out[(size_t)ro * n_tail + i] = (bf16)0.f;
            continue;
        }
        const bf16* xr = x + (size_t)ri * ldx;
        bf16x8 v[CH];
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            v[c] = gld16(xr + 8 * (lane + 64 * c));
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (float)v[c][i] * (float)v[c][i];
        }
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const float inv = rsqrtf(ss / (float)n + eps);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bf16x8 gw = gld16(g + 8 * (lane + 64 * c));
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[c][i] * inv * (float)gw[i]);
            gst16(yr + 8 * (lane + 64 * c), o);
        }
        if (tail_out)
            for (int i = lane; i < n_tail; i += 64) tail_out[(size_t)ro * n_tail + i] = xr[n + i];
    }
}

template <typename T>
hipError_t launch_rmsnorm(const T* x, size_t ldx, const T* g, T* y, size_t ldy, T* tail,
                          int n_tail, size_t rows, int n, float eps, hipStream_t s,
                          const int32_t* in_map = nullptr, const int32_t* out_map = nullptr) {
    if (rows == 0) return hipSuccess;
    const auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    if constexpr (sizeof(T) == 2) {
        const int ch = n / 512;
        if (n % 512 == 0 && ch >= 1 && ch <= kMaxChunks && ldx % 8 == 0 && ldy % 8 == 0 &&
            al(x) && al(y) && al(g)) {
            const size_t want = (rows + 3) / 4;
            const int grid = (int)(want < 16384 ? want : 16384);
#define DSPARK_NORM_CASE(C)                                                                   \
    case C:                                                                                   \
        hipLaunchKernelGGL(rmsnorm_wave_kernel<C>, dim3(grid), dim3(256), 0, s, x, ldx, g, y, \
                           ldy, tail, n_tail, rows, eps, in_map, out_map);                    \
        return hipGetLastError();
            switch (ch) {
                DSPARK_NORM_CASE(1) DSPARK_NORM_CASE(2) DSPARK_NORM_CASE(3) DSPARK_NORM_CASE(4)
                DSPARK_NORM_CASE(6) DSPARK_NORM_CASE(8) DSPARK_NORM_CASE(12) DSPARK_NORM_CASE(16)
                default: break;
            }
#undef DSPARK_NORM_CASE
        }
    }
    const int grid = (int)(rows < 8192 ? rows : 8192);
    hipLaunchKernelGGL(rmsnorm_kernel<T>, dim3(grid), dim3(kNormThreads), 0, s, x, ldx, g, y, ldy,
                       tail, n_tail, rows, n, eps, in_map, out_map);
    return hipGetLastError();
}

// [rows][H][dc + dr] -> [rows][H][dc] and [rows][H][dr], in 16-byte pieces
// when dc and dr allow (vec elements of 16 bytes), element by element
// otherwise (vec = 1).  Output row of row r: full_row(out_map, r) (empty
// slots are skipped).
template <typename T>
__global__ __launch_bounds__(256) void split_heads_kernel(const T* __restrict__ q, T* __restrict__ qn,
                                                          T* __restrict__ qr, size_t rows, int H,
                                                          int dc, int dr, int vec,
                                                          const int32_t* __restrict__ out_map) {
    const int w = dc + dr;
    const size_t per_row = (size_t)H * w / vec;
    const size_t total = rows * per_row;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (size_t)gridDim.x * blockDim.x) {
        const size_t r = e / per_row;
        const long long ro = full_row(out_map, (long long)r);
        if (ro < 0) continue;
        const int k = (int)(e % per_row) * vec, h = k / w, j = k % w;
        const T* src = q + r * (size_t)H * w + k;
        T* dst = (j < dc) ? qn + ((size_t)ro * H + h) * (size_t)dc + j
                          : qr + ((size_t)ro * H + h) * (size_t)dr + (j - dc);
        if (vec * sizeof(T) == 16) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
            *dst = *src;
        }
    }
}

// Kept-block slots of the block: blocks in (b, n) order, keep != 0 gets the
// next slot.  slot_blk [cap] (-1 past the last), blk_slot [B*N] (-1 for
// padding), status words: kept count, first kept block with an anchor
// outside [0, S-2] (-1 when none), overflow (kept > cap).  One workgroup.
constexpr int kLayerIndexThreads = 1024;
enum LayerStatus { kLyKept = 0, kLyFirstBad = 1, kLyOverflow = 2, kLyWords = 16 };
__global__ __launch_bounds__(kLayerIndexThreads) void layer_index_kernel(
    int total, int S, int cap, const int32_t* __restrict__ anchors, const uint8_t* __restrict__ keep,
    int32_t* __restrict__ status, int32_t* __restrict__ slot_blk, int32_t* __restrict__ blk_slot) {
    __shared__ int wsum[kLayerIndexThreads / 64];
    __shared__ int base_s, bad_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) {
        base_s = 0;
        bad_s = 0x7fffffff;
    }
    __syncthreads();
    for (int c0 = 0; c0 < total; c0 += kLayerIndexThreads) {
        const int i = c0 + tid;
        int kp = 0;
        if (i < total) {
            kp = keep[i] != 0 ? 1 : 0;
            const int A = anchors[i];
            if (kp && (A < 0 || A > S - 2)) atomicMin(&bad_s, i);
        }
        int incl = kp;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int before = base_s, all = 0;
        for (int j = 0; j < kLayerIndexThreads / 64; ++j) {
            if (j < w) before += wsum[j];
            all += wsum[j];
        }
        const int slot = before + incl - kp;
        if (i < total) {
            blk_slot[i] = (kp && slot < cap) ? slot : -1;
            if (kp && slot < cap) slot_blk[slot] = i;
        }
        __syncthreads();
        if (tid == 0) base_s += all;
        __syncthreads();
    }
    const int kept = base_s;
    for (int j = kept + tid; j < cap; j += kLayerIndexThreads) slot_blk[j] = -1;
    if (tid == 0) {
        status[kLyKept] = kept;
        status[kLyFirstBad] = bad_s == 0x7fffffff ? -1 : bad_s;
        status[kLyOverflow] = kept > cap ? 1 : 0;
    }
}

// dst[r] = src[full_row(slot_blk, r)] (zero rows for empty slots): the
// attention output rows of the kept blocks, compacted for o_proj.  One wave
// per row, n elements of 16 bytes / sizeof(T) each when VEC.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void gather_rows_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                          size_t rows, int n,
                                                          const int32_t* __restrict__ slot_blk) {
    const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const long long ri = full_row(slot_blk, (long long)r);
    T* d = dst + r * n;
    if (VEC) {
        constexpr int E = 16 / (int)sizeof(T);
        for (int i = lane; i < n / E; i += 64)
            reinterpret_cast<uint4*>(d)[i] =
                ri < 0 ? make_uint4(0, 0, 0, 0) : reinterpret_cast<const uint4*>(src + (size_t)ri * n)[i];
    } else {
        for (int i = lane; i < n; i += 64) d[i] = ri < 0 ? T(0) : src[(size_t)ri * n + i];
    }
}

// out[R] = proj[5 * slot + R % 5] (H + o W_o^T of the kept rows, already
// rounded once) for rows of blocks with a slot, H[R] for the others; NaN
// everywhere when the kept blocks overflowed the slots.  One wave per row of
// the [B * 5N] layout, 16-byte pieces when VEC.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void residual_scatter_kernel(
    const T* __restrict__ H, const T* __restrict__ proj, T* __restrict__ out, size_t rows, int n,
    const int32_t* __restrict__ blk_slot, const int32_t* __restrict__ status) {
    const size_t R = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (R >= rows) return;
    const bool overflow = status[kLyOverflow] != 0;
    const int slot = blk_slot[R / kBlock];
    T* o = out + R * n;
    if (overflow) {
        for (int i = lane; i < n; i += 64) o[i] = T(NAN);
        return;
    }
    const T* src = slot < 0 ? H + R * n : proj + ((size_t)slot * kBlock + R % kBlock) * n;
    if (VEC) {
        constexpr int E = 16 / (int)sizeof(T);
        for (int i = lane; i < n / E; i += 64)
            reinterpret_cast<uint4*>(o)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        for (int i = lane; i < n; i += 64) o[i] = src[i];
    }
}

}  // namespace

// Workspace of dspark_mla_layer_fwd: a status area (offset 0), the slot
// lists, the block's intermediates -- the draft-row ones compacted to 5 rows
// per kept-block slot, the ones the attention reads in its [B * 5N] layout
// -- then the attention's own workspace.
struct LayerLayout {
    size_t status = 0, slot_blk = 0, blk_slot = 0, hn = 0, cq = 0, qf = 0, qn = 0, qr = 0,
           kvc = 0, kvb = 0, ckv_c = 0, kr_c = 0, ckv_b = 0, kr_b = 0, o = 0, o_c = 0, h_c = 0,
           proj = 0, blas = 0, attn = 0, total = 0;
    int cap = 0;
};

int layer_cap(const dspark_layer_desc& L) {
    const long long bn = (long long)L.attn.B * L.attn.N;
    return (int)(L.max_kept_blocks > 0 ? std::min<long long>(L.max_kept_blocks, bn) : bn);
}

LayerLayout layer_layout(const dspark_layer_desc& L, size_t attn_ws) {
    const dspark_attn_desc& d = L.attn;
    const size_t e = d.dtype == DSPARK_BF16 ? 2 : 4;
    LayerLayout w;
    w.cap = layer_cap(L);
    const size_t q_rows = size_t(d.B) * kBlock * d.N, c_rows = size_t(d.B) * d.S;
    const size_t k_rows = size_t(kBlock) * w.cap;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    w.status = take(kLyWords * 4);
    w.slot_blk = take(size_t(w.cap) * 4);
    w.blk_slot = take(size_t(d.B) * d.N * 4);
    w.hn = take(k_rows * L.hidden * e);
    w.cq = take(k_rows * L.q_rank * e);
    w.qf = take(k_rows * d.n_heads * (d.d_nope + d.d_rope) * e);
    w.qn = take(q_rows * d.n_heads * d.d_nope * e);
    w.qr = take(q_rows * d.n_heads * d.d_rope * e + 16);
    w.kvc = take(c_rows * (d.d_latent + d.d_rope) * e);
    w.kvb = take(k_rows * (d.d_latent + d.d_rope) * e);
    w.ckv_c = take(c_rows * d.d_latent * e);
    w.kr_c = take(c_rows * d.d_rope * e + 16);
    w.ckv_b = take(q_rows * d.d_latent * e);
    w.kr_b = take(q_rows * d.d_rope * e + 16);
    w.o = take(q_rows * d.n_heads * d.d_v * e);
    w.o_c = take(k_rows * d.n_heads * d.d_v * e);
    w.h_c = take(k_rows * L.hidden * e);
    w.proj = take(k_rows * L.hidden * e);
    w.blas = take(DSPARK_BLAS_WORKSPACE_BYTES);
    w.attn = take(attn_ws);
    w.total = off;
    return w;
}

}  // namespace dspark

using namespace dspark;

namespace dspark {
void set_last_error(const char* msg);    // api.hip: the text dspark_last_error() returns
}

namespace {

thread_local char t_msg[512];   // formatting buffer for the error text

dspark_status lfail(dspark_status code, const char* msg, long long detail) {
    snprintf(t_msg, sizeof(t_msg), "%s (%lld)", msg, detail);
    set_last_error(t_msg);
    return code;
}

dspark_status lfail(dspark_status code, const char* msg) {
    set_last_error(msg);
    return code;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

size_t dspark_mla_layer_workspace_size(const dspark_layer_desc* desc) {
    if (!desc || desc->hidden < 1 || desc->q_rank < 1 || desc->max_kept_blocks < 0) return 0;
    const size_t a = dspark_attn_workspace_size(&desc->attn);
    if (a == 0) return 0;
    return layer_layout(*desc, a).total;
}

}  // extern "C"

namespace {

dspark_status layer_fwd(const dspark_layer_desc* desc, const void* h_draft, const void* h_ctx,
                        const void* g_in, const void* w_qa, const void* g_qa, const void* w_qb,
                        const void* w_kva, const void* g_kva, const void* w_uk, const void* w_uv,
                        const void* w_o, const int32_t* anchors, const uint8_t* keep, void* out,
                        void* workspace, size_t ws_bytes, void* stream,
                        const dspark_attn_opts* opts, dspark_gemm_choices* tuned) {
    set_last_error("");
    if (!desc) return lfail(DSPARK_EINVAL, "desc is NULL");
    if (desc->hidden < 1 || desc->q_rank < 1)
        return lfail(DSPARK_EINVAL, "hidden and q_rank must be >= 1");
    if (!(desc->rms_eps >= 0.0)) return lfail(DSPARK_EINVAL, "rms_eps must be >= 0");
    if (desc->max_kept_blocks < 0) return lfail(DSPARK_EINVAL, "max_kept_blocks must be >= 0");
    const dspark_attn_desc& d = desc->attn;
    const size_t attn_ws = dspark_attn_workspace_size(&d);
    if (attn_ws == 0) return DSPARK_EINVAL;     // dspark_last_error() says why
    if ((long long)d.B * d.N == 0) return DSPARK_OK;
    const void* ptrs[] = {h_draft, h_ctx, g_in, w_qa, g_qa, w_qb, w_kva, g_kva, w_uk, w_uv,
                          w_o, anchors, keep, out};
    const char* names[] = {"h_draft", "h_ctx", "g_in", "w_qa", "g_qa", "w_qb", "w_kva", "g_kva",
                           "w_uk", "w_uv", "w_o", "anchors", "keep", "out"};
    for (int i = 0; i < 14; ++i) {
        if (!ptrs[i]) {
            snprintf(t_msg, sizeof(t_msg), "%s is NULL", names[i]);
            return lfail(DSPARK_EINVAL, t_msg);
        }
        if (i != 12 && !al16(ptrs[i])) {
            snprintf(t_msg, sizeof(t_msg), "%s must be 16-byte aligned", names[i]);
            return lfail(DSPARK_EINVAL, t_msg);
        }
    }
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return lfail(DSPARK_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    const LayerLayout L = layer_layout(*desc, attn_ws);
    if (ws_bytes < L.total)
        return lfail(DSPARK_EWORKSPACE, "workspace too small; bytes needed", (long long)L.total);
    void* const* ev = (opts && opts->stage_events) ? opts->stage_events : nullptr;
    constexpr int kEvents = 7;
    if (ev && opts->n_stage_events < kEvents)
        return lfail(DSPARK_EINVAL, "this call records 7 stage events; n_stage_events is",
                     opts->n_stage_events);

    hipStream_t s = static_cast<hipStream_t>(stream);
    rocblas_handle h;
    rocblas_status bs = blas_handle(s, &h);
    if (bs != rocblas_status_success) return lfail(DSPARK_EHIP, "rocBLAS handle set-up failed", bs);
    bs = blas_use_workspace(h, static_cast<char*>(workspace) + L.blas, DSPARK_BLAS_WORKSPACE_BYTES);
    if (bs != rocblas_status_success) return lfail(DSPARK_EHIP, "rocblas_set_workspace failed", bs);
    if (tuned) *tuned = dspark_gemm_choices{};
    GemmPick pick{tuned ? tuned : const_cast<dspark_gemm_choices*>(opts ? opts->gemm_choices
                                                                          : nullptr),
                  tuned != nullptr, 0};

    const bool bf = d.dtype == DSPARK_BF16;
    const rocblas_datatype tio = bf ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    char* base = static_cast<char*>(workspace);
    int32_t* status = reinterpret_cast<int32_t*>(base + L.status);
    int32_t* slot_blk = reinterpret_cast<int32_t*>(base + L.slot_blk);
    int32_t* blk_slot = reinterpret_cast<int32_t*>(base + L.blk_slot);
    void *hn = base + L.hn, *cq = base + L.cq, *qn = base + L.qn, *qr = base + L.qr;
    void *kvc = base + L.kvc, *kvb = base + L.kvb, *ckv_c = base + L.ckv_c, *kr_c = base + L.kr_c;
    void *ckv_b = base + L.ckv_b, *kr_b = base + L.kr_b, *o = base + L.o, *aws = base + L.attn;
    void* o_c = base + L.o_c;
    void* h_c = base + L.h_c;
    void* proj = base + L.proj;
    const int hid = desc->hidden, qk = desc->q_rank, H = d.n_heads;
    const int D = d.d_latent, dc = d.d_nope, dr = d.d_rope, dv = d.d_v;
    const int q_rows = d.B * kBlock * d.N, c_rows = d.B * d.S;
    const int k_rows = kBlock * L.cap;            // compacted draft rows
    const float eps = (float)desc->rms_eps;
    int k_ev = 0;
    auto mark = [&]() -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k_ev++]), s) : hipSuccess;
    };
    hipError_t he;
    auto norm = [&](const void* x, size_t ldx, const void* g, void* y, size_t ldy, void* tail,
                    int n_tail, size_t rows, int n, const int32_t* in_map,
                    const int32_t* out_map) -> hipError_t {
        return bf ? launch_rmsnorm((const bf16*)x, ldx, (const bf16*)g, (bf16*)y, ldy,
                                   (bf16*)tail, n_tail, rows, n, eps, s, in_map, out_map)
                  : launch_rmsnorm((const float*)x, ldx, (const float*)g, (float*)y, ldy,
                                   (float*)tail, n_tail, rows, n, eps, s, in_map, out_map);
    };
    auto waves_grid = [](size_t rows) { return dim3((unsigned)((rows + 3) / 4)); };
#define LSTEP_HIP(call, what)                                                     \
    do {                                                                          \
        if ((he = (call)) != hipSuccess) {                                        \
            snprintf(t_msg, sizeof(t_msg), "%s: %s", what, hipGetErrorString(he)); \
            return lfail(DSPARK_EHIP, t_msg);                                     \
        }                                                                         \
    } while (0)
#define LSTEP_BLAS(call, what)                                                    \
    do {                                                                          \
        if ((bs = (call)) != rocblas_status_success) return lfail(DSPARK_EHIP, what, bs); \
    } while (0)
#define LMARK() LSTEP_HIP(mark(), "hipEventRecord")

    LMARK();
    // kept-block slots; h = RMSNorm(H) for the rows of kept blocks, compacted
    hipLaunchKernelGGL(layer_index_kernel, dim3(1), dim3(kLayerIndexThreads), 0, s, d.B * d.N, d.S,
                       L.cap, anchors, keep, status, slot_blk, blk_slot);
    LSTEP_HIP(hipGetLastError(), "index launch");
    LSTEP_HIP(norm(h_draft, hid, g_in, hn, hid, nullptr, 0, k_rows, hid, slot_blk, nullptr),
              "input RMSNorm launch");
    LMARK();
    // c^Q = RMSNorm(h W_qa^T)
    LSTEP_BLAS(gemm_nt(h, tio, tio, k_rows, qk, hid, hn, hid, w_qa, hid, 0.f, nullptr, 0, cq, qk,
                       &pick), "q_a_proj GEMM");
    LSTEP_HIP(norm(cq, qk, g_qa, cq, qk, nullptr, 0, k_rows, qk, nullptr, nullptr),
              "q_a RMSNorm launch");
    LMARK();
    // [q^C ; q^R] per head = c^Q W_qb^T (one GEMM: per-head strided-batched GEMMs
    // of 192 and 64 columns ran at half the rate), then split into the
    // attention's [row][head][dim] layouts at the blocks' own rows
    void* qf = base + L.qf;
    LSTEP_BLAS(gemm_nt(h, tio, tio, k_rows, H * (dc + dr), qk, cq, qk, w_qb, qk, 0.f, nullptr, 0, qf,
                       H * (dc + dr), &pick), "q_b_proj GEMM");
    {
        const int vec = (dc % 8 == 0 && dr % 8 == 0 && bf) ? 8 : ((dc % 4 == 0 && dr % 4 == 0 && !bf) ? 4 : 1);
        const size_t total = (size_t)k_rows * H * (dc + dr) / vec;
        const size_t want = (total + 255) / 256;
        const int grid = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
        if (bf)
            hipLaunchKernelGGL(split_heads_kernel<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)qf,
                               (bf16*)qn, (bf16*)qr, (size_t)k_rows, H, dc, dr, vec, slot_blk);
        else
            hipLaunchKernelGGL(split_heads_kernel<float>, dim3(grid), dim3(256), 0, s,
                               (const float*)qf, (float*)qn, (float*)qr, (size_t)k_rows, H, dc, dr,
                               vec, slot_blk);
        LSTEP_HIP(hipGetLastError(), "q split launch");
    }
    LMARK();
    // [c^KV ; k^R] = [H^ctx ; h] W_kva^T, then c^KV <- RMSNorm(c^KV) and the k^R
    // split (the draft rows written back to the blocks' own rows)
    LSTEP_BLAS(gemm_nt(h, tio, tio, c_rows, D + dr, hid, h_ctx, hid, w_kva, hid, 0.f, nullptr, 0, kvc,
                       D + dr, &pick), "kv_a_proj (context) GEMM");
    LSTEP_BLAS(gemm_nt(h, tio, tio, k_rows, D + dr, hid, hn, hid, w_kva, hid, 0.f, nullptr, 0, kvb,
                       D + dr, &pick), "kv_a_proj (draft) GEMM");
    LSTEP_HIP(norm(kvc, D + dr, g_kva, ckv_c, D, kr_c, dr, c_rows, D, nullptr, nullptr),
              "kv_a RMSNorm launch");
    LSTEP_HIP(norm(kvb, D + dr, g_kva, ckv_b, D, kr_b, dr, k_rows, D, nullptr, slot_blk),
              "kv_a RMSNorm launch");
    LMARK();
    // the attention
    dspark_attn_opts ao;
    std::memset(&ao, 0, sizeof(ao));
    if (opts) ao.force_generic = opts->force_generic;
    const dspark_status ast =
        dspark_attn_fwd_ex(&d, qn, dr > 0 ? qr : nullptr, ckv_c, dr > 0 ? kr_c : nullptr, ckv_b,
                           dr > 0 ? kr_b : nullptr, w_uk, w_uv, anchors, keep, o, aws, attn_ws, s,
                           &ao);
    if (ast != DSPARK_OK) return ast;            // dspark_last_error() says why
    LMARK();
    // out = H + o W_o^T: the kept rows' o and H compacted, one GEMM with the
    // residual as its C operand (one rounding), then scattered back (padding
    // rows copy H)
    {
        const int n = H * dv;
        const size_t e = bf ? 2 : 4;
        const bool vo = ((size_t)n * e) % 16 == 0, vh = ((size_t)hid * e) % 16 == 0;
#define LGATHER(T, VV, src, dst, cols)                                                        \
    hipLaunchKernelGGL((gather_rows_kernel<T, VV>), waves_grid(k_rows), dim3(256), 0, s,       \
                       (const T*)(src), (T*)(dst), (size_t)k_rows, cols, slot_blk)
        if (bf) {
            if (vo) LGATHER(bf16, true, o, o_c, n); else LGATHER(bf16, false, o, o_c, n);
            if (vh) LGATHER(bf16, true, h_draft, h_c, hid); else LGATHER(bf16, false, h_draft, h_c, hid);
        } else {
            if (vo) LGATHER(float, true, o, o_c, n); else LGATHER(float, false, o, o_c, n);
            if (vh) LGATHER(float, true, h_draft, h_c, hid); else LGATHER(float, false, h_draft, h_c, hid);
        }
#undef LGATHER
        LSTEP_HIP(hipGetLastError(), "o / H gather launch");
        LSTEP_BLAS(gemm_nt(h, tio, tio, k_rows, hid, n, o_c, n, w_o, n, 1.f, h_c, hid, proj, hid,
                           &pick), "o_proj GEMM");
#define LSCATTER(T, VV)                                                                       \
    hipLaunchKernelGGL((residual_scatter_kernel<T, VV>), waves_grid(q_rows), dim3(256), 0, s,  \
                       (const T*)h_draft, (const T*)proj, (T*)out, (size_t)q_rows, hid, blk_slot, \
                       status)
        if (bf) {
            if (vh) LSCATTER(bf16, true); else LSCATTER(bf16, false);
        } else {
            if (vh) LSCATTER(float, true); else LSCATTER(float, false);
        }
#undef LSCATTER
        LSTEP_HIP(hipGetLastError(), "residual scatter launch");
    }
    LMARK();
#undef LSTEP_HIP
#undef LSTEP_BLAS
#undef LMARK
    return DSPARK_OK;
}

}  // namespace

extern "C" {

dspark_status dspark_mla_layer_fwd_ex(const dspark_layer_desc* desc, const void* h_draft,
                                      const void* h_ctx, const void* g_in, const void* w_qa,
                                      const void* g_qa, const void* w_qb, const void* w_kva,
                                      const void* g_kva, const void* w_uk, const void* w_uv,
                                      const void* w_o, const int32_t* anchors,
                                      const uint8_t* keep, void* out, void* workspace,
                                      size_t ws_bytes, void* stream,
                                      const dspark_attn_opts* opts) {
    return layer_fwd(desc, h_draft, h_ctx, g_in, w_qa, g_qa, w_qb, w_kva, g_kva, w_uk, w_uv, w_o,
                     anchors, keep, out, workspace, ws_bytes, stream, opts, nullptr);
}

dspark_status dspark_mla_layer_tune(const dspark_layer_desc* desc, const void* h_draft,
                                    const void* h_ctx, const void* g_in, const void* w_qa,
                                    const void* g_qa, const void* w_qb, const void* w_kva,
                                    const void* g_kva, const void* w_uk, const void* w_uv,
                                    const void* w_o, const int32_t* anchors, const uint8_t* keep,
                                    void* out, void* workspace, size_t ws_bytes, void* stream,
                                    dspark_gemm_choices* choices) {
    if (!choices) return lfail(DSPARK_EINVAL, "choices is NULL");
    return layer_fwd(desc, h_draft, h_ctx, g_in, w_qa, g_qa, w_qb, w_kva, g_kva, w_uk, w_uv, w_o,
                     anchors, keep, out, workspace, ws_bytes, stream, nullptr, choices);
}

dspark_status dspark_mla_layer_fwd(const dspark_layer_desc* desc, const void* h_draft,
                                   const void* h_ctx, const void* g_in, const void* w_qa,
                                   const void* g_qa, const void* w_qb, const void* w_kva,
                                   const void* g_kva, const void* w_uk, const void* w_uv,
                                   const void* w_o, const int32_t* anchors, const uint8_t* keep,
                                   void* out, void* workspace, size_t ws_bytes, void* stream) {
    return dspark_mla_layer_fwd_ex(desc, h_draft, h_ctx, g_in, w_qa, g_qa, w_qb, w_kva, g_kva,
                                   w_uk, w_uv, w_o, anchors, keep, out, workspace, ws_bytes,
                                   stream, nullptr);
}

}  // extern "C"

extern "C" dspark_status dspark_mla_layer_read_status(const void* workspace, void* stream,
                                                      int32_t* first_bad_block,
                                                      int32_t* kept_blocks) {
    if (first_bad_block) *first_bad_block = -1;
    if (kept_blocks) *kept_blocks = 0;
    if (!workspace) return lfail(DSPARK_EWORKSPACE, "workspace is NULL");
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    int32_t w[kLyWords];
    if (e == hipSuccess) e = hipMemcpy(w, workspace, sizeof(w), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        snprintf(t_msg, sizeof(t_msg), "reading the status area: %s", hipGetErrorString(e));
        return lfail(DSPARK_EHIP, t_msg);
    }
    if (first_bad_block) *first_bad_block = w[kLyFirstBad];
    if (kept_blocks) *kept_blocks = w[kLyKept];
    set_last_error("");
    if (w[kLyFirstBad] >= 0) return lfail(DSPARK_EANCHOR, "a kept block has an anchor outside [0, S-2]", w[kLyFirstBad]);
    if (w[kLyOverflow]) return lfail(DSPARK_ECAPACITY, "kept blocks exceed max_kept_blocks", w[kLyKept]);
    return DSPARK_OK;
}
