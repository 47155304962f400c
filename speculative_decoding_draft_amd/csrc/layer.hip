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
// One workgroup per row (grid-stride); the row is read twice (the second
// read hits the cache).
template <typename T>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const T* __restrict__ x, size_t ldx, const T* __restrict__ g, T* __restrict__ y, size_t ldy,
    T* __restrict__ tail_out, int n_tail, size_t rows, int n, float eps) {
    __shared__ float red[kNormThreads / 64];
    for (size_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const T* xr = x + r * ldx;
        float ss = 0.f;
        for (int i = threadIdx.x; i < n; i += kNormThreads) {
            const float v = ldf(xr, i);
            ss += v * v;
        }
        const float inv = rsqrtf(block_sum(ss, red) / (float)n + eps);
        T* yr = y + r * ldy;
        for (int i = threadIdx.x; i < n; i += kNormThreads)
            stf(yr, i, ldf(xr, i) * inv * ldf(g, i));
        if (tail_out)
            for (int i = threadIdx.x; i < n_tail; i += kNormThreads)
                stf(tail_out + r * (size_t)n_tail, i, ldf(xr, n + i));
    }
}

// bf16 rows with n % 512 == 0 (n <= 512 * kMaxChunks) and 16-byte aligned
// rows: one wave per row, the row held in registers (n / 512 chunks of 8
// per lane), reductions by shuffles only.
constexpr int kMaxChunks = 16;
template <int CH>
__global__ __launch_bounds__(256) void rmsnorm_wave_kernel(
    const bf16* __restrict__ x, size_t ldx, const bf16* __restrict__ g, bf16* __restrict__ y,
    size_t ldy, bf16* __restrict__ tail_out, int n_tail, size_t rows, float eps) {
    const int lane = threadIdx.x & 63;
    constexpr int n = 512 * CH;
    for (size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows;
         r += (size_t)gridDim.x * 4) {
        const bf16* xr = x + r * ldx;
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
        bf16* yr = y + r * ldy;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const bf16x8 gw = gld16(g + 8 * (lane + 64 * c));
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)v[c][i] * inv * (float)gw[i]);
            gst16(yr + 8 * (lane + 64 * c), o);
        }
        if (tail_out)
            for (int i = lane; i < n_tail; i += 64) tail_out[r * (size_t)n_tail + i] = xr[n + i];
    }
}

template <typename T>
hipError_t launch_rmsnorm(const T* x, size_t ldx, const T* g, T* y, size_t ldy, T* tail,
                          int n_tail, size_t rows, int n, float eps, hipStream_t s) {
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
                           ldy, tail, n_tail, rows, eps);                                     \
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
                       tail, n_tail, rows, n, eps);
    return hipGetLastError();
}

// [rows][H][dc + dr] -> [rows][H][dc] and [rows][H][dr], in 16-byte pieces
// when dc and dr allow (vec elements of 16 bytes), element by element
// otherwise (vec = 1)
template <typename T>
__global__ __launch_bounds__(256) void split_heads_kernel(const T* __restrict__ q, T* __restrict__ qn,
                                                          T* __restrict__ qr, size_t rows, int H,
                                                          int dc, int dr, int vec) {
    const int w = dc + dr;
    const size_t per_row = (size_t)H * w / vec;
    const size_t total = rows * per_row;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (size_t)gridDim.x * blockDim.x) {
        const size_t r = e / per_row;
        const int k = (int)(e % per_row) * vec, h = k / w, j = k % w;
        const T* src = q + r * (size_t)H * w + k;
        T* dst = (j < dc) ? qn + (r * H + h) * (size_t)dc + j : qr + (r * H + h) * (size_t)dr + (j - dc);
        if (vec * sizeof(T) == 16) {
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
        } else {
            *dst = *src;
        }
    }
}

}  // namespace

// Workspace of dspark_mla_layer_fwd: the block's intermediates, then the
// attention's own workspace.
struct LayerLayout {
    size_t hn = 0, cq = 0, qf = 0, qn = 0, qr = 0, kvc = 0, kvb = 0, ckv_c = 0, kr_c = 0,
           ckv_b = 0, kr_b = 0, o = 0, attn = 0, total = 0;
};

LayerLayout layer_layout(const dspark_layer_desc& L, size_t attn_ws) {
    const dspark_attn_desc& d = L.attn;
    const size_t e = d.dtype == DSPARK_BF16 ? 2 : 4;
    const size_t q_rows = size_t(d.B) * kBlock * d.N, c_rows = size_t(d.B) * d.S;
    LayerLayout w;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    w.hn = take(q_rows * L.hidden * e);
    w.cq = take(q_rows * L.q_rank * e);
    w.qf = take(q_rows * d.n_heads * (d.d_nope + d.d_rope) * e);
    w.qn = take(q_rows * d.n_heads * d.d_nope * e);
    w.qr = take(q_rows * d.n_heads * d.d_rope * e + 16);
    w.kvc = take(c_rows * (d.d_latent + d.d_rope) * e);
    w.kvb = take(q_rows * (d.d_latent + d.d_rope) * e);
    w.ckv_c = take(c_rows * d.d_latent * e);
    w.kr_c = take(c_rows * d.d_rope * e + 16);
    w.ckv_b = take(q_rows * d.d_latent * e);
    w.kr_b = take(q_rows * d.d_rope * e + 16);
    w.o = take(q_rows * d.n_heads * d.d_v * e);
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
    if (!desc || desc->hidden < 1 || desc->q_rank < 1) return 0;
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
                        const dspark_attn_opts* opts, bool tune) {
    set_last_error("");
    if (!desc) return lfail(DSPARK_EINVAL, "desc is NULL");
    if (desc->hidden < 1 || desc->q_rank < 1)
        return lfail(DSPARK_EINVAL, "hidden and q_rank must be >= 1");
    if (!(desc->rms_eps >= 0.0)) return lfail(DSPARK_EINVAL, "rms_eps must be >= 0");
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

    const bool bf = d.dtype == DSPARK_BF16;
    const rocblas_datatype tio = bf ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    char* base = static_cast<char*>(workspace);
    void *hn = base + L.hn, *cq = base + L.cq, *qn = base + L.qn, *qr = base + L.qr;
    void *kvc = base + L.kvc, *kvb = base + L.kvb, *ckv_c = base + L.ckv_c, *kr_c = base + L.kr_c;
    void *ckv_b = base + L.ckv_b, *kr_b = base + L.kr_b, *o = base + L.o, *aws = base + L.attn;
    const int hid = desc->hidden, qk = desc->q_rank, H = d.n_heads;
    const int D = d.d_latent, dc = d.d_nope, dr = d.d_rope, dv = d.d_v;
    const int q_rows = d.B * kBlock * d.N, c_rows = d.B * d.S;
    const float eps = (float)desc->rms_eps;
    int k_ev = 0;
    auto mark = [&]() -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k_ev++]), s) : hipSuccess;
    };
    hipError_t he;
    auto norm = [&](const void* x, size_t ldx, const void* g, void* y, size_t ldy, void* tail,
                    int n_tail, size_t rows, int n) -> hipError_t {
        return bf ? launch_rmsnorm((const bf16*)x, ldx, (const bf16*)g, (bf16*)y, ldy,
                                   (bf16*)tail, n_tail, rows, n, eps, s)
                  : launch_rmsnorm((const float*)x, ldx, (const float*)g, (float*)y, ldy,
                                   (float*)tail, n_tail, rows, n, eps, s);
    };
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
    // h = RMSNorm(H)
    LSTEP_HIP(norm(h_draft, hid, g_in, hn, hid, nullptr, 0, q_rows, hid), "input RMSNorm launch");
    LMARK();
    // c^Q = RMSNorm(h W_qa^T)
    LSTEP_BLAS(gemm_nt(h, tio, tio, q_rows, qk, hid, hn, hid, w_qa, hid, 0.f, nullptr, 0, cq, qk, tune),
               "q_a_proj GEMM");
    LSTEP_HIP(norm(cq, qk, g_qa, cq, qk, nullptr, 0, q_rows, qk), "q_a RMSNorm launch");
    LMARK();
    // [q^C ; q^R] per head = c^Q W_qb^T (one GEMM: per-head strided-batched GEMMs
    // of 192 and 64 columns ran at half the rate), then split into the
    // attention's [row][head][dim] layouts
    void* qf = base + L.qf;
    LSTEP_BLAS(gemm_nt(h, tio, tio, q_rows, H * (dc + dr), qk, cq, qk, w_qb, qk, 0.f, nullptr, 0, qf,
                       H * (dc + dr), tune), "q_b_proj GEMM");
    {
        const int vec = (dc % 8 == 0 && dr % 8 == 0 && bf) ? 8 : ((dc % 4 == 0 && dr % 4 == 0 && !bf) ? 4 : 1);
        const size_t total = (size_t)q_rows * H * (dc + dr) / vec;
        const size_t want = (total + 255) / 256;
        const int grid = (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
        if (bf)
            hipLaunchKernelGGL(split_heads_kernel<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)qf,
                               (bf16*)qn, (bf16*)qr, (size_t)q_rows, H, dc, dr, vec);
        else
            hipLaunchKernelGGL(split_heads_kernel<float>, dim3(grid), dim3(256), 0, s,
                               (const float*)qf, (float*)qn, (float*)qr, (size_t)q_rows, H, dc, dr,
                               vec);
        LSTEP_HIP(hipGetLastError(), "q split launch");
    }
    LMARK();
    // [c^KV ; k^R] = [H^ctx ; h] W_kva^T, then c^KV <- RMSNorm(c^KV) and the k^R split
    LSTEP_BLAS(gemm_nt(h, tio, tio, c_rows, D + dr, hid, h_ctx, hid, w_kva, hid, 0.f, nullptr, 0, kvc,
                       D + dr, tune), "kv_a_proj (context) GEMM");
    LSTEP_BLAS(gemm_nt(h, tio, tio, q_rows, D + dr, hid, hn, hid, w_kva, hid, 0.f, nullptr, 0, kvb, D + dr,
                       tune), "kv_a_proj (draft) GEMM");
    LSTEP_HIP(norm(kvc, D + dr, g_kva, ckv_c, D, kr_c, dr, c_rows, D), "kv_a RMSNorm launch");
    LSTEP_HIP(norm(kvb, D + dr, g_kva, ckv_b, D, kr_b, dr, q_rows, D), "kv_a RMSNorm launch");
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
    // out = H + o W_o^T
    LSTEP_BLAS(gemm_nt(h, tio, tio, q_rows, hid, H * dv, o, H * dv, w_o, H * dv, 1.f, h_draft, hid, out,
                       hid, tune), "o_proj GEMM");
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
                     anchors, keep, out, workspace, ws_bytes, stream, opts, false);
}

dspark_status dspark_mla_layer_tune(const dspark_layer_desc* desc, const void* h_draft,
                                    const void* h_ctx, const void* g_in, const void* w_qa,
                                    const void* g_qa, const void* w_qb, const void* w_kva,
                                    const void* g_kva, const void* w_uk, const void* w_uv,
                                    const void* w_o, const int32_t* anchors, const uint8_t* keep,
                                    void* out, void* workspace, size_t ws_bytes, void* stream) {
    return layer_fwd(desc, h_draft, h_ctx, g_in, w_qa, g_qa, w_qb, w_kva, g_kva, w_uk, w_uv, w_o,
                     anchors, keep, out, workspace, ws_bytes, stream, nullptr, true);
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
