// The output head and the loss of a DSpark draft for one batch (GLM 5.2
// DSpark training-design page, §5 "输出头" and §6 "训练目标"):
//   L_k = H^(L) W_lm^T + markov_w1[x_{A+k}] markov_w2^T     draft logits
//   T_k = z_{A+k} W_lm^T                                   teacher logits
//   c_k = w_conf . [H^(L) ; markov_w1[x_{A+k}]]            confidence logit
//   ce = lse(L_k) - L_k[x_{A+k+1}],  l1 = |softmax(L_k) - softmax(T_k)|_1,
//   bce = BCE-with-logits(c_k, clip(1 - l1/2, 0, 1)),
// and their means over the steps of the §6 eval mask.
//
// Launches (one stream):
//   index   one workgroup: eval mask, one compact row per counted step, status
//   gather  one workgroup per row: [H^(L) row ; markov_w1 row] and
//           [z row ; 0], side by side for the GEMMs
//   GEMMs   rocBLAS, fp32 out: L = E W2^T, then L += H W_lm^T (beta = 1),
//           T = Z W_lm^T  ([rows, V] each, materialised: 2 x 3.2 GB for
//           5120 rows -- small against the HBM, and it replaces a second
//           lm_head pass)
//   stats   one workgroup per (row, 8192-column chunk): max and sum of
//           exp for L and T
//   l1      the same grid: the row's log-sum-exps from the chunk partials,
//           then sum |p - q| over the chunk
//   terms   one wave per step: ce, l1, the confidence logit, bce
//   reduce  one workgroup: the masked means, in a fixed order (fp64)
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "blas.hpp"
#include "kernels.hpp"

namespace dspark {

void set_last_error(const char* msg);    // api.hip: the text dspark_last_error() returns

namespace {

constexpr int kChunk = 8192;        // vocabulary columns per statistics workgroup
constexpr int kStatThreads = 256;   // kChunk / kStatThreads = 32 values per thread
constexpr int kPerThread = kChunk / kStatThreads;
constexpr int kIndexThreads = 1024;

// Status area of the loss workspace (int32 words at offset 0; word 1 holds
// the first bad block as in the attention's status area).
enum LossStatus {
    kLsKept = 0, kLsFirstBad = 1, kLsOverflow = 2, kLsBadToken = 3, kLsCounted = 4, kLsWords = 16
};

struct LossLayout {
    size_t status = 0, row_step = 0, step_row = 0, xd = 0, xt = 0, ld = 0, lt = 0, part = 0,
           l1p = 0, blas = 0, total = 0;
    int rows = 0;      // compact rows: one per counted step, at most this many
    int chunks = 0;    // ceil(V / kChunk)
};

// Rows the logits are formed for: max_counted_steps, else 5 per block of the
// block bound (max_kept_blocks, else B * N).
long long loss_rows(const dspark_loss_desc& d) {
    const long long bn = (long long)d.B * d.N;
    const long long all = (long long)kBlock * bn;
    if (d.max_counted_steps > 0) return std::min<long long>(d.max_counted_steps, all);
    const long long blocks = d.max_kept_blocks > 0 ? std::min<long long>(d.max_kept_blocks, bn) : bn;
    return (long long)kBlock * blocks;
}

LossLayout loss_layout(const dspark_loss_desc& d) {
    LossLayout w;
    const size_t e = d.dtype == DSPARK_BF16 ? 2 : 4;
    w.rows = (int)loss_rows(d);
    w.chunks = (d.vocab + kChunk - 1) / kChunk;
    const size_t rows = (size_t)w.rows, V = (size_t)d.vocab;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    w.status = take(kLsWords * 4);
    w.row_step = take(rows * 4);
    w.step_row = take((size_t)d.B * d.N * kBlock * 4);
    // draft rows [H^(L) | e] then teacher rows [z | 0], one [2 rows, d + r]
    // operand; the draft logits then the teacher's, one [2 rows, V] array
    w.xd = take(2 * rows * (size_t)(d.hidden + d.markov_rank) * e);
    w.xt = w.xd + rows * (size_t)(d.hidden + d.markov_rank) * e;
    w.ld = take(2 * rows * V * 4);
    w.lt = w.ld + rows * V * 4;
    w.part = take(rows * (size_t)w.chunks * 16);
    w.l1p = take(rows * (size_t)w.chunks * 4);
    w.blas = take(DSPARK_BLAS_WORKSPACE_BYTES);
    w.total = off;
    return w;
}

template <typename T> __device__ inline float tof(T v);
template <> __device__ inline float tof<float>(float v) { return v; }
template <> __device__ inline float tof<bf16>(bf16 v) { return (float)v; }

__device__ inline float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---- index: eval mask, one compact row per counted step, status --------
// Blocks are taken in (b, n) order; the counted steps of a kept block with a
// valid anchor (a prefix of its 5, by the cumprod) get the next rows.
// row_step [rows]: step b*N*5 + n*5 + k of each row (-1 past the last);
// step_row [B*N*5]: the row of each counted step (-1 otherwise).  One
// workgroup, any B * N.
__global__ __launch_bounds__(kIndexThreads) void loss_index_kernel(
    int B, int S, int N, int cap_rows, const int32_t* __restrict__ anchors,
    const uint8_t* __restrict__ keep, const uint8_t* __restrict__ loss_mask,
    int32_t* __restrict__ status, int32_t* __restrict__ row_step, int32_t* __restrict__ step_row,
    uint8_t* __restrict__ emask) {
    __shared__ int wsum[kIndexThreads / 64];
    __shared__ int base_s, bad_s, kept_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int total = B * N;
    if (tid == 0) {
        base_s = 0;
        bad_s = INT_MAX;
        kept_s = 0;
    }
    __syncthreads();
    for (int c0 = 0; c0 < total; c0 += kIndexThreads) {
        const int i = c0 + tid;
        int cnt = 0;
        if (i < total) {
            const int b = i / N;
            const int A = anchors[i];
            const bool kp = keep[i] != 0;
            const bool valid = kp && A >= 0 && A <= S - 2;
            if (kp && !valid) atomicMin(&bad_s, i);
            if (valid) atomicAdd(&kept_s, 1);
            // §6 eval_mask: A+k+1 < S, loss_mask[A+k+1] (position S-1 read
            // as 0), prefix cumprod along the block
            bool on = valid;
            for (int k = 0; k < kBlock; ++k) {
                const long long p = (long long)A + k + 1;
                on = on && p < S - 1 && loss_mask[(size_t)b * S + p] != 0;
                emask[(size_t)i * kBlock + k] = on ? 1 : 0;
                cnt += on ? 1 : 0;
            }
        }
        // exclusive scan of the counted steps over the workgroup
        int incl = cnt;
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        if (lane == 63) wsum[w] = incl;
        __syncthreads();
        int before = base_s, all = 0;
        for (int j = 0; j < kIndexThreads / 64; ++j) {
            if (j < w) before += wsum[j];
            all += wsum[j];
        }
        const int row0 = before + incl - cnt;
        if (i < total) {
            for (int k = 0; k < kBlock; ++k) {
                const int row = row0 + k;
                const bool here = k < cnt && row < cap_rows;
                step_row[(size_t)i * kBlock + k] = here ? row : -1;
                if (here) row_step[row] = i * kBlock + k;
            }
        }
        __syncthreads();                       // wsum and base_s are reused
        if (tid == 0) base_s += all;
        __syncthreads();
    }
    const int counted = base_s;
    for (int j = counted + tid; j < cap_rows; j += kIndexThreads) row_step[j] = -1;
    if (tid == 0) {
        status[kLsKept] = kept_s;
        status[kLsFirstBad] = bad_s == INT_MAX ? -1 : bad_s;
        status[kLsOverflow] = counted > cap_rows ? 1 : 0;
        status[kLsBadToken] = 0;
        status[kLsCounted] = counted;
    }
}

// ---- gather: for the row of step (b, n, k): xd[row] = [H^(L)[b, 5n+k] ;
// markov_w1[x_{A+k}]], xt[row] = [z[b, A+k] ; 0] (A+k <= S-2 for a counted
// step).  Rows past the last counted step are zero.  One workgroup per row.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void loss_gather_kernel(
    int S, int N, int V, int d, int r, const int32_t* __restrict__ row_step,
    const int32_t* __restrict__ anchors, const int32_t* __restrict__ ids,
    const T* __restrict__ h_final, const T* __restrict__ z, const T* __restrict__ w_m1,
    T* __restrict__ xd, T* __restrict__ xt, int32_t* __restrict__ status) {
    const int row = blockIdx.x;
    const int step = row_step[row];
    const int blk = step < 0 ? -1 : step / kBlock, k = step < 0 ? 0 : step % kBlock;
    T* xdr = xd + (size_t)row * (d + r);
    T* xtr = xt + (size_t)row * (d + r);     // [z | 0]: the Markov columns are 0
    constexpr int E = VEC ? 16 / (int)sizeof(T) : 1;    // elements per copy
    auto copy = [&](T* dst, const T* src, int n) {
        if (VEC) {
            for (int i = threadIdx.x; i < n / E; i += blockDim.x)
                reinterpret_cast<uint4*>(dst)[i] = src ? reinterpret_cast<const uint4*>(src)[i]
                                                       : make_uint4(0, 0, 0, 0);
        } else {
            for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = src ? src[i] : T(0);
        }
    };
    copy(xtr + d, nullptr, r);
    if (blk < 0) {
        copy(xdr, nullptr, d + r);
        copy(xtr, nullptr, d);
        return;
    }
    const int b = blk / N, n = blk % N;
    const int A = anchors[blk];
    const int pos = min(A + k, S - 1);
    int prev = ids[(size_t)b * S + pos];
    if (prev < 0 || prev >= V) {
        if (threadIdx.x == 0) status[kLsBadToken] = 1;   // every writer stores 1
        prev = prev < 0 ? 0 : V - 1;
    }
    copy(xdr, h_final + ((size_t)b * kBlock * N + (size_t)kBlock * n + k) * d, d);
    copy(xdr + d, w_m1 + (size_t)prev * r, r);
    copy(xtr, z + ((size_t)b * S + pos) * d, d);
}

__device__ inline bool row_live(int row, const int32_t* row_step) { return row_step[row] >= 0; }

// Loads this thread's values of a kChunk-column chunk [v0, v1) of a row
// (-inf outside it).
template <bool VEC>
__device__ inline void load_chunk(const float* __restrict__ rowp, int v0, int v1, float* x) {
    if (VEC) {
#pragma unroll
        for (int i = 0; i < kPerThread / 4; ++i) {
            const int v = v0 + 4 * (threadIdx.x + kStatThreads * i);
            if (v < v1) {          // v1 - v0 is a multiple of 4 here
                const float4 q = *reinterpret_cast<const float4*>(rowp + v);
                x[4 * i] = q.x; x[4 * i + 1] = q.y; x[4 * i + 2] = q.z; x[4 * i + 3] = q.w;
            } else {
                x[4 * i] = x[4 * i + 1] = x[4 * i + 2] = x[4 * i + 3] = -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int v = v0 + threadIdx.x + kStatThreads * i;
            x[i] = v < v1 ? rowp[v] : -INFINITY;
        }
    }
}

// Sum (or max) over the workgroup of two values; every thread gets them.
template <bool MAX>
__device__ inline float2 block_reduce2(float a, float b, float2* red) {
    a = MAX ? wave_max(a) : wave_sum(a);
    b = MAX ? wave_max(b) : wave_sum(b);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = make_float2(a, b);
    __syncthreads();
    float2 s = red[0];
#pragma unroll
    for (int i = 1; i < kStatThreads / 64; ++i) {
        s.x = MAX ? fmaxf(s.x, red[i].x) : s.x + red[i].x;
        s.y = MAX ? fmaxf(s.y, red[i].y) : s.y + red[i].y;
    }
    return s;
}

// ---- stats: per (row, chunk): {max L, sum exp(L - max), max T, sum exp(T - max)}
template <bool VEC>
__global__ __launch_bounds__(kStatThreads) void loss_stats_kernel(
    int V, int C, const int32_t* __restrict__ row_step,
    const float* __restrict__ ld, const float* __restrict__ lt, float4* __restrict__ part) {
    __shared__ float2 red[kStatThreads / 64];
    const int row = blockIdx.x / C, c = blockIdx.x % C;
    if (!row_live(row, row_step)) return;
    const int v0 = c * kChunk, v1 = min(V, v0 + kChunk);
    float x[kPerThread], y[kPerThread];
    load_chunk<VEC>(ld + (size_t)row * V, v0, v1, x);
    load_chunk<VEC>(lt + (size_t)row * V, v0, v1, y);
    float mx = -INFINITY, my = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        mx = fmaxf(mx, x[i]);
        my = fmaxf(my, y[i]);
    }
    const float2 m = block_reduce2<true>(mx, my, red);
    float sx = 0.f, sy = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        sx += __expf(x[i] - m.x);
        sy += __expf(y[i] - m.y);
    }
    const float2 s = block_reduce2<false>(sx, sy, red);
    if (threadIdx.x == 0) part[(size_t)row * C + c] = make_float4(m.x, s.x, m.y, s.y);
}

// The row's log-sum-exps of L and T from its C chunk partials (one wave).
__device__ inline float2 row_lse(const float4* __restrict__ p, int C) {
    const int lane = threadIdx.x & 63;
    float ml = -INFINITY, mt = -INFINITY;
    for (int c = lane; c < C; c += 64) {
        ml = fmaxf(ml, p[c].x);
        mt = fmaxf(mt, p[c].z);
    }
    ml = wave_max(ml);
    mt = wave_max(mt);
    float sl = 0.f, st = 0.f;
    for (int c = lane; c < C; c += 64) {
        sl += p[c].y * __expf(p[c].x - ml);
        st += p[c].w * __expf(p[c].z - mt);
    }
    sl = wave_sum(sl);
    st = wave_sum(st);
    return make_float2(ml + __logf(sl), mt + __logf(st));
}

// ---- l1: per (row, chunk): sum over the chunk of |p - q|
template <bool VEC>
__global__ __launch_bounds__(kStatThreads) void loss_l1_kernel(
    int V, int C, const int32_t* __restrict__ row_step,
    const float* __restrict__ ld, const float* __restrict__ lt, const float4* __restrict__ part,
    float* __restrict__ l1p) {
    __shared__ float2 red[kStatThreads / 64];
    __shared__ float2 lse_s;
    const int row = blockIdx.x / C, c = blockIdx.x % C;
    if (!row_live(row, row_step)) return;
    const int v0 = c * kChunk, v1 = min(V, v0 + kChunk);
    float x[kPerThread], y[kPerThread];
    load_chunk<VEC>(ld + (size_t)row * V, v0, v1, x);
    load_chunk<VEC>(lt + (size_t)row * V, v0, v1, y);
    if (threadIdx.x < 64) {
        const float2 l = row_lse(part + (size_t)row * C, C);
        if (threadIdx.x == 0) lse_s = l;
    }
    __syncthreads();
    const float2 lse = lse_s;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)      // padding: exp(-inf) = 0 on both sides
        acc += fabsf(__expf(x[i] - lse.x) - __expf(y[i] - lse.y));
    const float2 s = block_reduce2<false>(acc, 0.f, red);
    if (threadIdx.x == 0) l1p[(size_t)row * C + c] = s.x;
}

// ---- terms: one wave per step (b, n, k)
template <typename T>
__global__ __launch_bounds__(256) void loss_terms_kernel(
    int S, int N, int V, int d, int r, int C, const int32_t* __restrict__ step_row,
    const int32_t* __restrict__ anchors, const uint8_t* __restrict__ keep,
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ emask,
    const float4* __restrict__ part, const float* __restrict__ l1p, const float* __restrict__ ld,
    const T* __restrict__ xd, const T* __restrict__ w_conf, int32_t* __restrict__ status,
    float* __restrict__ terms, int n_pos) {
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (p >= n_pos) return;
    const int blk = p / kBlock, k = p % kBlock;
    float ce = 0.f, l1 = 0.f, cf = 0.f, bce = 0.f;
    const bool overflow = status[kLsOverflow] != 0;
    const int A = anchors[blk];
    const bool kp = keep[blk] != 0;
    const bool bad = kp && (A < 0 || A > S - 2);
    if (overflow || bad) {
        ce = l1 = cf = bce = NAN;
    } else if (kp && emask[p]) {
        const int row = step_row[p];                 // a counted step has a row (no overflow)
        const float2 lse = row_lse(part + (size_t)row * C, C);
        float s = 0.f;
        for (int c = lane; c < C; c += 64) s += l1p[(size_t)row * C + c];
        l1 = wave_sum(s);
        int y = ids[(size_t)(blk / N) * S + A + k + 1];
        if (y < 0 || y >= V) {                         // poisons the loss (reduce)
            if (lane == 0) status[kLsBadToken] = 1;
            y = y < 0 ? 0 : V - 1;
        }
        ce = lse.x - ld[(size_t)row * V + y];
        const T* xr = xd + (size_t)row * (d + r);
        float acc = 0.f;
        for (int i = lane; i < d + r; i += 64) acc += tof(xr[i]) * tof(w_conf[i]);
        cf = wave_sum(acc);
        const float a = fminf(fmaxf(1.f - 0.5f * l1, 0.f), 1.f);
        bce = fmaxf(cf, 0.f) - cf * a + log1pf(__expf(-fabsf(cf)));
    }
    if (lane == 0) {
        terms[p] = ce;
        terms[(size_t)n_pos + p] = l1;
        terms[2 * (size_t)n_pos + p] = cf;
        terms[3 * (size_t)n_pos + p] = bce;
    }
}

// ---- reduce: the masked means, in a fixed order, fp64
constexpr int kReduceThreads = 1024;
__global__ __launch_bounds__(kReduceThreads) void loss_reduce_kernel(
    int n_pos, const float* __restrict__ terms, const uint8_t* __restrict__ emask,
    const int32_t* __restrict__ status, double a_ce, double a_l1, double a_conf,
    float* __restrict__ loss) {
    __shared__ double red[4][kReduceThreads / 64];
    double s_ce = 0, s_l1 = 0, s_bce = 0, cnt = 0;
    for (int p = threadIdx.x; p < n_pos; p += kReduceThreads) {
        if (!emask[p]) continue;
        s_ce += terms[p];
        s_l1 += terms[(size_t)n_pos + p];
        s_bce += terms[3 * (size_t)n_pos + p];
        cnt += 1;
    }
    double v[4] = {s_ce, s_l1, s_bce, cnt};
    for (int q = 0; q < 4; ++q)
        for (int o = 32; o > 0; o >>= 1) v[q] += __shfl_xor(v[q], o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
        for (int q = 0; q < 4; ++q) red[q][w] = v[q];
    __syncthreads();
    if (threadIdx.x == 0) {
        double t[4] = {0, 0, 0, 0};
        for (int q = 0; q < 4; ++q)
            for (int i = 0; i < kReduceThreads / 64; ++i) t[q] += red[q][i];
        const bool poisoned = status[kLsFirstBad] >= 0 || status[kLsOverflow] != 0 ||
                              status[kLsBadToken] != 0;
        double m_ce = 0, m_l1 = 0, m_bce = 0;
        if (t[3] > 0) {
            m_ce = t[0] / t[3];
            m_l1 = t[1] / t[3];
            m_bce = t[2] / t[3];
        }
        if (poisoned) m_ce = m_l1 = m_bce = NAN;
        loss[0] = (float)(a_ce * m_ce + a_l1 * m_l1 + a_conf * m_bce);
        loss[1] = (float)m_ce;
        loss[2] = (float)m_l1;
        loss[3] = (float)m_bce;
        loss[4] = (float)t[3];
    }
}

thread_local char t_msg[512];

dspark_status lsfail(dspark_status code, const char* msg) {
    set_last_error(msg);
    return code;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* check_desc(const dspark_loss_desc* d) {
    if (!d) return "desc is NULL";
    if (d->B < 0 || d->S < 1 || d->N < 0) return "need B >= 0, S >= 1, N >= 0";
    if (d->vocab < 1 || d->hidden < 1 || d->markov_rank < 1)
        return "vocab, hidden and markov_rank must be >= 1";
    if (d->dtype != DSPARK_BF16 && d->dtype != DSPARK_F32) return "dtype must be DSPARK_BF16 or DSPARK_F32";
    if (d->max_kept_blocks < 0 || d->max_counted_steps < 0)
        return "max_kept_blocks and max_counted_steps must be >= 0";
    if ((d->w_lm_ld != 0 && d->w_lm_ld < d->hidden) || (d->w_m2_ld != 0 && d->w_m2_ld < d->markov_rank))
        return "w_lm_ld / w_m2_ld must be 0 or at least hidden / markov_rank";
    if ((long long)d->B * d->N * kBlock > INT_MAX / 4) return "B * N too large";
    if ((long long)d->B * d->S > INT_MAX) return "B * S too large";
    const long long rows = loss_rows(*d);
    const long long C = (d->vocab + kChunk - 1) / kChunk;
    if (rows * C > INT_MAX) return "rows x vocabulary chunks exceeds the grid limit";
    if ((long long)d->hidden + d->markov_rank > INT_MAX / 2) return "hidden + markov_rank too large";
    return nullptr;
}

dspark_status loss_fwd(const dspark_loss_desc* desc, const int32_t* ids, const uint8_t* lmask,
                       const int32_t* anchors, const uint8_t* keep, const void* h_final,
                       const void* z, const void* w_lm, const void* w_m1, const void* w_m2,
                       const void* w_conf, float* terms, uint8_t* emask, float* loss,
                       void* workspace, size_t ws_bytes, void* stream,
                       const dspark_attn_opts* opts, dspark_gemm_choices* tuned) {
    set_last_error("");
    if (const char* why = check_desc(desc)) return lsfail(DSPARK_EINVAL, why);
    const dspark_loss_desc& d = *desc;
    const void* ptrs[] = {ids, lmask, anchors, keep, h_final, z, w_lm, w_m1, w_m2, w_conf,
                          terms, emask, loss};
    const char* names[] = {"input_ids", "loss_mask", "anchors", "keep", "h_final", "z", "w_lm",
                           "w_m1", "w_m2", "w_conf", "terms", "eval_mask", "loss"};
    for (int i = 0; i < 13; ++i) {
        if (!ptrs[i]) {
            snprintf(t_msg, sizeof(t_msg), "%s is NULL", names[i]);
            return lsfail(DSPARK_EINVAL, t_msg);
        }
        if (i >= 4 && i <= 9 && !al16(ptrs[i])) {
            snprintf(t_msg, sizeof(t_msg), "%s must be 16-byte aligned", names[i]);
            return lsfail(DSPARK_EINVAL, t_msg);
        }
    }
    if (((reinterpret_cast<uintptr_t>(terms) | reinterpret_cast<uintptr_t>(loss)) & 3u) ||
        (reinterpret_cast<uintptr_t>(ids) & 3u) || (reinterpret_cast<uintptr_t>(anchors) & 3u))
        return lsfail(DSPARK_EINVAL, "input_ids, anchors, terms and loss must be 4-byte aligned");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return lsfail(DSPARK_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    const LossLayout L = loss_layout(d);
    if (ws_bytes < L.total) {
        snprintf(t_msg, sizeof(t_msg), "workspace too small; bytes needed (%zu)", L.total);
        return lsfail(DSPARK_EWORKSPACE, t_msg);
    }
    void* const* ev = (opts && opts->stage_events) ? opts->stage_events : nullptr;
    constexpr int kEvents = 6;
    if (ev && opts->n_stage_events < kEvents)
        return lsfail(DSPARK_EINVAL, "this call records 6 stage events");

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = d.dtype == DSPARK_BF16;
    const int B = d.B, S = d.S, N = d.N, V = d.vocab, hd = d.hidden, rk = d.markov_rank;
    const int n_pos = B * N * kBlock;
    char* base = static_cast<char*>(workspace);
    int32_t* status = reinterpret_cast<int32_t*>(base + L.status);
    int32_t* row_step = reinterpret_cast<int32_t*>(base + L.row_step);
    int32_t* step_row = reinterpret_cast<int32_t*>(base + L.step_row);
    void* xd = base + L.xd;
    void* xt = base + L.xt;
    float* ld = reinterpret_cast<float*>(base + L.ld);
    float* lt = reinterpret_cast<float*>(base + L.lt);
    float4* part = reinterpret_cast<float4*>(base + L.part);
    float* l1p = reinterpret_cast<float*>(base + L.l1p);
    const int C = L.chunks, rows = L.rows;

    int k_ev = 0;
    hipError_t he = hipSuccess;
    auto mark = [&]() -> hipError_t {
        return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[k_ev++]), s) : hipSuccess;
    };
#define LS_HIP(call, what)                                                          \
    do {                                                                            \
        if ((he = (call)) != hipSuccess) {                                          \
            snprintf(t_msg, sizeof(t_msg), "%s: %s", what, hipGetErrorString(he));  \
            return lsfail(DSPARK_EHIP, t_msg);                                      \
        }                                                                           \
    } while (0)

    rocblas_handle h = nullptr;
    if (rows > 0) {
        const rocblas_status bs = blas_handle(s, &h);
        if (bs != rocblas_status_success) {
            snprintf(t_msg, sizeof(t_msg), "rocBLAS handle set-up failed (%d)", (int)bs);
            return lsfail(DSPARK_EHIP, t_msg);
        }
    }
    // rocBLAS works in the workspace's own area
    if (h) {
        const rocblas_status ws_st = blas_use_workspace(
            h, static_cast<char*>(workspace) + L.blas, DSPARK_BLAS_WORKSPACE_BYTES);
        if (ws_st != rocblas_status_success) {
            snprintf(t_msg, sizeof(t_msg), "rocblas_set_workspace failed (%d)", (int)ws_st);
            return lsfail(DSPARK_EHIP, t_msg);
        }
    }
    const bool tune = tuned != nullptr;
    if (tuned) *tuned = dspark_gemm_choices{};
    GemmPick pick{tuned ? tuned : const_cast<dspark_gemm_choices*>(opts ? opts->gemm_choices
                                                                          : nullptr),
                  tune, 0};
    LS_HIP(mark(), "hipEventRecord");
    hipLaunchKernelGGL(loss_index_kernel, dim3(1), dim3(kIndexThreads), 0, s, B, S, N, L.rows,
                       anchors, keep, lmask, status, row_step, step_row, emask);
    LS_HIP(hipGetLastError(), "index launch");
    if (rows > 0) {
        const bool vec = ((size_t)hd * (bf ? 2 : 4)) % 16 == 0 && ((size_t)rk * (bf ? 2 : 4)) % 16 == 0;
#define LS_GATHER(T, V_)                                                                      \
    hipLaunchKernelGGL((loss_gather_kernel<T, V_>), dim3(rows), dim3(256), 0, s, S, N, V, hd, rk, \
                       row_step, anchors, ids, (const T*)h_final, (const T*)z, (const T*)w_m1,    \
                       (T*)xd, (T*)xt, status)
        if (bf) {
            if (vec) LS_GATHER(bf16, true); else LS_GATHER(bf16, false);
        } else {
            if (vec) LS_GATHER(float, true); else LS_GATHER(float, false);
        }
#undef LS_GATHER
        LS_HIP(hipGetLastError(), "gather launch");
    }
    LS_HIP(mark(), "hipEventRecord");
    if (rows > 0) {
        const rocblas_datatype ti = bf ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
        const rocblas_datatype to = rocblas_datatype_f32_r;
        const int ldx = hd + rk;
        const char* bad = nullptr;
        rocblas_status bs = rocblas_status_success;
        const size_t e = bf ? 2 : 4;
        const int lm_ld = d.w_lm_ld > 0 ? d.w_lm_ld : hd, m2_ld = d.w_m2_ld > 0 ? d.w_m2_ld : rk;
        const bool fused = lm_ld == ldx && m2_ld == ldx &&
                           (const char*)w_m2 == (const char*)w_lm + (size_t)hd * e;
        if (fused) {
            // [H^(L) | e ; z | 0] [W_lm | W2]^T: draft and teacher logits at once
            if ((bs = gemm_nt(h, ti, to, 2 * rows, V, ldx, xd, ldx, w_lm, ldx, 0.f, nullptr, 0, ld,
                              V, &pick)) != rocblas_status_success)
                bad = "logits GEMM";
        } else {
            const void* xe = (const char*)xd + (size_t)hd * e;
            // L = E W2^T, then L += H W_lm^T in place (GEMMs 0 and 1).  Tuning
            // the in-place GEMM runs it many times over L, so after a tuning
            // pass both are run again with the choices just recorded.
            for (int pass = 0; pass < (tune ? 2 : 1) && !bad; ++pass) {
                GemmPick pp{pick.table, tune && pass == 0, 0};
                if ((bs = gemm_nt(h, ti, to, rows, V, rk, xe, ldx, w_m2, m2_ld, 0.f, nullptr, 0, ld,
                                  V, &pp)) != rocblas_status_success)
                    bad = "Markov GEMM";
                else if ((bs = gemm_nt(h, ti, to, rows, V, hd, xd, ldx, w_lm, lm_ld, 1.f, nullptr, 0,
                                       ld, V, &pp)) != rocblas_status_success)
                    bad = "draft lm_head GEMM";
            }
            pick.next = 2;
            if (!bad && (bs = gemm_nt(h, ti, to, rows, V, hd, xt, ldx, w_lm, lm_ld, 0.f, nullptr, 0,
                                      lt, V, &pick)) != rocblas_status_success)
                bad = "teacher lm_head GEMM";
        }
        if (bad) {
            snprintf(t_msg, sizeof(t_msg), "%s failed (rocBLAS status %d)", bad, (int)bs);
            return lsfail(DSPARK_EHIP, t_msg);
        }
    }
    LS_HIP(mark(), "hipEventRecord");
    const bool v4 = V % 4 == 0;
    if (rows > 0) {
        if (v4)
            hipLaunchKernelGGL(loss_stats_kernel<true>, dim3(rows * C), dim3(kStatThreads), 0, s, V, C,
                               row_step, ld, lt, part);
        else
            hipLaunchKernelGGL(loss_stats_kernel<false>, dim3(rows * C), dim3(kStatThreads), 0, s, V,
                               C, row_step, ld, lt, part);
        LS_HIP(hipGetLastError(), "stats launch");
    }
    LS_HIP(mark(), "hipEventRecord");
    if (rows > 0) {
        if (v4)
            hipLaunchKernelGGL(loss_l1_kernel<true>, dim3(rows * C), dim3(kStatThreads), 0, s, V, C,
                               row_step, ld, lt, part, l1p);
        else
            hipLaunchKernelGGL(loss_l1_kernel<false>, dim3(rows * C), dim3(kStatThreads), 0, s, V, C,
                               row_step, ld, lt, part, l1p);
        LS_HIP(hipGetLastError(), "l1 launch");
    }
    LS_HIP(mark(), "hipEventRecord");
    if (n_pos > 0) {
        const int grid = (n_pos + 3) / 4;
        if (bf)
            hipLaunchKernelGGL(loss_terms_kernel<bf16>, dim3(grid), dim3(256), 0, s, S, N, V, hd, rk, C,
                               step_row, anchors, keep, ids, emask, part, l1p, ld,
                               (const bf16*)xd, (const bf16*)w_conf, status, terms, n_pos);
        else
            hipLaunchKernelGGL(loss_terms_kernel<float>, dim3(grid), dim3(256), 0, s, S, N, V, hd, rk,
                               C, step_row, anchors, keep, ids, emask, part, l1p, ld,
                               (const float*)xd, (const float*)w_conf, status, terms, n_pos);
        LS_HIP(hipGetLastError(), "terms launch");
    }
    hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, s, n_pos, terms, emask,
                       status, d.alpha_ce, d.alpha_l1, d.alpha_conf, loss);
    LS_HIP(hipGetLastError(), "reduce launch");
    LS_HIP(mark(), "hipEventRecord");
#undef LS_HIP
    return DSPARK_OK;
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" {

size_t dspark_loss_workspace_size(const dspark_loss_desc* desc) {
    if (const char* why = check_desc(desc)) {
        set_last_error(why);
        return 0;
    }
    return loss_layout(*desc).total;
}

dspark_status dspark_loss_fwd_ex(const dspark_loss_desc* desc, const int32_t* input_ids,
                                 const uint8_t* loss_mask, const int32_t* anchors,
                                 const uint8_t* keep, const void* h_final, const void* z,
                                 const void* w_lm, const void* w_m1, const void* w_m2,
                                 const void* w_conf, float* terms, uint8_t* eval_mask,
                                 float* loss, void* workspace, size_t ws_bytes, void* stream,
                                 const dspark_attn_opts* opts) {
    return loss_fwd(desc, input_ids, loss_mask, anchors, keep, h_final, z, w_lm, w_m1, w_m2,
                    w_conf, terms, eval_mask, loss, workspace, ws_bytes, stream, opts, nullptr);
}

dspark_status dspark_loss_fwd(const dspark_loss_desc* desc, const int32_t* input_ids,
                              const uint8_t* loss_mask, const int32_t* anchors,
                              const uint8_t* keep, const void* h_final, const void* z,
                              const void* w_lm, const void* w_m1, const void* w_m2,
                              const void* w_conf, float* terms, uint8_t* eval_mask, float* loss,
                              void* workspace, size_t ws_bytes, void* stream) {
    return loss_fwd(desc, input_ids, loss_mask, anchors, keep, h_final, z, w_lm, w_m1, w_m2,
                    w_conf, terms, eval_mask, loss, workspace, ws_bytes, stream, nullptr, nullptr);
}

dspark_status dspark_loss_tune(const dspark_loss_desc* desc, const int32_t* input_ids,
                               const uint8_t* loss_mask, const int32_t* anchors,
                               const uint8_t* keep, const void* h_final, const void* z,
                               const void* w_lm, const void* w_m1, const void* w_m2,
                               const void* w_conf, float* terms, uint8_t* eval_mask, float* loss,
                               void* workspace, size_t ws_bytes, void* stream,
                               dspark_gemm_choices* choices) {
    if (!choices) return lsfail(DSPARK_EINVAL, "choices is NULL");
    return loss_fwd(desc, input_ids, loss_mask, anchors, keep, h_final, z, w_lm, w_m1, w_m2,
                    w_conf, terms, eval_mask, loss, workspace, ws_bytes, stream, nullptr, choices);
}

dspark_status dspark_loss_read_status(const void* workspace, void* stream,
                                      int32_t* first_bad_block, int32_t* kept_blocks,
                                      int32_t* counted_steps) {
    if (first_bad_block) *first_bad_block = -1;
    if (kept_blocks) *kept_blocks = 0;
    if (counted_steps) *counted_steps = 0;
    if (!workspace) return lsfail(DSPARK_EWORKSPACE, "workspace is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    int32_t w[kLsWords];
    if (e == hipSuccess) e = hipMemcpy(w, workspace, sizeof(w), hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
        snprintf(t_msg, sizeof(t_msg), "reading the status area: %s", hipGetErrorString(e));
        return lsfail(DSPARK_EHIP, t_msg);
    }
    if (first_bad_block) *first_bad_block = w[kLsFirstBad];
    if (kept_blocks) *kept_blocks = w[kLsKept];
    if (counted_steps) *counted_steps = w[kLsCounted];
    set_last_error("");
    if (w[kLsFirstBad] >= 0) {
        snprintf(t_msg, sizeof(t_msg), "kept block %d has an anchor outside [0, S-2]", w[kLsFirstBad]);
        return lsfail(DSPARK_EANCHOR, t_msg);
    }
    if (w[kLsOverflow]) {
        snprintf(t_msg, sizeof(t_msg), "%d counted steps exceed the row bound", w[kLsCounted]);
        return lsfail(DSPARK_ECAPACITY, t_msg);
    }
    if (w[kLsBadToken]) return lsfail(DSPARK_EINVAL, "a token id read by the loss lies outside [0, V)");
    return DSPARK_OK;
}

}  // extern "C"
