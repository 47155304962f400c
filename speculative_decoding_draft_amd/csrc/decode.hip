// Inference-time drafting (GLM 5.2 DSpark training-design page, parameter
// summary "KV cache": a draft layer keeps about W cached tokens of 576
// numbers; the MTP / DSA explainer page, "Rejection Sampling"):
//   * the draft cache: a ring of C slots per layer and sequence (position p
//     in slot p mod C) and its append kernel;
//   * decode attention: the ring window of each sequence's block gathered
//     into a short contiguous context, then the training attention
//     (dspark_attn_fwd_ex) on B one-block problems with every position
//     moved by the same offset -- RoPE scores depend only on position
//     differences;
//   * verification of drafted tokens by rejection sampling (or target-only):
//     per-chunk softmax statistics of every row, per-chunk overlap and
//     residual mass, and one workgroup per sequence that takes the
//     accept / reject decisions and draws the next token by inverse CDF.
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "kernels.hpp"

namespace dspark {

void set_last_error(const char* msg);    // api.hip

namespace {

thread_local char t_msg[512];

dspark_status dfail(dspark_status code, const char* msg) {
    set_last_error(msg);
    return code;
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// draft cache
// ---------------------------------------------------------------------------

// Copies n elements (16-byte pieces when VEC) with the 64 lanes of a wave.
template <typename T, bool VEC>
__device__ inline void copy_row(T* __restrict__ dst, const T* __restrict__ src, int n, int lane) {
    if (VEC) {
        constexpr int E = 16 / (int)sizeof(T);
        for (int i = lane; i < n / E; i += 64)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        for (int i = lane; i < n; i += 64) dst[i] = src[i];
    }
}

// One wave per (sequence, new row); 4 waves per workgroup.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void cache_append_kernel(
    int B, int C, int D, int dr, int max_new, const int32_t* __restrict__ pos0,
    const int32_t* __restrict__ n_new, const T* __restrict__ new_ckv, const T* __restrict__ new_kr,
    T* __restrict__ cache_ckv, T* __restrict__ cache_kr) {
    const long long id = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (id >= (long long)B * max_new) return;
    const int b = (int)(id / max_new), t = (int)(id % max_new);
    const int n = min(n_new[b], max_new);
    if (t >= n || t < n - C) return;              // beyond the rows, or overwritten later
    const long long p = (long long)pos0[b] + t;
    if (p < 0) return;
    const size_t slot = (size_t)(p % C);
    copy_row<T, VEC>(cache_ckv + ((size_t)b * C + slot) * D, new_ckv + ((size_t)b * max_new + t) * D,
                     D, lane);
    if (dr > 0)
        copy_row<T, VEC>(cache_kr + ((size_t)b * C + slot) * dr,
                         new_kr + ((size_t)b * max_new + t) * dr, dr, lane);
}

// The window of sequence b: rows i < A' = min(A, W-1) of win_ckv / win_kr
// hold position A - A' + i from the ring; anchors2[b] = A', keep2[b] =
// active.  One wave per (sequence, row).  A negative anchor is passed on as
// it is (the attention reports it).
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void decode_gather_kernel(
    int B, int C, int W, int D, int dr, int rows, const int32_t* __restrict__ anchors,
    const uint8_t* __restrict__ active, const T* __restrict__ cache_ckv,
    const T* __restrict__ cache_kr, T* __restrict__ win_ckv, T* __restrict__ win_kr,
    int32_t* __restrict__ anchors2, uint8_t* __restrict__ keep2) {
    const long long id = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (id >= (long long)B * rows) return;
    const int b = (int)(id / rows), i = (int)(id % rows);
    const int A = anchors[b];
    const bool act = active[b] != 0;
    const int A2 = A >= 0 ? min(A, W - 1) : A;
    if (i == 0 && lane == 0) {
        anchors2[b] = A2;
        keep2[b] = act ? 1 : 0;
    }
    if (!act || A < 0 || i >= A2) return;         // rows the attention does not read
    const long long p = (long long)A - A2 + i;
    const size_t slot = (size_t)(p % C);
    copy_row<T, VEC>(win_ckv + ((size_t)b * rows + i) * D, cache_ckv + ((size_t)b * C + slot) * D, D,
                     lane);
    if (dr > 0)
        copy_row<T, VEC>(win_kr + ((size_t)b * rows + i) * dr, cache_kr + ((size_t)b * C + slot) * dr,
                         dr, lane);
}

struct DecodeLayout {
    size_t attn = 0, anchors2 = 0, keep2 = 0, win_ckv = 0, win_kr = 0, total = 0;
    dspark_attn_desc sub{};
    size_t attn_bytes = 0;
};

const char* check_decode(const dspark_decode_desc* d) {
    if (!d) return "desc is NULL";
    if (d->attn.N != 1) return "decode descriptors have N = 1 (one block per sequence)";
    if (d->attn.window < 1) return "window must be >= 1";
    if (d->cache_slots < 1 || d->cache_slots < d->attn.window - 1)
        return "cache_slots must be >= max(1, window - 1)";
    return nullptr;
}

// The one-block problem the attention runs: S' = W + 1 context rows (the
// window occupies rows [0, A') with A' <= W - 1 <= S' - 2).
dspark_attn_desc sub_desc(const dspark_decode_desc& d) {
    dspark_attn_desc s = d.attn;
    s.S = d.attn.window + 1;
    s.N = 1;
    return s;
}

bool decode_layout(const dspark_decode_desc& d, DecodeLayout* w) {
    w->sub = sub_desc(d);
    w->attn_bytes = dspark_attn_workspace_size(&w->sub);
    if (w->attn_bytes == 0) return false;
    const size_t e = d.attn.dtype == DSPARK_BF16 ? 2 : 4;
    const size_t B = (size_t)d.attn.B, rows = (size_t)w->sub.S;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    w->attn = take(w->attn_bytes);                // status area at offset 0
    w->anchors2 = take(B * 4);
    w->keep2 = take(B);
    w->win_ckv = take(B * rows * (size_t)d.attn.d_latent * e);
    w->win_kr = take(B * rows * (size_t)d.attn.d_rope * e + 16);
    w->total = off;
    return true;
}

// ---------------------------------------------------------------------------
// verification
// ---------------------------------------------------------------------------

constexpr int kVChunk = 8192;
constexpr int kVThreads = 256;
constexpr int kVPer = kVChunk / kVThreads;     // 32 values per thread

__device__ inline float vwave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float vwave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Row r of the stacked rows: draft rows b*K + k first, then target rows
// b*(K+1) + k.
__device__ inline const float* row_ptr(int r, int B, int K, int V, const float* dl, const float* tl) {
    const int nd = B * K;
    return r < nd ? dl + (size_t)r * V : tl + (size_t)(r - nd) * V;
}

// This thread's values of the chunk [v0, v1) of a row, times inv_t (-inf
// outside the chunk), and their indices: 16-byte loads when VEC (V % 4 == 0),
// value 4 (t + 256 i) + e; single loads otherwise, value t + 256 i.
template <bool VEC>
__device__ inline void load_vals(const float* __restrict__ x, int v0, int v1, float inv_t,
                                 float* val) {
    if (VEC) {
#pragma unroll
        for (int i = 0; i < kVPer / 4; ++i) {
            const int v = v0 + 4 * (threadIdx.x + kVThreads * i);
            if (v < v1) {
                const float4 q = *reinterpret_cast<const float4*>(x + v);
                val[4 * i] = q.x * inv_t; val[4 * i + 1] = q.y * inv_t;
                val[4 * i + 2] = q.z * inv_t; val[4 * i + 3] = q.w * inv_t;
            } else {
                val[4 * i] = val[4 * i + 1] = val[4 * i + 2] = val[4 * i + 3] = -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kVPer; ++i) {
            const int v = v0 + threadIdx.x + kVThreads * i;
            val[i] = v < v1 ? x[v] * inv_t : -INFINITY;
        }
    }
}

template <bool VEC>
__device__ inline int val_index(int v0, int i) {
    return VEC ? v0 + 4 * ((int)threadIdx.x + kVThreads * (i / 4)) + (i % 4)
               : v0 + (int)threadIdx.x + kVThreads * i;
}

// Per (row, chunk): {max of x/T, sum exp(x/T - max), index of the first
// maximum, x/T at the row's drafted token when the chunk holds it (else 0)}.
// The drafted token of draft row b K + k and target row b (K+1) + k is
// tokens[b K + k]; the last target row of a sequence has none.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void verify_stats_kernel(
    int B, int K, int V, int C, float inv_t, const float* __restrict__ dl,
    const float* __restrict__ tl, const int32_t* __restrict__ tokens,
    float4* __restrict__ part) {
    __shared__ float red_m[kVThreads / 64];
    __shared__ int red_i[kVThreads / 64];
    __shared__ float red_s[kVThreads / 64];
    __shared__ float tok_val;
    // Rows in the order the overlap pass wants them still cached: every
    // sequence's last target row first (the overlap pass does not read it),
    // then per sequence its K drafted rows and K target rows.  The overlap
    // pass walks the sequences downwards, so it first reads the rows read
    // here last, which the Infinity Cache still holds.
    const int nb = blockIdx.x / C, c = blockIdx.x % C;
    int r;
    if (nb < B) {
        r = B * K + nb * (K + 1) + K;
    } else {
        const int bb = (nb - B) / (2 * K), j = (nb - B) % (2 * K);
        r = j < K ? bb * K + j : B * K + bb * (K + 1) + (j - K);
    }
    const float* x = row_ptr(r, B, K, V, dl, tl);
    const int v0 = c * kVChunk, v1 = min(V, v0 + kVChunk);
    const int w = threadIdx.x >> 6;
    int tok = -1;
    if (r < B * K) {
        tok = tokens[r];
    } else {
        const int bb = (r - B * K) / (K + 1), k = (r - B * K) % (K + 1);
        if (k < K) tok = tokens[bb * K + k];
    }
    const bool has_tok = tok >= v0 && tok < v1;     // uniform: one thread holds the value
    float val[kVPer];
    load_vals<VEC>(x, v0, v1, inv_t, val);
    if (has_tok) {
#pragma unroll
        for (int i = 0; i < kVPer; ++i)
            if (val_index<VEC>(v0, i) == tok) tok_val = val[i];
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kVPer; ++i) m = fmaxf(m, val[i]);
    m = vwave_max(m);
    if ((threadIdx.x & 63) == 0) red_m[w] = m;
    __syncthreads();
    m = red_m[0];
#pragma unroll
    for (int i = 1; i < kVThreads / 64; ++i) m = fmaxf(m, red_m[i]);
    // first index of the maximum, and the sum of exponentials
    int mi = INT_MAX;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
        if (val[i] == m) mi = min(mi, val_index<VEC>(v0, i));
        s += __expf(val[i] - m);
    }
    for (int o = 32; o > 0; o >>= 1) mi = min(mi, __shfl_xor(mi, o));
    s = vwave_sum(s);
    if ((threadIdx.x & 63) == 0) {
        red_i[w] = mi;
        red_s[w] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        int ti = INT_MAX;
        for (int i = 0; i < kVThreads / 64; ++i) {
            t += red_s[i];
            ti = min(ti, red_i[i]);
        }
        part[(size_t)r * C + c] = make_float4(m, t, __int_as_float(ti), has_tok ? tok_val : 0.f);
    }
}

// log-sum-exp of a row from its C partials (one wave; lanes stride the chunks).
__device__ inline float chunk_lse(const float4* __restrict__ p, int C) {
    const int lane = threadIdx.x & 63;
    float m = -INFINITY;
    for (int c = lane; c < C; c += 64) m = fmaxf(m, p[c].x);
    m = vwave_max(m);
    float s = 0.f;
    for (int c = lane; c < C; c += 64) s += p[c].y * __expf(p[c].x - m);
    return m + __logf(vwave_sum(s));
}

// Per (drafted row, chunk): {sum min(p, q), sum max(0, p - q)}.
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void verify_overlap_kernel(
    int B, int K, int V, int C, float inv_t, const float* __restrict__ dl,
    const float* __restrict__ tl, const float4* __restrict__ part, float2* __restrict__ ov) {
    __shared__ float2 lse_s;
    __shared__ float2 red[kVThreads / 64];
    // drafted rows from the last down (see verify_stats_kernel)
    const int r = B * K - 1 - (int)blockIdx.x / C, c = blockIdx.x % C;   // r = b*K + k
    const int b = r / K, k = r % K;
    const int rt = B * K + b * (K + 1) + k;                // the target row
    // wave 0 requests the two rows' chunk partials (one per lane when
    // C <= 64) before the chunk's values, so that the log-sum-exps overlap
    // the value loads
    const int lane = threadIdx.x & 63;
    const bool one_per_lane = C <= 64;
    float4 pq = make_float4(-INFINITY, 0.f, 0.f, 0.f), pp = pq;
    if (threadIdx.x < 64 && one_per_lane && lane < C) {
        pq = part[(size_t)r * C + lane];
        pp = part[(size_t)rt * C + lane];
    }
    const float* q = dl + (size_t)r * V;
    const float* p = tl + ((size_t)b * (K + 1) + k) * V;
    const int v0 = c * kVChunk, v1 = min(V, v0 + kVChunk);
    float xq[kVPer], xp[kVPer];
    load_vals<VEC>(q, v0, v1, inv_t, xq);
    load_vals<VEC>(p, v0, v1, inv_t, xp);
    if (threadIdx.x < 64) {
        float lq, lp;
        if (one_per_lane) {     // the same operations as chunk_lse
            const float mq = vwave_max(pq.x), mp = vwave_max(pp.x);
            lq = mq + __logf(vwave_sum(pq.y * __expf(pq.x - mq)));
            lp = mp + __logf(vwave_sum(pp.y * __expf(pp.x - mp)));
        } else {
            lq = chunk_lse(part + (size_t)r * C, C);
            lp = chunk_lse(part + (size_t)rt * C, C);
        }
        if (threadIdx.x == 0) lse_s = make_float2(lq, lp);
    }
    __syncthreads();
    const float2 lse = lse_s;
    float mn = 0.f, res = 0.f;
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {      // -inf padding: both terms 0
        const float qv = __expf(xq[i] - lse.x);
        const float pv = __expf(xp[i] - lse.y);
        mn += fminf(pv, qv);
        res += fmaxf(pv - qv, 0.f);
    }
    mn = vwave_sum(mn);
    res = vwave_sum(res);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = make_float2(mn, res);
    __syncthreads();
    if (threadIdx.x == 0) {
        float2 t = make_float2(0.f, 0.f);
        for (int i = 0; i < kVThreads / 64; ++i) {
            t.x += red[i].x;
            t.y += red[i].y;
        }
        ov[(size_t)r * C + c] = t;
    }
}

// Index of a row's first maximum from its C partials (one wave; lanes stride
// the chunks): the largest value, the smallest index among equal values.
__device__ inline int chunk_top(const float4* __restrict__ p, int C) {
    float m = -INFINITY;
    int mi = INT_MAX;
    for (int c = threadIdx.x & 63; c < C; c += 64) {
        const float x = p[c].x;
        const int qi = __float_as_int(p[c].z);
        if (x > m || (x == m && qi < mi)) {
            m = x;
            mi = qi;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        const float xm = __shfl_xor(m, o);
        const int xi = __shfl_xor(mi, o);
        if (xm > m || (xm == m && xi < mi)) {
            m = xm;
            mi = xi;
        }
    }
    return mi;
}

// One workgroup per sequence: decisions, outputs and the draw.  The
// sequence's chunk partials (which carry the drafted tokens' logits) and
// uniforms are first staged in LDS by the whole workgroup (dynamic LDS: (2K+1) C float4 +
// K C float2), so that the decisions read no global memory.  Every sum or
// search over the chunks runs across a wave's lanes: the per-row totals in
// one pass spread over the waves, the chunk of the draw by a prefix scan.
constexpr int kMaxK = 64;
template <bool VEC>
__global__ __launch_bounds__(kVThreads) void verify_decide_kernel(
    int B, int K, int V, int C, int mode, float inv_t, const float* __restrict__ dl,
    const float* __restrict__ tl, const int32_t* __restrict__ tokens,
    const float* __restrict__ uni, const float4* __restrict__ part,
    const float2* __restrict__ ov, float* __restrict__ accept_prob, float* __restrict__ overlap,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ next_token) {
    extern __shared__ float4 dyn[];
    float4* sp = dyn;                                         // [(2K+1) C] partials
    float2* so = reinterpret_cast<float2*>(dyn + (2 * K + 1) * C);   // [K C] overlap, residual
    __shared__ float lse_q[kMaxK], lse_p[kMaxK + 1];
    __shared__ float xq_s[kMaxK], xp_s[kMaxK], u_s[kMaxK + 1];
    __shared__ float ovl_s[kMaxK], zres_s[kMaxK];
    __shared__ int tok_s[kMaxK], top_s[kMaxK + 1];
    __shared__ int j_s, chunk_s, resid_s;
    __shared__ float rem_s, lq_s, lp_s;
    __shared__ float wsum[kVThreads / 64];
    __shared__ int found_w[kVThreads / 64], last_w[kVThreads / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool target_only = mode == DSPARK_VERIFY_TARGET_ONLY;
    for (int i = tid; i < (2 * K + 1) * C; i += kVThreads) {
        const int k = i / C, c = i % C;
        const size_t r = k < K ? (size_t)b * K + k : (size_t)B * K + (size_t)b * (K + 1) + (k - K);
        sp[i] = part[r * C + c];
    }
    for (int i = tid; i < K * C; i += kVThreads) so[i] = ov[(size_t)b * K * C + i];
    if (tid < K) tok_s[tid] = tokens[(size_t)b * K + tid];
    if (tid <= K) u_s[tid] = uni[(size_t)b * (K + 1) + tid];
    __syncthreads();
    // the drafted tokens' logits (/T), recorded by the statistics pass in
    // the partial of the chunk that holds each
    if (tid < K) {
        const int x = tok_s[tid];
        if (x >= 0 && x < V) {
            xq_s[tid] = sp[(size_t)tid * C + x / kVChunk].w;
            xp_s[tid] = sp[(size_t)(K + tid) * C + x / kVChunk].w;
        }
    }
    // per-row totals, one wave per task: the log-sum-exp of each of the
    // 2K + 1 rows, the overlap and residual totals of each drafted row and
    // (target-only) each target row's first maximum
    const int n_lse = 2 * K + 1;
    const int n_tasks = n_lse + K + (target_only ? K + 1 : 0);
    for (int t = w; t < n_tasks; t += kVThreads / 64) {
        if (t < n_lse) {
            const float l = chunk_lse(sp + (size_t)t * C, C);
            if (lane == 0) {
                if (t < K) lse_q[t] = l;
                else lse_p[t - K] = l;
            }
        } else if (t < n_lse + K) {
            const int k = t - n_lse;
            float o = 0.f, z = 0.f;
            for (int c = lane; c < C; c += 64) {
                const float2 v = so[k * C + c];
                o += v.x;
                z += v.y;
            }
            o = vwave_sum(o);
            z = vwave_sum(z);
            if (lane == 0) {
                ovl_s[k] = o;
                zres_s[k] = z;
            }
        } else {
            const int k = t - n_lse - K;
            const int top = chunk_top(sp + (size_t)(K + k) * C, C);
            if (lane == 0) top_s[k] = top;
        }
    }
    __syncthreads();
    if (tid == 0) {
        int bad = 0, j = K;
        for (int k = 0; k < K; ++k) {
            const int x = tok_s[k];
            float a = 0.f;
            if (x < 0 || x >= V) bad = 1;
            else a = fminf(1.f, __expf((xp_s[k] - lse_p[k]) - (xq_s[k] - lse_q[k])));
            accept_prob[(size_t)b * K + k] = a;
            overlap[(size_t)b * K + k] = ovl_s[k];
            if (j == K && !bad) {
                const bool ok = target_only ? x == top_s[k] : u_s[k] < a;
                if (!ok) j = k;
            }
        }
        j_s = j;
        resid_s = -1;            // decided here: no draw
        if (bad) {
            n_accept[b] = -1;
            next_token[b] = -1;
        } else if (target_only) {
            n_accept[b] = j;
            next_token[b] = top_s[j];
        } else {
            // the draw: the residual of row j, or p_j when it is empty, or p_K
            n_accept[b] = j;
            resid_s = (j < K && zres_s[j] > 0.f) ? 1 : 0;
        }
    }
    __syncthreads();
    if (resid_s < 0) return;
    const bool residual = resid_s != 0;
    const int j = j_s;
    // wave 0: the chunk holding the draw, the first whose cumulative weight
    // exceeds u Z (inclusive prefix over the lanes, 64 chunks at a time)
    if (w == 0) {
        const float4* pr = sp + (size_t)(K + j) * C;       // target row j (j = K: p_K)
        const float lpj = lse_p[j];
        auto mass = [&](int c) {
            return residual ? so[j * C + c].y : pr[c].y * __expf(pr[c].x - lpj);
        };
        float Z;
        if (residual) {
            Z = zres_s[j];
        } else {
            float z = 0.f;
            for (int c = lane; c < C; c += 64) z += mass(c);
            Z = vwave_sum(z);
        }
        const float target = u_s[K] * Z;
        float carry = 0.f, cum = 0.f;
        int cs = -1, last_nz = -1;
        for (int c0 = 0; c0 < C; c0 += 64) {
            const int c = c0 + lane;
            const float mc = c < C ? mass(c) : 0.f;
            float incl = mc;
            for (int o = 1; o < 64; o <<= 1) {
                const float t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            const unsigned long long nz = __ballot(mc > 0.f);
            const unsigned long long hit = __ballot(mc > 0.f && carry + incl > target);
            if (nz) last_nz = c0 + 63 - __builtin_clzll(nz);
            if (hit) {
                const int first = __builtin_ctzll(hit);
                const float excl = __shfl(incl - mc, first);
                cs = c0 + first;
                cum = carry + excl;
                break;
            }
            carry += __shfl(incl, 63);
        }
        if (cs < 0 && last_nz >= 0) {    // rounding: the total fell short of u Z
            cs = last_nz;
            float s = 0.f;
            for (int c = lane; c < cs; c += 64) s += mass(c);
            cum = vwave_sum(s);
        }
        if (lane == 0) {
            chunk_s = cs;
            rem_s = target - cum;
            lq_s = residual ? lse_q[j] : 0.f;
            lp_s = lpj;
        }
    }
    __syncthreads();
    const int cs = chunk_s;
    if (cs < 0) return;
    // scan chunk cs: the first v whose cumulative weight exceeds rem
    const float* q = dl + ((size_t)b * K + (j < K ? j : 0)) * V;
    const float* p = tl + ((size_t)b * (K + 1) + j) * V;
    const float lq = lq_s, lp = lp_s, rem = rem_s;
    const int v0 = cs * kVChunk, v1 = min(V, v0 + kVChunk);
    // thread t owns the contiguous values [v0 + 32 t, v0 + 32 t + 32)
    float xp[kVPer], xq[kVPer];
    auto load_row = [&](const float* x, float* out) {
        if (VEC) {     // V % 4 == 0: a 4-value group is wholly inside or outside
#pragma unroll
            for (int i = 0; i < kVPer / 4; ++i) {
                const int v = v0 + kVPer * tid + 4 * i;
                float4 t4 = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                if (v < v1) t4 = *reinterpret_cast<const float4*>(x + v);
                out[4 * i] = t4.x * inv_t;
                out[4 * i + 1] = t4.y * inv_t;
                out[4 * i + 2] = t4.z * inv_t;
                out[4 * i + 3] = t4.w * inv_t;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kVPer; ++i) {
                const int v = v0 + kVPer * tid + i;
                out[i] = v < v1 ? x[v] * inv_t : -INFINITY;
            }
        }
    };
    load_row(p, xp);
    if (residual) load_row(q, xq);
    float wv[kVPer];
    float tsum = 0.f;
    int tlast = -1;
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
        const int v = v0 + kVPer * tid + i;
        float x = 0.f;
        if (v < v1) {
            const float pv = __expf(xp[i] - lp);
            x = residual ? fmaxf(pv - __expf(xq[i] - lq), 0.f) : pv;
        }
        wv[i] = x;
        tsum += x;
        if (x > 0.f) tlast = v;
    }
    // exclusive prefix of the per-thread sums
    float incl = tsum;
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    float before = incl - tsum;
    for (int i = 0; i < w; ++i) before += wsum[i];
    int hit = INT_MAX;
    float cum = before;
#pragma unroll
    for (int i = 0; i < kVPer; ++i) {
        cum += wv[i];
        if (hit == INT_MAX && wv[i] > 0.f && cum > rem) hit = v0 + kVPer * tid + i;
    }
    // threads own ascending value ranges: the first hit is the lowest
    // hitting lane's, the last positive value the highest positive lane's
    // (per wave by ballot, then over the waves; same-address LDS atomics
    // from every lane serialise)
    const unsigned long long hb = __ballot(hit != INT_MAX);
    const unsigned long long lb = __ballot(tlast >= 0);
    const int hit_w = __builtin_amdgcn_readlane(hit, hb ? __builtin_ctzll(hb) : 0);
    const int last_v = __builtin_amdgcn_readlane(tlast, lb ? 63 - __builtin_clzll(lb) : 0);
    if (lane == 0) {
        found_w[w] = hb ? hit_w : INT_MAX;
        last_w[w] = lb ? last_v : -1;
    }
    __syncthreads();
    if (tid == 0) {
        int found = INT_MAX, last = -1;
        for (int i = 0; i < kVThreads / 64; ++i) {
            found = min(found, found_w[i]);
            last = max(last, last_w[i]);
        }
        next_token[b] = found != INT_MAX ? found : last;
    }
}

size_t decide_lds_bytes(int K, int C) { return (size_t)(2 * K + 1) * C * 16 + (size_t)K * C * 8; }
constexpr size_t kMaxDecideLds = 64 * 1024;

struct VerifyLayout {
    size_t part = 0, ov = 0, total = 0;
    int chunks = 0;
};

const char* check_verify(const dspark_verify_desc* d) {
    if (!d) return "desc is NULL";
    if (d->B < 0 || d->K < 1 || d->K > kMaxK || d->vocab < 1)
        return "need B >= 0, 1 <= K <= 64, vocab >= 1";
    if (d->mode != DSPARK_VERIFY_REJECTION && d->mode != DSPARK_VERIFY_TARGET_ONLY)
        return "mode must be DSPARK_VERIFY_REJECTION or DSPARK_VERIFY_TARGET_ONLY";
    if (!(d->temperature > 0.0) || !std::isfinite(d->temperature)) return "temperature must be > 0";
    const long long C = (d->vocab + kVChunk - 1) / kVChunk;
    if ((long long)d->B * (2 * d->K + 1) * C > INT_MAX) return "B * (2K + 1) * chunks too large";
    if (decide_lds_bytes(d->K, (int)C) > kMaxDecideLds)
        return "K x vocabulary chunks too large for the decision kernel's LDS ((3K+1) x ceil(V/8192) x 8 B <= 64 KB)";
    return nullptr;
}

VerifyLayout verify_layout(const dspark_verify_desc& d) {
    VerifyLayout w;
    w.chunks = (d.vocab + kVChunk - 1) / kVChunk;
    const size_t rows = (size_t)d.B * (2 * d.K + 1);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    w.part = take(rows * w.chunks * 16);
    w.ov = take((size_t)d.B * d.K * w.chunks * 8);
    w.total = off;
    return w;
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" {

dspark_status dspark_cache_append(const dspark_decode_desc* desc, const int32_t* pos0,
                                  const int32_t* n_new, int32_t max_new, const void* new_ckv,
                                  const void* new_kr, void* cache_ckv, void* cache_kr,
                                  void* stream) {
    set_last_error("");
    if (const char* why = check_decode(desc)) return dfail(DSPARK_EINVAL, why);
    const dspark_attn_desc& a = desc->attn;
    if (a.B < 0 || a.d_latent < 1 || a.d_rope < 0 || max_new < 0)
        return dfail(DSPARK_EINVAL, "need B >= 0, d_latent >= 1, d_rope >= 0, max_new >= 0");
    if (a.dtype != DSPARK_BF16 && a.dtype != DSPARK_F32) return dfail(DSPARK_EINVAL, "bad dtype");
    if ((long long)a.B * max_new == 0) return DSPARK_OK;
    const bool need_kr = a.d_rope > 0;
    if (!pos0 || !n_new || !new_ckv || !cache_ckv || (need_kr && (!new_kr || !cache_kr)))
        return dfail(DSPARK_EINVAL, "a pointer is NULL");
    if (!al16(new_ckv) || !al16(cache_ckv) || (need_kr && (!al16(new_kr) || !al16(cache_kr))))
        return dfail(DSPARK_EINVAL, "latent pointers must be 16-byte aligned");
    const bool bf = a.dtype == DSPARK_BF16;
    const size_t e = bf ? 2 : 4;
    const bool vec = ((size_t)a.d_latent * e) % 16 == 0 && ((size_t)a.d_rope * e) % 16 == 0;
    const long long waves = (long long)a.B * max_new;
    if ((waves + 3) / 4 > INT_MAX) return dfail(DSPARK_EINVAL, "B * max_new too large");
    const dim3 grid((unsigned)((waves + 3) / 4));
    hipStream_t s = static_cast<hipStream_t>(stream);
#define DSPARK_APPEND(T, VV)                                                                     \
    hipLaunchKernelGGL((cache_append_kernel<T, VV>), grid, dim3(256), 0, s, a.B,                 \
                       desc->cache_slots, a.d_latent, a.d_rope, max_new, pos0, n_new,            \
                       (const T*)new_ckv, (const T*)new_kr, (T*)cache_ckv, (T*)cache_kr)
    if (bf) {
        if (vec) DSPARK_APPEND(bf16, true); else DSPARK_APPEND(bf16, false);
    } else {
        if (vec) DSPARK_APPEND(float, true); else DSPARK_APPEND(float, false);
    }
#undef DSPARK_APPEND
    const hipError_t he = hipGetLastError();
    if (he != hipSuccess) {
        snprintf(t_msg, sizeof(t_msg), "cache append launch: %s", hipGetErrorString(he));
        return dfail(DSPARK_EHIP, t_msg);
    }
    return DSPARK_OK;
}

size_t dspark_decode_workspace_size(const dspark_decode_desc* desc) {
    if (const char* why = check_decode(desc)) {
        set_last_error(why);
        return 0;
    }
    DecodeLayout L;
    if (!decode_layout(*desc, &L)) return 0;       // the attention's message stands
    return L.total;
}

dspark_status dspark_decode_attn(const dspark_decode_desc* desc, const void* q_nope,
                                 const void* q_rope, const void* cache_ckv, const void* cache_kr,
                                 const void* ckv_blk, const void* kr_blk, const void* w_uk,
                                 const void* w_uv, const int32_t* anchors, const uint8_t* active,
                                 void* out, void* workspace, size_t ws_bytes, void* stream) {
    set_last_error("");
    if (const char* why = check_decode(desc)) return dfail(DSPARK_EINVAL, why);
    DecodeLayout L;
    if (!decode_layout(*desc, &L)) return DSPARK_EINVAL;     // dspark_last_error() says why
    const dspark_attn_desc& a = desc->attn;
    if (a.B == 0) return DSPARK_OK;
    const bool need_kr = a.d_rope > 0;
    if (!cache_ckv || !anchors || !active || (need_kr && !cache_kr))
        return dfail(DSPARK_EINVAL, "cache_ckv, cache_kr, anchors or active is NULL");
    if (!al16(cache_ckv) || (need_kr && !al16(cache_kr)))
        return dfail(DSPARK_EINVAL, "cache pointers must be 16-byte aligned");
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return dfail(DSPARK_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    if (ws_bytes < L.total) {
        snprintf(t_msg, sizeof(t_msg), "workspace too small; bytes needed (%zu)", L.total);
        return dfail(DSPARK_EWORKSPACE, t_msg);
    }
    char* base = static_cast<char*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = a.dtype == DSPARK_BF16;
    const size_t e = bf ? 2 : 4;
    const bool vec = ((size_t)a.d_latent * e) % 16 == 0 && ((size_t)a.d_rope * e) % 16 == 0;
    const int rows = L.sub.S;
    const long long waves = (long long)a.B * rows;
    const dim3 grid((unsigned)((waves + 3) / 4));
    int32_t* anchors2 = reinterpret_cast<int32_t*>(base + L.anchors2);
    uint8_t* keep2 = reinterpret_cast<uint8_t*>(base + L.keep2);
    void* win_ckv = base + L.win_ckv;
    void* win_kr = base + L.win_kr;
#define DSPARK_GATHER(T, VV)                                                                   \
    hipLaunchKernelGGL((decode_gather_kernel<T, VV>), grid, dim3(256), 0, s, a.B,              \
                       desc->cache_slots, a.window, a.d_latent, a.d_rope, rows, anchors, active, \
                       (const T*)cache_ckv, (const T*)cache_kr, (T*)win_ckv, (T*)win_kr,       \
                       anchors2, keep2)
    if (bf) {
        if (vec) DSPARK_GATHER(bf16, true); else DSPARK_GATHER(bf16, false);
    } else {
        if (vec) DSPARK_GATHER(float, true); else DSPARK_GATHER(float, false);
    }
#undef DSPARK_GATHER
    const hipError_t he = hipGetLastError();
    if (he != hipSuccess) {
        snprintf(t_msg, sizeof(t_msg), "decode gather launch: %s", hipGetErrorString(he));
        return dfail(DSPARK_EHIP, t_msg);
    }
    return dspark_attn_fwd(&L.sub, q_nope, q_rope, win_ckv, need_kr ? win_kr : nullptr, ckv_blk,
                           kr_blk, w_uk, w_uv, anchors2, keep2, out, base + L.attn, L.attn_bytes,
                           stream);
}

size_t dspark_verify_workspace_size(const dspark_verify_desc* desc) {
    if (const char* why = check_verify(desc)) {
        set_last_error(why);
        return 0;
    }
    return verify_layout(*desc).total;
}

dspark_status dspark_spec_verify(const dspark_verify_desc* desc, const float* draft_logits,
                                 const float* target_logits, const int32_t* draft_tokens,
                                 const float* uniforms, float* accept_prob, float* overlap,
                                 int32_t* n_accept, int32_t* next_token, void* workspace,
                                 size_t ws_bytes, void* stream) {
    set_last_error("");
    if (const char* why = check_verify(desc)) return dfail(DSPARK_EINVAL, why);
    const dspark_verify_desc& d = *desc;
    if (d.B == 0) return DSPARK_OK;
    const void* ptrs[] = {draft_logits, target_logits, draft_tokens, uniforms, accept_prob,
                          overlap, n_accept, next_token};
    for (const void* p : ptrs) {
        if (!p) return dfail(DSPARK_EINVAL, "a pointer is NULL");
        if (reinterpret_cast<uintptr_t>(p) & 3u) return dfail(DSPARK_EINVAL, "pointers must be 4-byte aligned");
    }
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return dfail(DSPARK_EWORKSPACE, "workspace must be non-NULL and 256-byte aligned");
    const VerifyLayout L = verify_layout(d);
    if (ws_bytes < L.total) {
        snprintf(t_msg, sizeof(t_msg), "workspace too small; bytes needed (%zu)", L.total);
        return dfail(DSPARK_EWORKSPACE, t_msg);
    }
    char* base = static_cast<char*>(workspace);
    float4* part = reinterpret_cast<float4*>(base + L.part);
    float2* ov = reinterpret_cast<float2*>(base + L.ov);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int C = L.chunks;
    const float inv_t = (float)(1.0 / d.temperature);
    const int rows = d.B * (2 * d.K + 1);
    const bool vec = d.vocab % 4 == 0 && al16(draft_logits) && al16(target_logits);
    if (vec) {
        hipLaunchKernelGGL(verify_stats_kernel<true>, dim3(rows * C), dim3(kVThreads), 0, s, d.B,
                           d.K, d.vocab, C, inv_t, draft_logits, target_logits, draft_tokens, part);
        hipLaunchKernelGGL(verify_overlap_kernel<true>, dim3(d.B * d.K * C), dim3(kVThreads), 0, s,
                           d.B, d.K, d.vocab, C, inv_t, draft_logits, target_logits, part, ov);
    } else {
        hipLaunchKernelGGL(verify_stats_kernel<false>, dim3(rows * C), dim3(kVThreads), 0, s, d.B,
                           d.K, d.vocab, C, inv_t, draft_logits, target_logits, draft_tokens, part);
        hipLaunchKernelGGL(verify_overlap_kernel<false>, dim3(d.B * d.K * C), dim3(kVThreads), 0,
                           s, d.B, d.K, d.vocab, C, inv_t, draft_logits, target_logits, part, ov);
    }
    auto* decide = vec ? verify_decide_kernel<true> : verify_decide_kernel<false>;
    hipLaunchKernelGGL(decide, dim3(d.B), dim3(kVThreads), decide_lds_bytes(d.K, C), s, d.B, d.K,
                       d.vocab, C, d.mode, inv_t, draft_logits, target_logits, draft_tokens,
                       uniforms, part, ov, accept_prob, overlap, n_accept, next_token);
    const hipError_t he = hipGetLastError();
    if (he != hipSuccess) {
        snprintf(t_msg, sizeof(t_msg), "verify launch: %s", hipGetErrorString(he));
        return dfail(DSPARK_EHIP, t_msg);
    }
    return DSPARK_OK;
}

}  // extern "C"
