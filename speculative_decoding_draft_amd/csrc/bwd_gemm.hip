// Backward of the masked latent attention, MFMA path: the dense products
// around the attention kernel, as tiled bf16 MFMA GEMMs with fp32
// accumulation (W_UV^T dout runs on the forward's absorb kernel).
//
//   dq^C   = W_UK[h] dq_abs              per head, over the kept query rows
//   dW_UV[h] = sum_rows dout (o_lat)^T   per head, reduction over every row
//   dW_UK[h] = sum_rows q^C (dq_abs)^T   per head
//   dc_k  = sum_rows P d_olat + dS' q_abs, d(R k^R)_k = sum_rows dS' (R q^R)
//                                         per block, over its 5 x 64 rows
// (the chain rule on the design page's attention in absorbed form: the
// relations are listed at the top of bwd_misc.hip).
//
// One workgroup computes a BM x BN tile of C = A B (A: M x K, B: K x N) with
// 4 waves.  Operands go through LDS 32 k at a time, double buffered (one
// barrier per step); the global loads of step s + 1 are issued before the
// MFMAs of step s.  An operand is either K-contiguous in memory (its rows
// are M or N indices; read with 16-byte LDS loads) or M/N-contiguous (its
// rows are k indices; read with the gfx950 transposing LDS load).  Every
// fragment carries its 8 k values in the order the transposing load
// produces: inside each 32-group, k-slot 8g + e holds k = 16(e/4) + 4g + e%4
// for k-group g.  That is also the order the latent rows are stored in
// ("permuted"), so a K-contiguous latent operand is read with plain 16-byte
// loads and a K-contiguous natural-order operand with two 8-byte loads.
//
// The M side is always the output's contiguous dimension: lane l of a wave
// receives C[4(l/16) + i][l%16], i = 0..3, i.e. 4 consecutive output elements.
#include "bwd.hpp"

namespace dspark {

namespace {

// dim of position p (0..31) of a permuted 32-group, and the inverse
__device__ inline int perm_dim(int p) { return 16 * ((p & 7) >> 2) + 4 * (p >> 3) + (p & 3); }
__device__ inline int perm_pos(int d) { return 8 * ((d & 15) >> 2) + 4 * (d >> 4) + (d & 3); }

// the first of 4 consecutive dims held at permuted positions pos .. pos+3
__device__ inline int dim_of_pos4(int pos) { return (pos & ~31) + perm_dim(pos & 31); }
__device__ inline int pos_of_dim4(int dim) { return (dim & ~31) + perm_pos(dim & 31); }

template <int BM_, int BN_, int WM_, int WN_, bool A_TR_, bool A_PERM_, bool B_TR_, bool B_PERM_,
          int PF_ = 1>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int PF = PF_;                      // k-steps of global loads in flight
    static constexpr bool A_TR = A_TR_, A_PERM = A_PERM_, B_TR = B_TR_, B_PERM = B_PERM_;
    static_assert(WM * WN == 4, "4 waves");
    static constexpr int MT = BM / WM / 16, NT = BN / WN / 16;
    static_assert(MT * WM * 16 == BM && NT * WN * 16 == BN, "16-row tiles");
    static constexpr int A_LD = A_TR ? BM + 8 : 40;     // LDS row stride (bf16)
    static constexpr int B_LD = B_TR ? BN + 8 : 40;
    static constexpr int A_SZ = A_TR ? 32 * A_LD : BM * A_LD;
    static constexpr int B_SZ = B_TR ? 32 * B_LD : BN * B_LD;
    static constexpr int A_CH = BM * 4, B_CH = BN * 4;  // 16-byte chunks per 32-k tile
    static constexpr int A_PT = (A_CH + 255) / 256, B_PT = (B_CH + 255) / 256;
    static constexpr int STAGE = A_SZ + B_SZ;
    static constexpr int LDS_ELEMS = 2 * STAGE;
};

template <class C>
__device__ inline void gemm_zero(f32x4 (&acc)[C::MT][C::NT]) {
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc += the k-steps [s0, s1) of the tile product.
// K-contiguous operand: row(r) is the start of row r (r < BM or BN), or
// nullptr (zeros).  Transposed operand: row(k) is the element (k, tile
// column 0) of k-row k, or nullptr (zeros).  The global loads of C::PF
// k-steps are in flight in a ring of registers; vmcnt retires in order, so
// row() must not itself load from global memory (it may read LDS).
template <class C, class AF, class BF>
__device__ inline void gemm_tile(const AF& arow, const BF& brow, int s0, int s1, bf16* lds,
                                 f32x4 (&acc)[C::MT][C::NT]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const bf16x8 zero8 = {};

    const bf16* apr[C::A_PT];
    const bf16* bpr[C::B_PT];
    if constexpr (!C::A_TR) {
#pragma unroll
        for (int i = 0; i < C::A_PT; ++i) {
            const int c = tid + 256 * i;
            apr[i] = (c < C::A_CH) ? arow(c >> 2) : nullptr;
        }
    }
    if constexpr (!C::B_TR) {
#pragma unroll
        for (int i = 0; i < C::B_PT; ++i) {
            const int c = tid + 256 * i;
            bpr[i] = (c < C::B_CH) ? brow(c >> 2) : nullptr;
        }
    }
    bf16x8 ra[C::PF][C::A_PT], rb[C::PF][C::B_PT];
    auto load = [&](int s, bf16x8 (&xa)[C::A_PT], bf16x8 (&xb)[C::B_PT]) {
#pragma unroll
        for (int i = 0; i < C::A_PT; ++i) {
            const int c = tid + 256 * i;
            const bf16* p = nullptr;
            if (c < C::A_CH) {
                if constexpr (C::A_TR) {
                    constexpr int per = C::BM / 8;
                    p = arow(32 * s + c / per);
                    if (p) p += 8 * (c % per);
                } else {
                    p = apr[i];
                    if (p) p += 32 * s + 8 * (c & 3);
                }
            }
            xa[i] = p ? gld16(p) : zero8;
        }
#pragma unroll
        for (int i = 0; i < C::B_PT; ++i) {
            const int c = tid + 256 * i;
            const bf16* p = nullptr;
            if (c < C::B_CH) {
                if constexpr (C::B_TR) {
                    constexpr int per = C::BN / 8;
                    p = brow(32 * s + c / per);
                    if (p) p += 8 * (c % per);
                } else {
                    p = bpr[i];
                    if (p) p += 32 * s + 8 * (c & 3);
                }
            }
            xb[i] = p ? gld16(p) : zero8;
        }
    };
    auto store = [&](bf16* st, const bf16x8 (&xa)[C::A_PT], const bf16x8 (&xb)[C::B_PT]) {
#pragma unroll
        for (int i = 0; i < C::A_PT; ++i) {
            const int c = tid + 256 * i;
            if (c < C::A_CH) {
                constexpr int per = C::BM / 8;
                const int off = C::A_TR ? (c / per) * C::A_LD + 8 * (c % per)
                                        : (c >> 2) * C::A_LD + 8 * (c & 3);
                st16(st + off, xa[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < C::B_PT; ++i) {
            const int c = tid + 256 * i;
            if (c < C::B_CH) {
                constexpr int per = C::BN / 8;
                const int off = C::B_TR ? (c / per) * C::B_LD + 8 * (c % per)
                                        : (c >> 2) * C::B_LD + 8 * (c & 3);
                st16(st + C::A_SZ + off, xb[i]);
            }
        }
    };
    auto frag = [&](const bf16* base, int ld, bool tr, bool perm, int r0) -> bf16x8 {
        if (tr) {
            const int col = r0 + 4 * (l16 & 3);
            const int rr = 4 * g + (l16 >> 2);
            return cat(lds_read_tr(base + rr * ld + col), lds_read_tr(base + (rr + 16) * ld + col));
        }
        const bf16* row = base + (r0 + l16) * ld;
        return perm ? ld16(row + 8 * g) : cat(ld8(row + 4 * g), ld8(row + 16 + 4 * g));
    };
    if (s0 >= s1) return;
#pragma unroll
    for (int u = 0; u < C::PF; ++u)
        if (s0 + u < s1) load(s0 + u, ra[u], rb[u]);
    for (int s = s0; s < s1; s += C::PF) {
#pragma unroll
        for (int u = 0; u < C::PF; ++u) {
            const int ss = s + u;
            if (ss < s1) {
                bf16* st = lds + ((ss - s0) & 1) * C::STAGE;
                store(st, ra[u], rb[u]);
                __syncthreads();
                if (ss + C::PF < s1) load(ss + C::PF, ra[u], rb[u]);
                bf16x8 af[C::MT], bfr[C::NT];
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
                    af[i] = frag(st, C::A_LD, C::A_TR, C::A_PERM, wm * (C::BM / C::WM) + 16 * i);
#pragma unroll
                for (int j = 0; j < C::NT; ++j)
                    bfr[j] = frag(st + C::A_SZ, C::B_LD, C::B_TR, C::B_PERM,
                                  wn * (C::BN / C::WN) + 16 * j);
#pragma unroll
                for (int i = 0; i < C::MT; ++i)
#pragma unroll
                    for (int j = 0; j < C::NT; ++j)
                        acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
            }
        }
    }
}

// input row (b * 5N + 5n + t) of latent row R = 5 * slot + t
__device__ inline size_t input_row(const int4* srec, int R, int N, int L5) {
    const int blk = srec[R / kBlock].w;
    return (size_t)(blk / N) * L5 + (size_t)kBlock * (blk % N) + R % kBlock;
}

__device__ inline bf16x4 to_bf16x4(f32x4 v) {
    return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// ---- dq^C[R][h] = W_UK[h] dq_abs[R][h]: M = d_c, N = rows, K = D.
// A = W_UK[h] rows (natural), B = dq_abs rows (permuted).
using CfgDqn = Cfg<192, 128, 2, 2, false, false, false, true, 1>;
__global__ __launch_bounds__(256) void dqnope_kernel(const bf16* __restrict__ dqabs,
                                                     const bf16* __restrict__ w_uk,
                                                     const int4* __restrict__ srec,
                                                     const int32_t* __restrict__ status,
                                                     bf16* __restrict__ dq_nope, int N, int L5) {
    __shared__ __attribute__((aligned(16))) bf16 lds[CfgDqn::LDS_ELEMS];
    const int rows = kBlock * status[kStKeptCount];
    const int m0 = blockIdx.x * CfgDqn::BM, n0 = blockIdx.y * CfgDqn::BN, h = blockIdx.z;
    if (n0 >= rows) return;
    const bf16* wh = w_uk + ((size_t)h * kDc + m0) * kD;
    auto arow = [&](int r) -> const bf16* { return wh + (size_t)r * kD; };
    auto brow = [&](int r) -> const bf16* {
        const int R = n0 + r;
        return R < rows ? dqabs + ((size_t)R * kH + h) * kD : nullptr;
    };
    f32x4 acc[CfgDqn::MT][CfgDqn::NT];
    gemm_zero<CfgDqn>(acc);
    gemm_tile<CfgDqn>(arow, brow, 0, kD / 32, lds, acc);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const int wm = wave / CfgDqn::WN, wn = wave % CfgDqn::WN;
#pragma unroll
    for (int j = 0; j < CfgDqn::NT; ++j) {
        const int R = n0 + wn * (CfgDqn::BN / CfgDqn::WN) + 16 * j + l16;
        if (R >= rows) continue;
        bf16* dst = dq_nope + (input_row(srec, R, N, L5) * kH + h) * kDc;
#pragma unroll
        for (int i = 0; i < CfgDqn::MT; ++i)
            gst8(dst + m0 + wm * (CfgDqn::BM / CfgDqn::WM) + 16 * i + 4 * g,
                 to_bf16x4(acc[i][j]));
    }
}

// ---- weight gradients, a reduction over every kept row: M = D (latent
// positions, permuted), N = d_v or d_c, K = rows.  Both operands transposed.
// 128 x 64 tiles (16 of dW_UV and 12 of dW_UK per head; small tiles keep
// four workgroups resident per compute unit) are consecutive per head in the
// XCD-remapped order, so a head's tiles share the rows they stream through
// one L2.
using CfgDwuv = Cfg<128, 64, 2, 2, true, false, true, false, 2>;
using CfgDwuk = Cfg<128, 64, 2, 2, true, false, true, false, 2>;
constexpr int kSlotChunk = 2048;     // slots whose input rows one LDS table holds

template <class C, int NOUT>
__device__ inline void dw_tile(const bf16* __restrict__ lat, const bf16* __restrict__ rowsrc,
                               const int4* __restrict__ srec, int n_slots, int h, int m0, int n0,
                               int N, int L5, bf16* __restrict__ dw, bf16* lds, int* rbase) {
    f32x4 acc[C::MT][C::NT];
    gemm_zero<C>(acc);
    for (int c0 = 0; c0 < n_slots; c0 += kSlotChunk) {
        const int nsl = min(kSlotChunk, n_slots - c0);
        __syncthreads();                 // the previous chunk is done with the table and LDS
        for (int i = threadIdx.x; i < nsl; i += blockDim.x) {
            const int blk = srec[c0 + i].w;
            rbase[i] = (blk / N) * L5 + kBlock * (blk % N);
        }
        __syncthreads();
        const int k0 = kBlock * c0, k1 = kBlock * (c0 + nsl);
        auto arow = [&](int k) -> const bf16* {
            return (k >= k0 && k < k1) ? lat + ((size_t)k * kH + h) * kD + m0 : nullptr;
        };
        auto brow = [&](int k) -> const bf16* {
            if (k < k0 || k >= k1) return nullptr;
            const int sl = k / kBlock;
            const size_t row = (size_t)rbase[sl - c0] + (k - kBlock * sl);
            return rowsrc + (row * kH + h) * NOUT + n0;
        };
        // chunks start on a 32-row boundary (5 * 4096 = 640 * 32)
        gemm_tile<C>(arow, brow, k0 / 32, (k1 + 31) / 32, lds, acc);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const int wm = wave / C::WN, wn = wave % C::WN;
#pragma unroll
    for (int j = 0; j < C::NT; ++j) {
        const int o = n0 + wn * (C::BN / C::WN) + 16 * j + l16;
        bf16* dst = dw + ((size_t)h * NOUT + o) * kD;
#pragma unroll
        for (int i = 0; i < C::MT; ++i) {
            const int pos = m0 + wm * (C::BM / C::WM) + 16 * i + 4 * g;
            gst8(dst + dim_of_pos4(pos), to_bf16x4(acc[i][j]));
        }
    }
}

__global__ __launch_bounds__(256) void dw_kernel(const bf16* __restrict__ olat,
                                                 const bf16* __restrict__ dout,
                                                 const bf16* __restrict__ dqabs,
                                                 const bf16* __restrict__ q_nope,
                                                 const int4* __restrict__ srec,
                                                 const int32_t* __restrict__ status,
                                                 bf16* __restrict__ dw_uv, bf16* __restrict__ dw_uk,
                                                 int N, int L5) {
    constexpr int kUvTiles = (kD / CfgDwuv::BM) * (kDv / CfgDwuv::BN);
    constexpr int kUkTiles = (kD / CfgDwuk::BM) * (kDc / CfgDwuk::BN);
    static_assert(kDv % CfgDwuv::BN == 0 && kDc % CfgDwuk::BN == 0, "whole tiles");
    constexpr int kLds = CfgDwuv::LDS_ELEMS > CfgDwuk::LDS_ELEMS ? CfgDwuv::LDS_ELEMS
                                                                  : CfgDwuk::LDS_ELEMS;
    __shared__ __attribute__((aligned(16))) bf16 lds[kLds];
    __shared__ int rbase[kSlotChunk];
    const int n_slots = status[kStKeptCount];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid / (kUvTiles + kUkTiles), t = lid % (kUvTiles + kUkTiles);
    if (t < kUvTiles) {
        const int m0 = (t / (kDv / CfgDwuv::BN)) * CfgDwuv::BM;
        const int n0 = (t % (kDv / CfgDwuv::BN)) * CfgDwuv::BN;
        dw_tile<CfgDwuv, kDv>(olat, dout, srec, n_slots, h, m0, n0, N, L5, dw_uv, lds, rbase);
    } else {
        const int m0 = ((t - kUvTiles) / (kDc / CfgDwuk::BN)) * CfgDwuk::BM;
        const int n0 = ((t - kUvTiles) % (kDc / CfgDwuk::BN)) * CfgDwuk::BN;
        dw_tile<CfgDwuk, kDc>(dqabs, q_nope, srec, n_slots, h, m0, n0, N, L5, dw_uk, lds, rbase);
    }
}

// ---- per block: dc_k (M = D, permuted positions) and d(R k^R)_k (M = d_r,
// natural) for its key slots (N = 144), K = its 320 rows taken twice
// (P with d_olat, then dS' with q_abs; the k^R part only dS' with R q^R).
// When every sample's kept anchors ascend, each block writes its partial
// rows and the final pass sums, per context row, the contiguous range of
// blocks whose windows hold it; otherwise the sums go to the fp32
// accumulator with atomics.  A block's own 5 keys are its alone.
using CfgDkv = Cfg<64, kKeySlots, 4, 1, true, false, true, false>;
__global__ __launch_bounds__(256) void dkv_kernel(const bf16* __restrict__ dolat,
                                                  const bf16* __restrict__ qabs,
                                                  const bf16* __restrict__ qrot,
                                                  const bf16* __restrict__ pmat,
                                                  const bf16* __restrict__ dsmat,
                                                  const int4* __restrict__ srec,
                                                  const int32_t* __restrict__ status,
                                                  float* __restrict__ part,
                                                  float* __restrict__ acc, int S, int N, int L5) {
    __shared__ __attribute__((aligned(16))) bf16 lds[CfgDkv::LDS_ELEMS];
    constexpr int kTiles = (kD + kDr) / CfgDkv::BM;    // 9
    constexpr int kRows = kBlock * kH;                 // 320
    const int n_live = status[kStKeptCount];
    const int lid = xcd_balance(blockIdx.x, n_live * kTiles);
    if (lid < 0) return;
    const int slot = lid / kTiles, mt = lid % kTiles;
    const int m0 = mt * CfgDkv::BM;
    const size_t lat0 = (size_t)kBlock * slot * kH;    // first latent row (t = 0, h = 0)
    const bf16* pm = pmat + (size_t)slot * kRows * kKeySlots;
    const bf16* ds = dsmat + (size_t)slot * kRows * kKeySlots;
    const bool rope_tile = m0 >= kD;
    auto arow = [&](int k) -> const bf16* {
        if (rope_tile) return qrot + (lat0 + (k - kRows)) * kDr;
        return (k < kRows) ? dolat + (lat0 + k) * kD + m0 : qabs + (lat0 + k - kRows) * kD + m0;
    };
    auto brow = [&](int k) -> const bf16* {
        return (k < kRows) ? pm + (size_t)k * kKeySlots : ds + (size_t)(k - kRows) * kKeySlots;
    };
    f32x4 a[CfgDkv::MT][CfgDkv::NT];
    gemm_zero<CfgDkv>(a);
    gemm_tile<CfgDkv>(arow, brow, rope_tile ? kRows / 32 : 0, 2 * kRows / 32, lds, a);

    const int4 rec = srec[slot];
    const int blk = rec.w, b = blk / N, n = blk % N;
    const int ctx_lo = rec.x, ctx_len = rec.y, nkeys = ctx_len + kBlock;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const size_t arow0 = (size_t)b * (S + L5);
    const int pos = wave * 16 + 4 * g;                  // CfgDkv: WM = 4, MT = 1
    const int dim = rope_tile ? kD + pos : dim_of_pos4(m0 + pos);
    if (status[kStUnsorted] == 0) {
        // the block's own partial rows; the final pass sums the blocks whose
        // windows cover each context row
        float* base = part + (size_t)slot * kMaxKeys * (kD + kDr) + dim;
#pragma unroll
        for (int j = 0; j < CfgDkv::NT; ++j) {
            const int key = 16 * j + l16;
            if (key < nkeys) *reinterpret_cast<f32x4*>(base + (size_t)key * (kD + kDr)) = a[0][j];
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < CfgDkv::NT; ++j) {
        const int key = 16 * j + l16;
        if (key >= nkeys) continue;
        const size_t r = arow0 + ((key < ctx_len) ? (size_t)(ctx_lo + key)
                                                  : (size_t)S + kBlock * n + (key - ctx_len));
        float* dst = acc + r * (kD + kDr) + dim;
#pragma unroll
        for (int i = 0; i < 4; ++i) atomicAdd(dst + i, a[0][j][i]);
    }
}

}  // namespace

hipError_t launch_bwd_dqnope(const Problem& p, const Inputs& in, const BwdGrads& g,
                             const BwdWork& w, hipStream_t s) {
    const int rows = kBlock * p.B * p.N;
    static_assert(kDc % CfgDqn::BM == 0, "whole tiles");
    const dim3 grid(kDc / CfgDqn::BM, (rows + CfgDqn::BN - 1) / CfgDqn::BN, kH);
    hipLaunchKernelGGL(dqnope_kernel, grid, dim3(256), 0, s, w.dqabs, (const bf16*)in.w_uk,
                       w.fwd.srec, w.fwd.status, (bf16*)g.dq_nope, p.N, p.L5);
    return hipGetLastError();
}

hipError_t launch_bwd_dw(const Problem& p, const Inputs& in, const BwdGrads& g,
                         const BwdWork& w, hipStream_t s) {
    constexpr int kPerHead = (kD / CfgDwuv::BM) * (kDv / CfgDwuv::BN) +
                             (kD / CfgDwuk::BM) * (kDc / CfgDwuk::BN);
    hipLaunchKernelGGL(dw_kernel, dim3(kH * kPerHead), dim3(256), 0, s, w.fwd.olat,
                       (const bf16*)g.dout, w.dqabs, (const bf16*)in.q_nope, w.fwd.srec,
                       w.fwd.status, (bf16*)g.dw_uv, (bf16*)g.dw_uk, p.N, p.L5);
    return hipGetLastError();
}

hipError_t launch_bwd_dkv(const Problem& p, const BwdWork& w, hipStream_t s) {
    constexpr int kTiles = (kD + kDr) / CfgDkv::BM;
    int grid = p.B * p.N * kTiles;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL(dkv_kernel, dim3(grid), dim3(256), 0, s, w.dolat, w.fwd.qabs, w.qrot,
                       w.pmat, w.dsmat, w.fwd.srec, w.fwd.status, w.part, w.acc, p.S, p.N, p.L5);
    return hipGetLastError();
}

}  // namespace dspark
