// Backward of the masked latent attention, MFMA path: the dense products
// around the attention kernel, as tiled bf16 MFMA GEMMs with fp32
// accumulation (W_UV^T dout runs on the forward's absorb kernel, dq^C =
// W_UK[h] dq_abs on its W_UV kernel).
//
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

__device__ inline bf16x4 to_bf16x4(f32x4 v) {
    return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
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

// ---- weight gradients with LDS DMA: the same reduction in 256-position x
// (256 or 192)-output tiles (every output column of the head), 4 per head
// (dW_UV and dW_UK, two position halves each), one 8-wave workgroup per
// compute unit.  Each head's o_lat / dq_abs columns are read by one
// workgroup only; the narrower input rows (dout, q^C) by two.  The 2 x 4
// waves each own a 128 x 64 (or 128 x 48) part, which halves the LDS bytes
// read per MFMA against 64 x 32 parts; LDS bandwidth, not HBM, bounded the
// smaller tiles.
// Operands reach LDS by buffer DMA (no register staging, no LDS store
// instructions) in a ring of three 32-row stages, two stages in flight while
// the third is consumed.  Each stage row holds its 16-byte chunks XOR-
// swizzled by row ((2 row) mod 16), so that the transposing reads of eight
// consecutive rows hit distinct banks.  Rows past the last kept row read
// zero: the lat operand through the bound of its buffer resource, the
// gathered operand through an offset past it.
constexpr int kDwBM = 256;                          // latent positions per tile
constexpr int kDwArow = kDwBM;                      // A stage row (elements, 512 B)
constexpr int kDwBrow = 256;                        // B stage row (elements, 512 B)
constexpr int kDwStage = 32 * (kDwArow + kDwBrow);  // elements per stage
constexpr int kDwStages = 3;
constexpr int kDwSlots = 1024;                      // slots per LDS row table
constexpr int kDwWaves = 8;
constexpr int kDwCopies = 4;                        // DMA instructions per wave per stage
constexpr int kDwPerHead = (kD / kDwBM) * 2;        // 2 dW_UV + 2 dW_UK tiles
constexpr uint32_t kPastEnd = 0x80000000u;          // an offset beyond every bound used

__device__ inline int dw_swz(int row) { return (2 * row) & 15; }

template <int NT, int NOUT>
__device__ inline void dw_dma_tile(const bf16* __restrict__ lat, const bf16* __restrict__ rowsrc,
                                   const int4* __restrict__ srec, int n_slots, int h, int m0,
                                   int n0, int N, int L5, size_t src_rows, bf16* __restrict__ dw,
                                   bf16* lds, int* rbase) {
    constexpr int MT = 8;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;
    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the gathered operand: every input row of head h from column n0 on
    const bf16* bbase = rowsrc + (size_t)h * NOUT + n0;
    const i32x4 rs_b = rsrc_words(bbase, (uint32_t)(src_rows * kH * NOUT * 2 -
                                                    ((size_t)h * NOUT + n0) * 2));
    constexpr uint32_t kLatRow = kH * kD * 2, kSrcRow = kH * NOUT * 2;

    // transposing fragment read of a swizzled stage: 16 rows of k (two
    // reads of 4 x 4), columns r0 .. r0 + 15
    auto frag = [&](const bf16* base, int rowlen, int r0) -> bf16x8 {
        const int col = r0 + 4 * (l16 & 3);
        const int rr = 4 * g + (l16 >> 2);
        const bf16* p0 = base + rr * rowlen + ((((col >> 3) ^ dw_swz(rr)) << 3) | (col & 7));
        const bf16* p1 = base + (rr + 16) * rowlen +
                         ((((col >> 3) ^ dw_swz(rr + 16)) << 3) | (col & 7));
        return cat(lds_read_tr(p0), lds_read_tr(p1));
    };

    for (int c0 = 0; c0 < n_slots; c0 += kDwSlots) {
        const int nsl = min(kDwSlots, n_slots - c0);
        __syncthreads();                 // the previous chunk is done with the table and stages
        for (int i = tid; i < nsl; i += blockDim.x) {
            const int blk = srec[c0 + i].w;
            rbase[i] = (blk / N) * L5 + kBlock * (blk % N);
        }
        __syncthreads();
        const int krows = kBlock * nsl;
        const int steps = (krows + 31) / 32;
        const i32x4 rs_a = rsrc_words(lat + ((size_t)kBlock * c0 * kH + h) * kD + m0,
                                      (uint32_t)krows * kLatRow);

        // stage s (rows 32 s .. 32 s + 31 of this chunk) into ring slot s % 3:
        // A and B each as 16 copies of two 512-byte rows; wave w issues copies
        // 2w and 2w + 1 of each
        auto issue = [&](int s) {
            char* st = reinterpret_cast<char*>(lds + (s % kDwStages) * kDwStage);
            uint32_t boff[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = 2 * (2 * wave + q) + (lane >> 5);
                const int k = 32 * s + row;
                const int lc = (lane & 31) ^ dw_swz(row);
                boff[q] = kPastEnd;
                if (k < krows) {
                    const int sl = k / kBlock;
                    boff[q] = (uint32_t)(rbase[sl] + (k - kBlock * sl)) * kSrcRow + 16 * lc;
                }
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r2 = 2 * (2 * wave + q);
                const int row = r2 + (lane >> 5);
                const int lc = (lane & 31) ^ dw_swz(row);
                copy_16_untracked(rs_a, (uint32_t)(32 * s + row) * kLatRow + 16 * lc,
                                  st + r2 * (kDwArow * 2));
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                copy_16_untracked(rs_b, boff[q],
                                  st + 32 * kDwArow * 2 + 2 * (2 * wave + q) * (kDwBrow * 2));
        };

        issue(0);
        if (steps > 1) issue(1);
        for (int s = 0; s < steps; ++s) {
            // this wave's copies of stage s are done (only stage s + 1's may be
            // in flight); the barrier makes every wave's copies visible and
            // ends every read of the slot stage s + 2 reuses
            if (s + 1 < steps) __builtin_amdgcn_s_waitcnt(wait_vm(kDwCopies));
            else __builtin_amdgcn_s_waitcnt(wait_vm(0));
            __syncthreads();
            if (s + 2 < steps) issue(s + 2);
            const bf16* st = lds + (s % kDwStages) * kDwStage;
            bf16x8 af[MT], bfr[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i) af[i] = frag(st, kDwArow, wm * 16 * MT + 16 * i);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bfr[j] = frag(st + 32 * kDwArow, kDwBrow, wn * 16 * NT + 16 * j);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int o = n0 + wn * 16 * NT + 16 * j + l16;
        bf16* dst = dw + ((size_t)h * NOUT + o) * kD;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int pos = m0 + wm * 16 * MT + 16 * i + 4 * g;
            gst8(dst + dim_of_pos4(pos), to_bf16x4(acc[i][j]));
        }
    }
}

__global__ __launch_bounds__(kDwWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void dw_dma_kernel(
    const bf16* __restrict__ olat, const bf16* __restrict__ dout, const bf16* __restrict__ dqabs,
    const bf16* __restrict__ q_nope, const int4* __restrict__ srec,
    const int32_t* __restrict__ status, bf16* __restrict__ dw_uv, bf16* __restrict__ dw_uk, int N,
    int L5, int in_rows) {
    static_assert(kD % kDwBM == 0 && kDv == 4 * 64 && kDc == 4 * 48 && kDv <= kDwBrow, "tile split");
    __shared__ __attribute__((aligned(16))) bf16 lds[kDwStages * kDwStage];
    __shared__ int rbase[kDwSlots];
    const int n_slots = status[kStKeptCount];
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = lid / kDwPerHead, t = lid % kDwPerHead;
    const int m0 = (t & 1) * kDwBM;
    if (t < 2)
        dw_dma_tile<4, kDv>(olat, dout, srec, n_slots, h, m0, 0, N, L5, in_rows, dw_uv, lds,
                            rbase);
    else
        dw_dma_tile<3, kDc>(dqabs, q_nope, srec, n_slots, h, m0, 0, N, L5, in_rows, dw_uk, lds,
                            rbase);
}

// ---- per block: dc_k (M = D, permuted positions) and d(R k^R)_k (M = d_r,
// natural) for its key slots (N = 144): four 128-position tiles of dc (K =
// the 320 rows twice: P with d_olat, then dS' with q_abs) and one 64-dim
// tile of the rotated-key gradient (K = dS' with R q^R).  When every
// sample's kept anchors ascend, each block writes its partial rows and the
// final pass sums, per context row, the contiguous range of blocks whose
// windows hold it; otherwise the sums go to the fp32 accumulator with
// atomics.  A block's own 5 keys are its alone.
// Each wave owns 32 (or 16) rows x 144 keys, so a k-step reads 11 fragments
// for 18 MFMAs (64-row tiles: 10 for 9), and the P / dS' rows go to L2 five
// times per block instead of nine.  Operands reach LDS by buffer DMA in a
// three-stage ring, like the weight gradients.  A block's operand rows are
// contiguous, so every copy is a plain range: A rows XOR-swizzled by row
// (256-byte rows: (2 row) mod 16; 128-byte rows: row & 6), B rows (288
// bytes, 8 dwords past a multiple of 64 banks) stored as they are, which
// already keeps eight rows' transposing reads on distinct banks.
constexpr int kKvBM = 128;                          // dc positions per tile
constexpr int kKvBrow = kKeySlots;                  // B stage row (elements, 288 B)
constexpr int kKvAbytes = 32 * kKvBM * 2;           // 8 KB
constexpr int kKvStageBytes = kKvAbytes + 32 * kKvBrow * 2;   // + 9 KB
constexpr int kKvStages = 3;
constexpr int kKvTiles = kD / kKvBM + 1;            // 4 dc tiles + the k^R tile
constexpr int kKvBcopies = 32 * kKvBrow * 2 / 1024; // 9 one-KB copies per stage

template <int MT>
__device__ inline void dkv_dma_tile(const bf16* __restrict__ dolat, const bf16* __restrict__ qabs,
                                    const bf16* __restrict__ qrot, const bf16* __restrict__ pm,
                                    const bf16* __restrict__ ds, size_t lat0, int m0, char* lds,
                                    f32x4 (&acc)[MT][9]) {
    constexpr bool kRope = MT == 1;                 // rope tile: 64 dims, rows 128 B
    constexpr int kRows = kBlock * kH;              // 320
    constexpr int kArow = kRope ? kDr : kKvBM;      // A stage row (elements)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 9; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const i32x4 rs_p = rsrc_words(pm, kRows * kKeySlots * 2);
    const i32x4 rs_ds = rsrc_words(ds, kRows * kKeySlots * 2);
    const i32x4 rs_dol = rsrc_words(dolat + lat0 * kD + m0, kRows * kD * 2);
    const i32x4 rs_qa = rsrc_words(qabs + lat0 * kD + m0, kRows * kD * 2);
    const i32x4 rs_qr = rsrc_words(qrot + lat0 * kDr, kRows * kDr * 2);
    auto swz = [](int row) { return kRope ? (row & 6) : ((2 * row) & 15); };

    // stage s: k rows 32 s .. 32 s + 31 of [P | dS'] x [d_olat | q_abs]
    // (rope: of dS' x R q^R, s >= 10)
    auto issue = [&](int s) {
        char* st = lds + (s % kKvStages) * kKvStageBytes;
        const bool second = s >= kRows / 32;
        const int r0 = 32 * (second ? s - kRows / 32 : s);
        if constexpr (kRope) {
            // 4 copies of eight 128-byte rows, one per wave
            const int row = 8 * wave + (lane >> 3);
            const int lc = (lane & 7) ^ swz(row);
            copy_16_untracked(rs_qr, (uint32_t)(r0 + row) * (kDr * 2) + 16 * lc,
                              st + 8 * wave * (kDr * 2));
        } else {
            // 8 copies of four 256-byte rows, two per wave
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r4 = 4 * (2 * wave + q);
                const int row = r4 + (lane >> 4);
                const int lc = (lane & 15) ^ swz(row);
                copy_16_untracked(second ? rs_qa : rs_dol,
                                  (uint32_t)(r0 + row) * (kD * 2) + 16 * lc,
                                  st + r4 * (kKvBM * 2));
            }
        }
        // B: the stage's 32 rows are one contiguous 9 KB range
        const uint32_t b0 = (uint32_t)r0 * (kKeySlots * 2);
        for (int q = wave; q < kKvBcopies; q += 4)
            copy_16_untracked(second ? rs_ds : rs_p, b0 + 1024 * q + 16 * lane,
                              st + kKvAbytes + 1024 * q);
    };
    // copies per wave per stage: A (2, rope 1) + B (3 for wave 0, else 2)
    constexpr int kAc = kRope ? 1 : 2;

    auto frag_a = [&](const bf16* base, int r0) -> bf16x8 {
        const int col = r0 + 4 * (l16 & 3);
        const int rr = 4 * g + (l16 >> 2);
        const bf16* p0 = base + rr * kArow + ((((col >> 3) ^ swz(rr)) << 3) | (col & 7));
        const bf16* p1 = base + (rr + 16) * kArow +
                         ((((col >> 3) ^ swz(rr + 16)) << 3) | (col & 7));
        return cat(lds_read_tr(p0), lds_read_tr(p1));
    };
    auto frag_b = [&](const bf16* base, int r0) -> bf16x8 {
        const int col = r0 + 4 * (l16 & 3);
        const int rr = 4 * g + (l16 >> 2);
        return cat(lds_read_tr(base + rr * kKvBrow + col),
                   lds_read_tr(base + (rr + 16) * kKvBrow + col));
    };

    const int s0 = kRope ? kRows / 32 : 0, s1 = 2 * kRows / 32;
    issue(s0);
    issue(s0 + 1);
    for (int s = s0; s < s1; ++s) {
        if (s + 1 < s1) {
            if (wave == 0) __builtin_amdgcn_s_waitcnt(wait_vm(kAc + 3));
            else __builtin_amdgcn_s_waitcnt(wait_vm(kAc + 2));
        } else {
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
        }
        __syncthreads();
        if (s + 2 < s1) issue(s + 2);
        const char* st = lds + (s % kKvStages) * kKvStageBytes;
        const bf16* sa = reinterpret_cast<const bf16*>(st);
        const bf16* sb = reinterpret_cast<const bf16*>(st + kKvAbytes);
        bf16x8 af[MT], bfr[9];
#pragma unroll
        for (int i = 0; i < MT; ++i) af[i] = frag_a(sa, wave * 16 * MT + 16 * i);
#pragma unroll
        for (int j = 0; j < 9; ++j) bfr[j] = frag_b(sb, 16 * j);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 9; ++j) acc[i][j] = mfma_16x16x32(af[i], bfr[j], acc[i][j]);
    }
}

template <int MT>
__device__ inline void dkv_store(const f32x4 (&a)[MT][9], int m0, int slot, const int4* srec,
                                 const int32_t* status, float* part, float* acc, int S, int N,
                                 int L5) {
    constexpr bool kRope = MT == 1;
    const int4 rec = srec[slot];
    const int blk = rec.w, b = blk / N, n = blk % N;
    const int ctx_lo = rec.x, ctx_len = rec.y, nkeys = ctx_len + kBlock;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, l16 = lane & 15;
    const size_t arow0 = (size_t)b * (S + L5);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int pos = wave * 16 * MT + 16 * i + 4 * g;
        const int dim = kRope ? kD + pos : dim_of_pos4(m0 + pos);
        if (status[kStUnsorted] == 0) {
            float* base = part + (size_t)slot * kMaxKeys * (kD + kDr) + dim;
#pragma unroll
            for (int j = 0; j < 9; ++j) {
                const int key = 16 * j + l16;
                if (key < nkeys)
                    *reinterpret_cast<f32x4*>(base + (size_t)key * (kD + kDr)) = a[i][j];
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < 9; ++j) {
            const int key = 16 * j + l16;
            if (key >= nkeys) continue;
            const size_t r = arow0 + ((key < ctx_len) ? (size_t)(ctx_lo + key)
                                                      : (size_t)S + kBlock * n + (key - ctx_len));
            float* dst = acc + r * (kD + kDr) + dim;
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(dst + e, a[i][j][e]);
        }
    }
}

__global__ __launch_bounds__(256) void dkv_dma_kernel(
    const bf16* __restrict__ dolat, const bf16* __restrict__ qabs, const bf16* __restrict__ qrot,
    const bf16* __restrict__ pmat, const bf16* __restrict__ dsmat, const int4* __restrict__ srec,
    const int32_t* __restrict__ status, float* __restrict__ part, float* __restrict__ acc, int S,
    int N, int L5) {
    static_assert(kKeySlots == 9 * 16 && (32 * kKvBrow * 2) % 1024 == 0, "B stage copies");
    __shared__ __attribute__((aligned(16))) char lds[kKvStages * kKvStageBytes];
    constexpr int kRows = kBlock * kH;
    const int n_live = status[kStKeptCount];
    const int lid = xcd_balance(blockIdx.x, n_live * kKvTiles);
    if (lid < 0) return;
    const int slot = lid / kKvTiles, mt = lid % kKvTiles;
    const size_t lat0 = (size_t)kBlock * slot * kH;
    const bf16* pm = pmat + (size_t)slot * kRows * kKeySlots;
    const bf16* ds = dsmat + (size_t)slot * kRows * kKeySlots;
    if (mt < kKvTiles - 1) {
        f32x4 a[2][9];
        dkv_dma_tile<2>(dolat, qabs, qrot, pm, ds, lat0, mt * kKvBM, lds, a);
        dkv_store<2>(a, mt * kKvBM, slot, srec, status, part, acc, S, N, L5);
    } else {
        f32x4 a[1][9];
        dkv_dma_tile<1>(dolat, qabs, qrot, pm, ds, lat0, 0, lds, a);
        dkv_store<1>(a, 0, slot, srec, status, part, acc, S, N, L5);
    }
}

}  // namespace

hipError_t launch_bwd_dw(const Problem& p, const Inputs& in, const BwdGrads& g,
                         const BwdWork& w, hipStream_t s) {
    // the DMA kernel addresses the gathered inputs with 32-bit offsets
    const size_t in_rows = (size_t)p.B * p.L5;
    if (in_rows * kH * kDv * 2 < kPastEnd && in_rows * kH * kDc * 2 < kPastEnd &&
        (size_t)kBlock * kDwSlots * kH * kD * 2 < kPastEnd) {
        hipLaunchKernelGGL(dw_dma_kernel, dim3(kH * kDwPerHead), dim3(kDwWaves * 64), 0, s,
                           w.fwd.olat,
                           (const bf16*)g.dout, w.dqabs, (const bf16*)in.q_nope, w.fwd.srec,
                           w.fwd.status, (bf16*)g.dw_uv, (bf16*)g.dw_uk, p.N, p.L5, (int)in_rows);
        return hipGetLastError();
    }
    constexpr int kPerHead = (kD / CfgDwuv::BM) * (kDv / CfgDwuv::BN) +
                             (kD / CfgDwuk::BM) * (kDc / CfgDwuk::BN);
    hipLaunchKernelGGL(dw_kernel, dim3(kH * kPerHead), dim3(256), 0, s, w.fwd.olat,
                       (const bf16*)g.dout, w.dqabs, (const bf16*)in.q_nope, w.fwd.srec,
                       w.fwd.status, (bf16*)g.dw_uv, (bf16*)g.dw_uk, p.N, p.L5);
    return hipGetLastError();
}

hipError_t launch_bwd_dkv(const Problem& p, const BwdWork& w, hipStream_t s) {
    int grid = p.B * p.N * kKvTiles;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL(dkv_dma_kernel, dim3(grid), dim3(256), 0, s, w.dolat, w.fwd.qabs, w.qrot,
                       w.pmat, w.dsmat, w.fwd.srec, w.fwd.status, w.part, w.acc, p.S, p.N, p.L5);
    return hipGetLastError();
}

}  // namespace dspark
