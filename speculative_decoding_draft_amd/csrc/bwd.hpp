// Backward of the masked latent attention: workspace layout and launch
// wrappers (internal to libdspark_attn.so).
#pragma once

#include "kernels.hpp"

namespace dspark {

// Workspace of dspark_attn_bwd.  The first five areas have the forward's
// layout (status at offset 0), so the index builder is shared.
//
// MFMA path, per kept block (slot) s and query t, latent row R = 5 s + t:
//   qabs  bf16 [5*B*N][H][D]   W_UK[h]^T q^C         (permuted 32-dim groups)
//   dolat bf16 [5*B*N][H][D]   W_UV[h]^T dout        (permuted)
//   olat  bf16 [5*B*N][H][D]   softmax-weighted c^KV (permuted)
//   dqabs bf16 [5*B*N][H][D]   scale * sum_k dS_k c^KV_k (permuted)
//   qrot  bf16 [5*B*N][H][d_r] rotated q^R
//   pmat  bf16 [B*N][5H][144]  softmax weights, row = t*H + h, column = key slot
//   dsmat bf16 [B*N][5H][144]  scale * dS, same layout
//   part  f32 [B*N][132][D + d_r]  per block: dc^KV and d(rotated k^R) of its
//                                  key slots (summed over its 5 x 64 rows)
// Both paths:
//   acc   f32 [B][S + 5N][D + d_r]  sums over blocks and heads of dc^KV and of
//                                   d(rotated k^R), context rows then block rows
//   wacc  f32 [H][d_c + d_v][D]     generic path: dW_UK then dW_UV
// "Permuted" is the order the attention kernels read and write latent rows
// in: inside every 32-dim group, position 8g + e holds dim 16(e/4) + 4g + e%4.
struct BwdLayout {
    WsLayout fwd;
    size_t dolat = 0, dqabs = 0, qrot = 0, pmat = 0, dsmat = 0, part = 0, acc = 0, wacc = 0;
    size_t acc_rows = 0;   // B * (S + 5N)
    size_t total = 0;
};


inline BwdLayout bwd_layout(const dspark_attn_desc& d, bool mfma) {
    BwdLayout L;
    L.fwd = ws_layout(d, mfma);
    size_t off = L.fwd.total;
    const size_t blocks = size_t(d.B) * size_t(d.N);
    if (mfma) {
        const size_t lat = size_t(d.n_heads) * kBlock * blocks * size_t(d.d_latent) * 2;
        L.dolat = off; off = align256(off + lat);
        L.dqabs = off; off = align256(off + lat);
        L.qrot = off;  off = align256(off + size_t(d.n_heads) * kBlock * blocks * d.d_rope * 2);
        const size_t pm = blocks * kBlock * size_t(d.n_heads) * kKeySlots * 2;
        L.pmat = off;  off = align256(off + pm);
        L.dsmat = off; off = align256(off + pm);
        L.part = off;
        off = align256(off + blocks * kMaxKeys * size_t(d.d_latent + d.d_rope) * 4);
    }
    L.acc_rows = size_t(d.B) * (size_t(d.S) + size_t(kBlock) * d.N);
    L.acc = off; off = align256(off + L.acc_rows * size_t(d.d_latent + d.d_rope) * 4);
    if (!mfma) {
        L.wacc = off;
        off = align256(off + size_t(d.n_heads) * (d.d_nope + d.d_v) * size_t(d.d_latent) * 4);
    }
    L.total = off;
    return L;
}

struct BwdGrads {
    const void* dout;
    void* dq_nope;
    void* dq_rope;
    void* dckv_ctx;
    void* dkr_ctx;
    void* dckv_blk;
    void* dkr_blk;
    void* dw_uk;
    void* dw_uv;
};

struct BwdWork {
    Workspace fwd;
    bf16* dolat;
    bf16* dqabs;
    bf16* qrot;
    bf16* pmat;
    bf16* dsmat;
    float* part;
    float* acc;
    float* wacc;
};

// Zero the fp32 accumulators (and, on the generic path, the weight ones).
// only_if: nullptr (always), or a status word -- the clear runs only when
// that word is nonzero.
hipError_t launch_bwd_zero(float* p, size_t n, const int32_t* only_if, hipStream_t s);
// reuse_forward: unless status[kStPathTag] is expect or (when nonzero)
// expect2, flags the call (status[kStReuseBad] = 1) and turns the index into
// an all-padding one (no kept block, every record padding) so that the
// launches after it read no record of another forward.
hipError_t launch_bwd_reuse_check(const Problem& p, const BwdWork& w, int32_t expect,
                                  int32_t expect2, hipStream_t s);
// On a flagged call, every element of the eight gradients becomes NaN;
// otherwise the launch exits at once.  elem: 2 (bf16) or 4 (fp32) bytes.
hipError_t launch_bwd_reuse_fill(const Problem& p, const BwdGrads& g, const BwdWork& w,
                                 int elem, hipStream_t s);
// MFMA path final pass: per row, the block partials of the windows that
// cover it (ascending anchors) or the accumulator row (otherwise), converted
// to the output type with R^T applied to dk^R; plus the query-gradient rows
// of blocks that were not computed.
hipError_t launch_bwd_gather(const Problem& p, const BwdGrads& g, const BwdWork& w,
                             const RopeTheta& th, hipStream_t s);
// Generic path: one workgroup per (block, head), fp32 arithmetic, atomics
// into the accumulators.
hipError_t launch_bwd_generic(const Problem& p, bool bf16_io, const Inputs& in,
                              const BwdGrads& g, const BwdWork& w, hipStream_t s);
size_t bwd_generic_lds_bytes(const Problem& p);
// Accumulators -> dc^KV / dk^R outputs (R^T applied to dk^R); rows of query
// gradients of blocks that are not computed (0 for padding, NaN for a kept
// block with a bad anchor); on the generic path also the weight gradients.
// table: the RoPE table (generic path) or nullptr (angles evaluated from
// th, the theta_i of the descriptor).
hipError_t launch_bwd_finalize(const Problem& p, bool bf16_io, const BwdGrads& g,
                               const BwdWork& w, const int4* idx, const float2* table,
                               const RopeTheta& th, bool weights, hipStream_t s);

// MFMA path (bf16, GLM dims).
// d_olat = W_UV[h]^T dout for every kept row: the forward's absorb kernel
// with d_v = 256 input dims (absorb.hip); written in the permuted latent order.
// Its workgroups also clear the fp32 accumulator (n floats, a multiple of 4)
// first when status[kStUnsorted] is set (the atomic dc^KV sums need it).
hipError_t launch_absorb_dv(const Problem& p, const void* dout, const void* w_uv,
                            const Workspace& ws, bf16* dolat, float* acc, size_t n,
                            hipStream_t s);
// dq^C = W_UK[h] dq_abs for every kept row: the forward's W_UV kernel with
// 192 output dims (uv.hip).
hipError_t launch_uv_dqc(const Problem& p, const void* w_uk, const bf16* dqabs,
                         const Workspace& ws, void* dq_nope, hipStream_t s);
// write_olat: the backward has no forward before it (o_lat is recomputed);
// load_p: the forward before it left P in pmat (scores are not recomputed).
hipError_t launch_bwd_attn(const Problem& p, const Inputs& in, const BwdGrads& g,
                           const BwdWork& w, const RopeTheta& th, hipStream_t s, bool write_olat,
                           bool load_p);
hipError_t launch_bwd_dkv(const Problem& p, const BwdWork& w, hipStream_t s);
hipError_t launch_bwd_dw(const Problem& p, const Inputs& in, const BwdGrads& g,
                         const BwdWork& w, hipStream_t s);

}  // namespace dspark
