/*
 * dspark_attn.h -- C ABI of libdspark_attn.so, the MI355X (gfx950) DSpark
 * draft-attention forward and its backward.
 *
 * What is computed (GLM 5.2 DSpark training-design page, "GLM 5.2 DSpark
 * 投机训练设计"): for every draft block n of every sample b, anchored at
 * context position A_n, the 5 queries [x_A, MASK x4] attend over
 *   - the context window [A_n - W + 1, A_n) of the projected context
 *     (§3 "Causal attention"; the same window for all 5 queries, A_n itself
 *     excluded, clamped at 0), and
 *   - the 5 positions of their own block, bidirectionally (§3
 *     "Bidirectional attention");
 * a padding block (keep = 0) attends to nothing (§3 "Padding block").
 * Keys and values are the MLA ones of §4 "MLA Projection": per head
 * K_h = [W_UK[h] c^KV ; RoPE(k^R)], V_h = W_UV[h] c^KV; queries are
 * [q^C ; RoPE(q^R)]; the scale is (d_c + d_r)^(-1/2) (§4); RoPE rotates
 * interleaved adjacent pairs at the positions of §2 "QKV construction"
 * (context 0..S-1, block n: A_n .. A_n+4).  The attention itself is the
 * equation of the appendix "Attention implementation":
 * softmax(scale * Q K^T + Lambda(M)) V.
 *
 * The library computes the same values in the absorbed latent form
 * (q_abs = W_UK[h]^T q^C, scores over the 576 cached numbers per key,
 * P . c^KV over 512, then W_UV[h]), which is an algebraic identity.
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers to contiguous row-major data,
 *     16-byte aligned, unless the comment says "host";
 *   - the caller owns every buffer, including the workspace; the library
 *     allocates and frees no device memory of its own, so calls on different
 *     streams with different workspaces are independent.  The one exception:
 *     the MLA block and the loss head create one rocBLAS handle per host
 *     thread and device on first use (rocBLAS itself works in the caller's
 *     workspace, and GEMM kernel choices live in a caller-owned
 *     dspark_gemm_choices table);
 *   - `stream` is a hipStream_t (NULL = the default stream); device work is
 *     enqueued asynchronously and DSPARK_OK means "enqueued";
 *   - no C++ exception crosses the ABI; on error the function returns a
 *     negative dspark_status, enqueues nothing, and dspark_last_error()
 *     returns a thread-local message.
 */
#ifndef DSPARK_ATTN_H
#define DSPARK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_ABI_VERSION 13

typedef enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_EINVAL = -1,       /* bad argument: null/misaligned pointer, bad size */
    DSPARK_EUNSUPPORTED = -2, /* valid but unsupported shape or dtype */
    DSPARK_EWORKSPACE = -3,   /* workspace missing, misaligned or too small */
    DSPARK_EHIP = -4,         /* a HIP runtime call failed (message has the HIP error) */
    DSPARK_EANCHOR = -5,      /* a kept block had an anchor outside [0, S-2] */
    DSPARK_ECAPACITY = -6     /* more kept blocks than dspark_loss_desc.max_kept_blocks */
} dspark_status;

typedef enum dspark_dtype {
    DSPARK_F32 = 0,  /* fp32 inputs, weights and output */
    DSPARK_BF16 = 1  /* bf16 inputs, weights and output */
} dspark_dtype;

/* Problem description.
 *   B         samples; S context length; N anchor blocks per sample
 *   block     draft block length; must be 5 (design page, §2 "Draft inputs")
 *   window    W of the sliding window: W-1 context positions visible (§3)
 *   n_heads   H;  d_latent D (kv rank, 512 for GLM);  d_nope d_c (192);
 *   d_rope    d_r (64, even);  d_v (256)
 *   rope_base RoPE base (> 0); theta_i = rope_base^(-2i/d_r)
 *   softmax_scale  > 0 overrides the scale; <= 0 selects (d_nope+d_rope)^-1/2
 *   dtype     a dspark_dtype
 * Supported: any positive dims with d_rope even (generic kernels, fp32
 * arithmetic); the MFMA fast path is taken for dtype BF16 with H = 64,
 * D = 512, d_c = 192, d_r = 64, d_v = 256, window <= 128, and q_nope and
 * ckv_ctx each below 4 GiB (B * 5N <= 174762, B * S < 4194304). */
typedef struct dspark_attn_desc {
    int32_t B, S, N, block, window;
    int32_t n_heads, d_latent, d_nope, d_rope, d_v;
    double rope_base;
    double softmax_scale;
    int32_t dtype;
} dspark_attn_desc;

/* Bytes of workspace dspark_attn_fwd(_ex) needs for `desc` whatever the
 * options (0 on an invalid descriptor; see dspark_last_error).  The
 * workspace holds the per-block index records, the compacted list of kept
 * blocks and a small status area, and then, by path:
 *   - generic kernels: the RoPE cos/sin table;
 *   - three-kernel MFMA forward (the default for the MFMA shapes): the
 *     bf16 latent intermediates q_abs and o_lat of every kept block
 *     ([5*B*N, H, D] each, row = 5 * slot + query);
 *   - one-launch MFMA forward (dspark_attn_opts.one_launch on a device with
 *     256 compute units): the pipeline's control words and two rings of 32
 *     kept blocks x 8 XCDs (the bf16 q_abs and o_lat of a block's 5 queries
 *     and one XCD's 8 heads, 40 KB each), about 21 MB in all.
 * It must be 256-byte aligned. */
size_t dspark_attn_workspace_size(const dspark_attn_desc* desc);

/* The masked MLA attention forward of one draft layer.
 *   q_nope  [B, 5N, H, d_c]   q^C of the draft queries (§4 "MLA Projection")
 *   q_rope  [B, 5N, H, d_r]   q^R, NOT yet rotated
 *   ckv_ctx [B, S, D]         c^KV of the context (after kv_a_layernorm)
 *   kr_ctx  [B, S, d_r]       k^R of the context, not rotated
 *   ckv_blk [B, 5N, D]        c^KV of the draft-block positions
 *   kr_blk  [B, 5N, d_r]      k^R of the draft-block positions, not rotated
 *   w_uk    [H, d_c, D]       k^C_h = w_uk[h] @ c^KV   (kv_b_proj, key part)
 *   w_uv    [H, d_v, D]       v_h   = w_uv[h] @ c^KV   (kv_b_proj, value part)
 *   anchors [B, N] int32      A_n; read only where keep = 1
 *   keep    [B, N] uint8      block_keep_mask (0 = padding block)
 *   out     [B, 5N, H, d_v]   attention output per head (before o_proj)
 * Rows of padding blocks are written as 0.  A kept block whose anchor lies
 * outside [0, S-2] is an error detected on the device: its rows are written
 * as NaN and dspark_read_device_status reports DSPARK_EANCHOR.
 * Inputs and output share desc->dtype.  Tensors must not alias `out` or the
 * workspace. */
dspark_status dspark_attn_fwd(const dspark_attn_desc* desc,
                              const void* q_nope, const void* q_rope,
                              const void* ckv_ctx, const void* kr_ctx,
                              const void* ckv_blk, const void* kr_blk,
                              const void* w_uk, const void* w_uv,
                              const int32_t* anchors, const uint8_t* keep,
                              void* out, void* workspace, size_t ws_bytes,
                              void* stream);

/* rocBLAS kernel choices for the GEMMs of one dspark_mla_layer_fwd_ex or
 * dspark_loss_fwd_ex call, in the order the call runs them.  Filled by
 * dspark_mla_layer_tune / dspark_loss_tune; handed back through
 * dspark_attn_opts.gemm_choices.  Owned by the caller (host memory); the
 * library keeps no table of its own.  A GEMM whose (m, n, k) differs from its
 * entry's, or past n_gemms, uses rocBLAS's own choice. */
#define DSPARK_MAX_GEMMS 8
typedef struct dspark_gemm_choice {
    int32_t m, n, k;        /* the GEMM's row-major shape: D[m][n] = A[m][k] B[n][k]^T */
    int32_t solution;       /* rocBLAS solution index; 0 = rocBLAS's own choice */
} dspark_gemm_choice;
typedef struct dspark_gemm_choices {
    int32_t n_gemms;
    dspark_gemm_choice gemm[DSPARK_MAX_GEMMS];
} dspark_gemm_choices;

/* Bytes of the MLA block's and the loss head's workspace set aside for
 * rocBLAS, handed to it with rocblas_set_workspace at the start of each
 * call (the handle keeps pointing there until the next call sets its own).
 * Measured on the logits GEMM at V = 154880: with rocBLAS's own memory 462
 * of its 682 kernels refuse to run, with 4 MiB 402, with 64 MiB 18, and the
 * fastest needs more than 4 MiB. */
#define DSPARK_BLAS_WORKSPACE_BYTES ((size_t)64 << 20)

/* Extra controls for dspark_attn_fwd_ex (zero-initialise, then set fields). */
typedef struct dspark_attn_opts {
    /* NULL, or hipEvent_t handles recorded between the kernels of the call,
     * in launch order: [0] before the index build, [1] after the index
     * build, padding fill and (generic path) RoPE table, both on `stream`,
     * then for round c
     * (see dspark_attn_plan), on the stream that runs the round: [2 + 4c]
     * before its absorb, [3 + 4c] after it, [4 + 4c] after its attention
     * kernel, [5 + 4c] after its W_UV projection.  The generic path and
     * the one-launch forward record [0], [1] and [2] after their single
     * kernel. */
    void* const* stage_events;
    int32_t n_stage_events;   /* at least the count dspark_attn_plan reports */
    int32_t force_generic;    /* nonzero: use the generic fp32 kernels even
                                 where the MFMA path applies */
    int32_t chunk_blocks;     /* > 0: kept blocks per kernel round on the MFMA
                                 path; 0: one round over all B*N blocks */
    /* NULL, or a second hipStream_t.  With two or more rounds, odd rounds
     * run on aux_stream and even rounds on `stream`, so that a round's
     * kernels overlap the ramp-up and tail of the other stream's; the call
     * records aux_events[0] on `stream` after the preparation launch and
     * makes aux_stream wait for it, records aux_events[1] on aux_stream after
     * its last round and makes `stream` wait for it, so work enqueued on
     * `stream` afterwards sees the whole result.  Both events are created by
     * the caller (timing may be disabled) and must not be in use elsewhere
     * during the call.  aux_stream must not be `stream`. */
    void* aux_stream;
    void* aux_events[2];
    /* dspark_attn_bwd_ex, 1 or 2: the workspace was last used by
     * dspark_attn_fwd(_ex) with the same descriptor, inputs, anchors and keep
     * and the same force_generic, and nothing else has written it since (a
     * training step runs the forward on the backward's workspace: its
     * layout begins with the forward's).  The backward then reuses the
     * forward's block index, q_abs and o_lat instead of rebuilding them
     * (dW_UV then uses the forward's o_lat rows).  2 on the MFMA path: the
     * forward also left its softmax probabilities (it ran with this option
     * set, below), and the backward reads them instead of recomputing the
     * scores; the gradients are the same bits as with 1.  This is checked on
     * the device: the index build of a forward (or of a backward without
     * this option) tags the workspace with its descriptor, its path and
     * whether it left the probabilities, and a backward whose workspace does
     * not carry a tag it accepts (1: this descriptor on the path it takes,
     * MFMA or generic, with or without probabilities; 2: this descriptor on
     * the MFMA path with probabilities; the one-launch forward leaves no
     * latents and never matches) writes NaN to every gradient and
     * dspark_read_device_status then returns DSPARK_EINVAL.
     * dspark_attn_fwd_ex, nonzero: the workspace is a backward's for this
     * descriptor (dspark_attn_workspace_size_ex with this option gives its
     * size on the MFMA path; a smaller one is refused with
     * DSPARK_EWORKSPACE), and the MFMA forward also writes its softmax
     * probabilities there (bf16) for a backward with reuse_forward 2.
     * Refused (DSPARK_EINVAL) with the one-launch forward; ignored on the
     * generic path. */
    int32_t reuse_forward;
    /* dspark_attn_fwd_ex on the MFMA shapes, nonzero: the one-launch
     * forward instead of the three kernels (ignored with chunk_blocks or
     * aux_stream; on a device without 256 compute units the three kernels
     * run).  It runs absorb, attention and W_UV side by side on different
     * compute units of each XCD, each XCD owning 8 heads, and passes q_abs
     * and o_lat through rings in that XCD's L2 instead of HBM; it needs all
     * 256 of its workgroups resident at once (nothing else running on the
     * device), bounds every internal wait in time, and reports a stall
     * through dspark_read_device_status (DSPARK_EHIP) instead of hanging.
     * It leaves no q_abs / o_lat for reuse_forward.  Measured on the
     * headline workload it is slower than the three kernels (each XCD
     * re-reads every block's keys for its heads, and its units wait on one
     * another); it is kept as a parity-tested alternative. */
    int32_t one_launch;
    /* dspark_mla_layer_fwd_ex and dspark_loss_fwd_ex: NULL (rocBLAS chooses
     * every GEMM kernel), or the choices a *_tune call filled. */
    const dspark_gemm_choices* gemm_choices;
} dspark_attn_opts;

/* Bytes of workspace dspark_attn_fwd_ex needs for (desc, opts) on a device
 * with 256 compute units (opts may be NULL; 0 on an invalid descriptor):
 * the size of the path those options select, which is smaller than
 * dspark_attn_workspace_size for the one-launch forward, and a backward's
 * (MFMA path) with reuse_forward set.  On a device where
 * the one-launch forward cannot run, the call falls back to the three-kernel
 * forward and needs dspark_attn_workspace_size(desc) bytes (a smaller
 * workspace is then refused with DSPARK_EWORKSPACE). */
size_t dspark_attn_workspace_size_ex(const dspark_attn_desc* desc, const dspark_attn_opts* opts);

/* Launch plan of dspark_attn_fwd_ex for (desc, opts) (opts may be NULL) on
 * the current device: *n_chunks kernel rounds of *chunk_blocks kept blocks
 * each (the count is an upper bound: chunks past the number of kept blocks
 * exit at once; the one-launch forward is one round over all B*N blocks,
 * the generic path none), and *n_events stage events recorded when
 * opts->stage_events is given.  Any output pointer may be NULL. */
dspark_status dspark_attn_plan(const dspark_attn_desc* desc, const dspark_attn_opts* opts,
                               int32_t* n_chunks, int32_t* chunk_blocks, int32_t* n_events);

/* dspark_attn_fwd with options; opts may be NULL. */
dspark_status dspark_attn_fwd_ex(const dspark_attn_desc* desc,
                                 const void* q_nope, const void* q_rope,
                                 const void* ckv_ctx, const void* kr_ctx,
                                 const void* ckv_blk, const void* kr_blk,
                                 const void* w_uk, const void* w_uv,
                                 const int32_t* anchors, const uint8_t* keep,
                                 void* out, void* workspace, size_t ws_bytes,
                                 void* stream, const dspark_attn_opts* opts);

/* Bytes of the status area at the start of every workspace (16 int32
 * words), and of the status buffer dspark_attn_fwd_noalloc may be given. */
#define DSPARK_STATUS_BYTES 64

/* Size of the scratch array dspark_attn_fwd_noalloc works in (64 MiB). */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* The forward of dspark_attn_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc): the same inputs, output and results, and no workspace
 * argument.  The library keeps one scratch array of
 * DSPARK_NOALLOC_SCRATCH_BYTES in the memory of each device its code runs
 * on, until the process ends, and this call works in it.  It calls no
 * hipMalloc, hipFree or other allocating routine; its first call on a device
 * looks up the array's address on that device.
 *   status  NULL, or device memory of DSPARK_STATUS_BYTES (4-byte aligned)
 *           that receives the call's status words, to be read with
 *           dspark_read_device_status(status, stream, &first_bad_block).
 *           With NULL the words stay in the array and are not readable.
 * On the MFMA shapes (see dspark_attn_fwd) the three kernels run in rounds of
 * as many kept blocks as the array holds q_abs / o_lat rows for (640 KiB per
 * block at H = 64, D = 512: about 100 blocks), one round after another on
 * `stream`; other shapes run the generic kernel.  Returns DSPARK_EUNSUPPORTED
 * before any device work when the shape does not fit: the index (36 bytes per
 * block of B*N) plus one block's latent rows, or on the generic path the
 * index plus the RoPE table ((S + 8) * d_rope * 4 bytes), above the array's
 * size.  Nothing in the array has to start at zero (each call writes all it
 * reads).  All calls on one device share its array: calls that overlap in
 * time on one device (on different streams or host threads) race, and their
 * results are undefined. */
dspark_status dspark_attn_fwd_noalloc(const dspark_attn_desc* desc,
                                      const void* q_nope, const void* q_rope,
                                      const void* ckv_ctx, const void* kr_ctx,
                                      const void* ckv_blk, const void* kr_blk,
                                      const void* w_uk, const void* w_uv,
                                      const int32_t* anchors, const uint8_t* keep,
                                      void* out, int32_t* status, void* stream);

/* The anchor/window index builder alone (the first stage of the forward).
 * index_out [B, N, 4] int32 per block: {ctx_lo, ctx_len, pos0, slot}
 *   kept block with 0 <= A <= S-2: ctx_lo = max(0, A-W+1), ctx_len = A-ctx_lo
 *     (the visible context columns [ctx_lo, A), §3), pos0 = A (RoPE position
 *     of the block's first query, §2), slot = rank among kept blocks in
 *     (b, n) order;
 *   padding block: {0, 0, 0, -1};  kept block with a bad anchor: {0, 0, 0, -2}.
 * The block's draft columns are S + 5n .. S + 5n + 4 (§3).  The workspace
 * must be sized by dspark_attn_workspace_size(desc). */
dspark_status dspark_build_index(const dspark_attn_desc* desc,
                                 const int32_t* anchors, const uint8_t* keep,
                                 int32_t* index_out, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Host-side anchor sampler (§2 "Anchor sampling"; loss_mask[S-1] is taken as 0,
 * §6 "eval_mask" / appendix A option 2).  All pointers are HOST pointers.
 *   loss_mask [S] uint8 (nonzero = 1), anchors [num_anchors] int32 out,
 *   keep [num_anchors] uint8 out.
 * Candidates C = {A in [0, S-2] : lm[A] = lm[A+1] = 1}, ascending.  If
 * |C| <= num_anchors: C then padding slots (A = 0, keep = 0).  Otherwise a
 * partial Fisher-Yates over C driven by SplitMix64(seed):
 * for i < N: j = i + next() mod (|C| - i), swap C[i], C[j]; then the first N
 * sorted ascending, keep = 1.  Integer-only, hence reproducible exactly. */
dspark_status dspark_select_anchors_host(const uint8_t* loss_mask, int32_t S,
                                         int32_t num_anchors, uint64_t seed,
                                         int32_t* anchors, uint8_t* keep);

/* ---- backward ----------------------------------------------------------
 * Gradients of the same forward: with L = sum over the rows of kept blocks of
 * <dout, out>, the chain rule on softmax(scale * Q K^T + Lambda(M)) V
 * (appendix "Attention implementation") with the keys, values and queries of
 * §4 "MLA Projection" and the rotations of §4 "RoPE".  The forward is
 * recomputed inside the call (no forward state is kept between calls). */

/* Bytes of workspace dspark_attn_bwd needs for `desc` (0 on an invalid
 * descriptor).  Besides the forward's index area it holds fp32 accumulators
 * [B, S + 5N, D + d_r] for the sums over blocks and heads of dc^KV and d k^R
 * (and, on the generic path, [H, d_c + d_v, D] for the weight gradients), and
 * on the MFMA path the bf16 latent intermediates of every kept block (q_abs,
 * W_UV^T dout, o_lat, dq_abs: [5*B*N, H, D] each; rotated q^R; the softmax
 * weights and scaled score gradients, [B*N, 5*H, 144] each).  The size
 * covers both paths (force_generic included).  It must be 256-byte
 * aligned. */
size_t dspark_attn_bwd_workspace_size(const dspark_attn_desc* desc);

/* The backward of dspark_attn_fwd for one draft layer.
 *   q_nope ... keep   the forward's inputs, as in dspark_attn_fwd
 *   dout   [B, 5N, H, d_v]  dL/d out; rows of padding blocks are ignored
 * Outputs (every element written; same dtype as the inputs):
 *   dq_nope [B, 5N, H, d_c]   dq_rope [B, 5N, H, d_r]  (w.r.t. the UNrotated q^R)
 *   dckv_ctx [B, S, D]        dkr_ctx [B, S, d_r]      (w.r.t. the unrotated k^R)
 *   dckv_blk [B, 5N, D]       dkr_blk [B, 5N, d_r]
 *   dw_uk [H, d_c, D]         dw_uv [H, d_v, D]
 * Rows no kept block reaches (padding blocks' queries and keys, context rows
 * outside every window) are 0.  The query rows of a kept block whose anchor
 * lies outside [0, S-2] are NaN and the block contributes nothing else
 * (dspark_read_device_status reports DSPARK_EANCHOR).  Sums over heads and
 * over the blocks whose windows share a context row are fp32.  On the MFMA
 * path, when every sample's kept anchors ascend (as the sampler returns
 * them), each block's share is written once and summed per row in a fixed
 * order, so results are deterministic; otherwise (and on the generic path)
 * the sums use device atomics and their last bits can differ between runs.
 * d_rope = 0 allows NULL for q_rope, kr_ctx, kr_blk, dq_rope, dkr_ctx,
 * dkr_blk.  Outputs must not alias inputs, each other or the workspace. */
dspark_status dspark_attn_bwd(const dspark_attn_desc* desc,
                              const void* q_nope, const void* q_rope,
                              const void* ckv_ctx, const void* kr_ctx,
                              const void* ckv_blk, const void* kr_blk,
                              const void* w_uk, const void* w_uv,
                              const int32_t* anchors, const uint8_t* keep,
                              const void* dout,
                              void* dq_nope, void* dq_rope,
                              void* dckv_ctx, void* dkr_ctx,
                              void* dckv_blk, void* dkr_blk,
                              void* dw_uk, void* dw_uv,
                              void* workspace, size_t ws_bytes, void* stream);

/* dspark_attn_bwd with options (opts may be NULL).  Used fields:
 * force_generic, and stage_events: event [0] is recorded before the first
 * launch and event [k] after the k-th, all on `stream`; the MFMA path makes
 * 10 launches (index, anchor-order check, accumulator clear, absorb,
 * W_UV^T dout, attention backward, dc^KV / dk^R products, dq^C, weight
 * gradients, final pass), the generic path 4 (index and RoPE table,
 * accumulator clear, generic kernel, final pass).
 * chunk_blocks and aux_stream are ignored: the backward runs as one round. */
dspark_status dspark_attn_bwd_ex(const dspark_attn_desc* desc,
                                 const void* q_nope, const void* q_rope,
                                 const void* ckv_ctx, const void* kr_ctx,
                                 const void* ckv_blk, const void* kr_blk,
                                 const void* w_uk, const void* w_uv,
                                 const int32_t* anchors, const uint8_t* keep,
                                 const void* dout,
                                 void* dq_nope, void* dq_rope,
                                 void* dckv_ctx, void* dkr_ctx,
                                 void* dckv_blk, void* dkr_blk,
                                 void* dw_uk, void* dw_uv,
                                 void* workspace, size_t ws_bytes, void* stream,
                                 const dspark_attn_opts* opts);

/* Number of stage events dspark_attn_bwd_ex records for (desc, opts). */
dspark_status dspark_attn_bwd_plan(const dspark_attn_desc* desc, const dspark_attn_opts* opts,
                                   int32_t* n_events);

/* ---- the MLA block of one draft layer -----------------------------------
 * §4 "MLA Projection" around the attention: input_layernorm, q_a_proj,
 * q_a_layernorm, q_b_proj, kv_a_proj_with_mqa over [H^ctx ; h],
 * kv_a_layernorm, the attention above, o_proj added back to the residual:
 *   h = RMSNorm(H; g_in)          c^Q = RMSNorm(h W_qa^T; g_qa)
 *   [q^C ; q^R] per head = c^Q W_qb^T
 *   [c^KV ; k^R] = [H^ctx ; h] W_kva^T,   c^KV <- RMSNorm(c^KV; g_kva)
 *   out = H + attention(...) W_o^T
 * RMSNorm(x; g) = x / sqrt(mean(x^2) + rms_eps) * g (the page gives no
 * epsilon).  The FFN half of the layer is not part of this call. */
typedef struct dspark_layer_desc {
    dspark_attn_desc attn;   /* the attention's problem (B, S, N, dims, dtype) */
    int32_t hidden;          /* d: 6144 for GLM-5.2 */
    int32_t q_rank;          /* q_lora_rank: 2048 */
    double rms_eps;          /* >= 0 */
    int32_t max_kept_blocks; /* 0: B*N.  Otherwise an upper bound on the
                                blocks with keep = 1: the draft-row
                                projections and o_proj run on 5 * this many
                                rows (the kept blocks' rows, compacted) */
} dspark_layer_desc;

/* Bytes of workspace dspark_mla_layer_fwd needs (0 on an invalid descriptor):
 * a status area (first, as for the attention), the kept-block slot lists,
 * the block's intermediates (normalised h, c^Q, q^C, q^R, [c^KV ; k^R] of
 * every context and kept draft row, the attention output, the kept rows'
 * attention output and H compacted, o_proj's result) and the attention's own
 * workspace.  256-byte aligned. */
size_t dspark_mla_layer_workspace_size(const dspark_layer_desc* desc);

/* The MLA block of one draft layer.  Device pointers, desc->attn.dtype:
 *   h_draft [B, 5N, d]   H^(l), the layer input (residual stream)
 *   h_ctx   [B, S, d]    H^ctx (already projected and normalised by main_norm)
 *   g_in [d], w_qa [q_rank, d], g_qa [q_rank],
 *   w_qb [H * (d_c + d_r), q_rank]  (per head: d_c q^C rows, then d_r q^R rows)
 *   w_kva [D + d_r, d]   (c^KV rows, then k^R rows),  g_kva [D]
 *   w_uk [H, d_c, D], w_uv [H, d_v, D]   kv_b_proj, as in dspark_attn_fwd
 *   w_o [d, H * d_v]
 *   anchors, keep        as in dspark_attn_fwd
 *   out [B, 5N, d]       H + o_proj(attention); rows of padding blocks are H
 *                        (their attention rows are 0), rows of a kept block
 *                        with a bad anchor are NaN; every row is NaN when
 *                        more than max_kept_blocks blocks are kept
 *                        (dspark_mla_layer_read_status: DSPARK_ECAPACITY)
 * The rows of kept blocks are compacted (5 per kept block, in (b, n) order)
 * for the draft-row projections and o_proj.  The projections run on rocBLAS
 * (fp32 accumulation, no atomics: the same call gives the same bits;
 * dspark_mla_layer_tune picks the kernels), which works in the
 * DSPARK_BLAS_WORKSPACE_BYTES the workspace sets aside.  The first call on a
 * device and host thread creates a rocBLAS handle that is kept until the
 * process ends -- the one allocation the library makes.  out must not alias
 * any input. */
dspark_status dspark_mla_layer_fwd(const dspark_layer_desc* desc,
                                   const void* h_draft, const void* h_ctx,
                                   const void* g_in, const void* w_qa, const void* g_qa,
                                   const void* w_qb, const void* w_kva, const void* g_kva,
                                   const void* w_uk, const void* w_uv, const void* w_o,
                                   const int32_t* anchors, const uint8_t* keep,
                                   void* out, void* workspace, size_t ws_bytes, void* stream);

/* dspark_mla_layer_fwd with options (opts may be NULL): force_generic is
 * passed to the attention; gemm_choices selects the GEMM kernels;
 * stage_events (at least 7) are recorded on
 * `stream` before the first launch and after: the input RMSNorm, q_a_proj
 * and its RMSNorm, q_b_proj, kv_a_proj and its RMSNorm / k^R split, the
 * attention, o_proj. */
dspark_status dspark_mla_layer_fwd_ex(const dspark_layer_desc* desc,
                                      const void* h_draft, const void* h_ctx,
                                      const void* g_in, const void* w_qa, const void* g_qa,
                                      const void* w_qb, const void* w_kva, const void* g_kva,
                                      const void* w_uk, const void* w_uv, const void* w_o,
                                      const int32_t* anchors, const uint8_t* keep,
                                      void* out, void* workspace, size_t ws_bytes, void* stream,
                                      const dspark_attn_opts* opts);

/* dspark_mla_layer_fwd, once, while choosing the GEMM kernels: for each of
 * the block's projections every rocBLAS solution that applies to its shape
 * (and rocBLAS's default) is timed on `stream` -- which this call
 * synchronises, repeatedly -- and the fastest is written to *choices (host
 * memory, required).  Pass it back through dspark_attn_opts.gemm_choices to
 * dspark_mla_layer_fwd_ex calls of the same shapes on a device of the same
 * kind.  Without it rocBLAS chooses (for the o_proj shape of GLM-5.2 its
 * choice ran at half the fastest one's rate).  Same arguments and outputs as
 * dspark_mla_layer_fwd; takes seconds; must not run under stream capture. */
dspark_status dspark_mla_layer_tune(const dspark_layer_desc* desc,
                                    const void* h_draft, const void* h_ctx,
                                    const void* g_in, const void* w_qa, const void* g_qa,
                                    const void* w_qb, const void* w_kva, const void* g_kva,
                                    const void* w_uk, const void* w_uv, const void* w_o,
                                    const int32_t* anchors, const uint8_t* keep,
                                    void* out, void* workspace, size_t ws_bytes, void* stream,
                                    dspark_gemm_choices* choices);

/* Synchronises `stream`, then reads the status area of a workspace used by
 * the last dspark_mla_layer_fwd on it: DSPARK_OK, DSPARK_EANCHOR
 * (first_bad_block = b*N + n of the first kept block with an anchor outside
 * [0, S-2]) or DSPARK_ECAPACITY (more kept blocks than max_kept_blocks).
 * kept_blocks receives the number of kept blocks.  Either pointer may be
 * NULL. */
dspark_status dspark_mla_layer_read_status(const void* workspace, void* stream,
                                           int32_t* first_bad_block, int32_t* kept_blocks);

/* ---- the output head and the loss ------------------------------------
 * §5 "输出头" and §6 "训练目标" of the design page, for one batch:
 *   L_k = H^(L) W_lm^T + markov_w1[x_{A+k}] markov_w2^T   draft logits (row 5n+k of H^(L))
 *   T_k = z_{A+k} W_lm^T                                 teacher logits (same frozen lm_head)
 *   c_k = w_conf . [H^(L) row ; markov_w1[x_{A+k}]]      confidence logit
 *   ce  = -log softmax(L_k)[x_{A+k+1}]
 *   l1  = || softmax(L_k) - softmax(T_k) ||_1,   a = clip(1 - l1/2, 0, 1)
 *   bce = BCE-with-logits(c_k, a)
 * per step k = 0..4 of every block, and the loss
 *   alpha_ce mean(ce) + alpha_l1 mean(l1) + alpha_conf mean(bce)
 * with the means over the steps the eval mask keeps (§6 "eval_mask": step k
 * counts when A+k+1 < S, loss_mask[A+k+1] = 1 (loss_mask[S-1] read as 0) and
 * keep = 1, with a prefix cumprod along the block); 0 when no step counts.
 * Readings: the Markov head is a bigram bias -- step k's predecessor token
 * x_{A+k} (the anchor at k = 0, the gold token after) is embedded by
 * markov_w1 as a lookup table and mapped back by markov_w2; H^(L) is the
 * draft's final hidden state after its last RMSNorm. */
typedef struct dspark_loss_desc {
    int32_t B, S, N;          /* batch, sequence length, anchor blocks per sample */
    int32_t vocab;            /* V (154880 for GLM-5.2), >= 1 */
    int32_t hidden;           /* d (6144), >= 1 */
    int32_t markov_rank;      /* r (256), >= 1 */
    int32_t dtype;            /* dspark_dtype of H^(L), z and the weights */
    int32_t max_kept_blocks;  /* 0: B*N.  Otherwise an upper bound on the kept
                                 blocks of the batch */
    double alpha_ce, alpha_l1, alpha_conf;   /* 1, 0.9, 1 in the page's recipe */
    int32_t w_lm_ld;          /* elements between rows of w_lm (0: hidden) */
    int32_t w_m2_ld;          /* elements between rows of w_m2 (0: markov_rank) */
    int32_t max_counted_steps;/* 0: 5 * the block bound.  Otherwise an upper
                                 bound on the steps the eval mask counts.  The
                                 logits are formed for one row per counted
                                 step, at most this many rows (5 * max_kept_blocks
                                 when 0); more counted steps than rows is
                                 DSPARK_ECAPACITY */
} dspark_loss_desc;

/* Bytes of workspace dspark_loss_fwd needs (0 on an invalid descriptor):
 * a status area, the row <-> step maps, the gathered rows, the draft and
 * teacher logits in fp32 ([rows, V] each: 1.9 GB per 3132 rows of
 * V = 154880) and per-chunk softmax statistics.  256-byte aligned. */
size_t dspark_loss_workspace_size(const dspark_loss_desc* desc);

/* The output head and loss.  Device pointers:
 *   input_ids  [B, S] int32 in [0, V)     x (token ids of the Target prefill)
 *   loss_mask  [B, S] uint8               (loss_mask[S-1] is read as 0)
 *   anchors, keep  [B, N]                 as in dspark_attn_fwd
 *   h_final    [B, 5N, d]                 H^(L)
 *   z          [B, S, d]                  the Target's last hidden states
 *   w_lm       [V, d]                     frozen lm_head (row stride w_lm_ld)
 *   w_m1, w_m2 [V, r]                     markov_w1 (lookup, dense), markov_w2
 *                                         (row stride w_m2_ld)
 *   w_conf     [d + r]                    confidence head (H^(L) part first)
 *   terms      [4, B, N, 5] fp32 out      planes ce, l1, c (confidence
 *                                         logit), bce; 0 where the eval mask is 0
 *   eval_mask  [B, N, 5] uint8 out
 *   loss       [5] fp32 out               total, mean ce, mean l1, mean bce,
 *                                         number of counted steps
 * A kept block whose anchor lies outside [0, S-2] is an error detected on
 * the device: its terms are NaN, the loss is NaN and
 * dspark_loss_read_status reports DSPARK_EANCHOR.  Only the counted steps'
 * logits are formed (one compact row each).  More counted steps than the row
 * bound: every term and the loss are NaN and the status is
 * DSPARK_ECAPACITY.  The logits are fp32 (rocBLAS GEMMs with fp32
 * accumulation, no atomics: the same call gives the same bits);
 * softmax statistics, L1 and the sums are fp32, the final means fp64.
 * When lm_head and markov_w2 sit side by side in one [V, d + r] array
 * (w_m2 = w_lm + d, w_lm_ld = w_m2_ld = d + r), the draft and teacher logits
 * are one GEMM over [H^(L) | e] and [z | 0] with K = d + r; otherwise three
 * (the Markov bias, the draft lm_head accumulated onto it, the teacher's).
 * Uses the library's rocBLAS handle, working in the workspace's
 * DSPARK_BLAS_WORKSPACE_BYTES (see dspark_mla_layer_fwd). */
dspark_status dspark_loss_fwd(const dspark_loss_desc* desc, const int32_t* input_ids,
                              const uint8_t* loss_mask, const int32_t* anchors,
                              const uint8_t* keep, const void* h_final, const void* z,
                              const void* w_lm, const void* w_m1, const void* w_m2,
                              const void* w_conf, float* terms, uint8_t* eval_mask, float* loss,
                              void* workspace, size_t ws_bytes, void* stream);

/* dspark_loss_fwd with options (opts may be NULL): gemm_choices selects the
 * GEMM kernels; stage_events (at least 6) are recorded on `stream` before the
 * first launch and after each stage: the block index and row gather, the
 * logits GEMMs, the softmax statistics, the L1 pass, the per-step terms and
 * the loss.  The other fields are ignored. */
dspark_status dspark_loss_fwd_ex(const dspark_loss_desc* desc, const int32_t* input_ids,
                                 const uint8_t* loss_mask, const int32_t* anchors,
                                 const uint8_t* keep, const void* h_final, const void* z,
                                 const void* w_lm, const void* w_m1, const void* w_m2,
                                 const void* w_conf, float* terms, uint8_t* eval_mask,
                                 float* loss, void* workspace, size_t ws_bytes, void* stream,
                                 const dspark_attn_opts* opts);

/* dspark_loss_fwd, once, while choosing the GEMM kernels for its shapes and
 * writing them to *choices (as dspark_mla_layer_tune does; synchronises
 * `stream`, takes seconds). */
dspark_status dspark_loss_tune(const dspark_loss_desc* desc, const int32_t* input_ids,
                               const uint8_t* loss_mask, const int32_t* anchors,
                               const uint8_t* keep, const void* h_final, const void* z,
                               const void* w_lm, const void* w_m1, const void* w_m2,
                               const void* w_conf, float* terms, uint8_t* eval_mask, float* loss,
                               void* workspace, size_t ws_bytes, void* stream,
                               dspark_gemm_choices* choices);

/* Synchronises `stream`, then reads the status area of a workspace used by
 * the last dspark_loss_fwd on it: DSPARK_OK, DSPARK_EANCHOR (first_bad_block
 * = b*N + n of the first kept block with a bad anchor), DSPARK_ECAPACITY or
 * DSPARK_EINVAL (a token id outside [0, V)).  kept_blocks receives the
 * number of kept blocks with valid anchors, counted_steps the number of
 * steps the eval mask counts (a caller can size max_counted_steps from it).
 * Any pointer may be NULL. */
dspark_status dspark_loss_read_status(const void* workspace, void* stream,
                                      int32_t* first_bad_block, int32_t* kept_blocks,
                                      int32_t* counted_steps);

/* ---- inference-time drafting -------------------------------------------
 * The draft's KV cache (parameter summary, "KV cache"): at inference a draft
 * layer keeps about W cached tokens, c^KV (D numbers) and k^R (d_r numbers)
 * each.  Here each layer and sequence owns a ring of C slots,
 * cache_ckv [B, C, D] and cache_kr [B, C, d_r] (k^R not rotated); position
 * p lives in slot p mod C, so C >= window - 1 keeps every context position
 * a block can see. */
typedef struct dspark_decode_desc {
    dspark_attn_desc attn;   /* B sequences, N = 1, block 5, window, dims,
                                rope_base, softmax_scale, dtype; S is ignored */
    int32_t cache_slots;     /* C >= window - 1 */
} dspark_decode_desc;

/* Writes new context rows into the rings: row t < n_new[b] of
 * new_ckv [B, max_new, D] / new_kr [B, max_new, d_r] is position
 * pos0[b] + t (slot (pos0[b] + t) mod C).  When n_new[b] > C only its last C
 * rows are written (the earlier ones would be overwritten); rows at negative
 * positions are skipped.  pos0 and n_new are device arrays [B]. */
dspark_status dspark_cache_append(const dspark_decode_desc* desc, const int32_t* pos0,
                                  const int32_t* n_new, int32_t max_new, const void* new_ckv,
                                  const void* new_kr, void* cache_ckv, void* cache_kr,
                                  void* stream);

/* Bytes of workspace dspark_decode_attn needs (0 on an invalid descriptor):
 * the attention's workspace for B blocks (its status area first, so that
 * dspark_read_device_status works on this workspace) and each sequence's
 * window gathered from its ring.  256-byte aligned. */
size_t dspark_decode_workspace_size(const dspark_decode_desc* desc);

/* The draft attention for one block per sequence at decode time: the block
 * [x_A, MASK x 4] at positions A..A+4 (anchors [B], A >= 0) attends to the
 * context positions [max(0, A-W+1), A) held in the ring and to its own 5
 * positions, as dspark_attn_fwd does for a training block (§3, §4).
 *   q_nope [B, 5, H, d_c], q_rope [B, 5, H, d_r] (not rotated)
 *   ckv_blk [B, 5, D], kr_blk [B, 5, d_r]   the block's own latents
 *   w_uk, w_uv                              as in dspark_attn_fwd
 *   active [B] uint8                        0: the sequence's rows are 0
 *   out [B, 5, H, d_v]
 * The window is gathered into a short contiguous context and the training
 * attention runs on it with every position moved by the same offset
 * (A - min(A, W-1)); RoPE scores depend only on differences of positions,
 * so the result is the same.  A negative anchor on an active sequence is
 * reported by dspark_read_device_status (DSPARK_EANCHOR) with NaN rows. */
dspark_status dspark_decode_attn(const dspark_decode_desc* desc, const void* q_nope,
                                 const void* q_rope, const void* cache_ckv, const void* cache_kr,
                                 const void* ckv_blk, const void* kr_blk, const void* w_uk,
                                 const void* w_uv, const int32_t* anchors, const uint8_t* active,
                                 void* out, void* workspace, size_t ws_bytes, void* stream);

/* Verification of drafted tokens (the MTP / DSA explainer page,
 * "Rejection Sampling"; acceptance sum_v min(p_v, q_v)). */
typedef enum dspark_verify_mode {
    DSPARK_VERIFY_REJECTION = 0,   /* accept x_k when u_k < min(1, p_k(x_k) / q_k(x_k)) */
    DSPARK_VERIFY_TARGET_ONLY = 1  /* accept x_k when it is p_k's top choice */
} dspark_verify_mode;

typedef struct dspark_verify_desc {
    int32_t B;            /* sequences */
    int32_t K;            /* drafted tokens per sequence (5 for a DSpark block), >= 1 */
    int32_t vocab;        /* V >= 1 */
    int32_t mode;         /* a dspark_verify_mode */
    double temperature;   /* > 0: p = softmax(target / T), q = softmax(draft / T) */
} dspark_verify_desc;

/* Bytes of workspace dspark_spec_verify needs (0 on an invalid descriptor). */
size_t dspark_verify_workspace_size(const dspark_verify_desc* desc);

/* Verifies K drafted tokens per sequence.  Device pointers:
 *   draft_logits  [B, K, V] fp32      q_k
 *   target_logits [B, K+1, V] fp32    p_k (p_k scores the token after the
 *                                     k-th drafted position; p_K follows the last)
 *   draft_tokens  [B, K] int32        x_k in [0, V)
 *   uniforms      [B, K+1] fp32       u in [0, 1): u_k decides x_k, u_K draws
 *                                     the next token
 *   accept_prob   [B, K] fp32 out     a_k = min(1, p_k(x_k) / q_k(x_k))
 *   overlap       [B, K] fp32 out     sum_v min(p_k, q_k)
 *   n_accept      [B] int32 out       j = accepted drafted tokens (first rejection)
 *   next_token    [B] int32 out       rejection mode: drawn from the residual
 *                                     max(0, p_j - q_j) (from p_j if that is 0)
 *                                     when j < K, from p_K when j = K -- the
 *                                     first index whose cumulative weight
 *                                     exceeds u_K times the total; target-only
 *                                     mode: p_j's top choice (lowest index on ties)
 * A drafted token outside [0, V) makes that sequence's n_accept and
 * next_token -1.  Sums in fp32; no atomics. */
dspark_status dspark_spec_verify(const dspark_verify_desc* desc, const float* draft_logits,
                                 const float* target_logits, const int32_t* draft_tokens,
                                 const float* uniforms, float* accept_prob, float* overlap,
                                 int32_t* n_accept, int32_t* next_token, void* workspace,
                                 size_t ws_bytes, void* stream);

/* Synchronises `stream`, then reads the status area of a workspace used by
 * the last dspark_attn_fwd / dspark_attn_bwd / dspark_build_index on it.  Returns DSPARK_OK, or
 * DSPARK_EANCHOR with *first_bad_block = b*N + n of the first kept block
 * whose anchor was outside [0, S-2] (-1 when none); DSPARK_EINVAL after a
 * dspark_attn_bwd_ex with reuse_forward on a workspace that held no forward
 * of its descriptor and path (its gradients are NaN); DSPARK_EHIP after a
 * stalled one-launch forward.  first_bad_block may be NULL. */
dspark_status dspark_read_device_status(const void* workspace, void* stream,
                                        int32_t* first_bad_block);

/* Thread-local text of the last error on the calling thread ("" if none). */
const char* dspark_last_error(void);

/* DSPARK_ABI_VERSION of the loaded library. */
int32_t dspark_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_ATTN_H */
