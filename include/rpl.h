/*
 * rpl.h -- C ABI of the row-parallel matmul + reduce library (librpl.so),
 * native to AMD Instinct MI355X (gfx950).
 *
 * The library computes, on one GPU, one tensor-parallel rank's share of the
 * RowParallelLinear layer and the epilogue that the rank runs on the token
 * chunk it receives:
 *
 *   rpl_partial               bf16 partial product of the rank's K-shard, laid
 *                             out as reduce-scatter token chunks;
 *   rpl_reduce_chunk_rmsnorm  sum of all ranks' partials for one token chunk
 *                             (what a reduce-scatter delivers), residual add,
 *                             RMSNorm;
 *   rpl_w8a8_partial          the int8 x int8 (w8a8 dynamic-quant) variant of
 *                             the partial, dequantised to bf16;
 *
 * and around them the per-token quantiser, the single-launch decode path, the
 * all-reduce and hidden-split forms of the reduction, and the token-row
 * shard/gather of the FlashComm1 layout.
 *
 * Sources (web pages; cited by title and section):
 *   [FC1]  xLLM pull request #1890, "feat: add FlashComm1 and MMRS fusion support
 *          for Qwen3.5 NPU": Summary; "MMRS Integration"; review thread diff
 *          excerpts of RowParallelLinear and of the sequence pad/shard helpers.
 *   [MMAR] vllm-ascend pull request #1926, "[Feature]: implement the fusion of
 *          allreduce and matmul in prefill phase when tp is enabled": PR
 *          description.
 *   [910C] Dewu tech blog, "国产算力·昇腾 910C 大模型推理优化（下）：源码修改与算子优化",
 *          communication-fusion section (the 910C fused o_proj matmul +
 *          AllReduce + residual add + RMSNorm operator and its two-level
 *          fallback) and the "small ops" section (RMSNorm weight 1+w).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor pointers are DEVICE pointers, owned by the caller (for instance
 *    allocated by PyTorch).  The library allocates nothing, keeps no state
 *    between calls, never synchronises and never aborts.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  Calls on different streams are independent; calls whose
 *    buffers overlap must be ordered by the caller.
 *  - bfloat16 values travel as their 16-bit patterns (rpl_bf16).  Matrices are
 *    row-major; "ld" is a row stride in ELEMENTS.
 *  - Tensor-parallel padding follows [FC1] (review thread, pad/shard helpers):
 *    M tokens are padded to M_pad = ceil(M / tp) * tp rows and chunk c
 *    (the rows rank c receives) is rows [c * M_pad/tp, (c + 1) * M_pad/tp).
 *  - m == 0 (an empty batch) is valid: RPL_OK, nothing is enqueued, and the
 *    row-indexed pointers (activations, their scales, outputs, partials,
 *    residuals) may then be NULL; the layer's parameters (weights, weight
 *    scales, gamma) are always required.
 *  - Arguments are checked on the host, in the order of the status codes
 *    below, before any HIP call.  On any status other than RPL_OK the outputs
 *    are untouched (the fallback convention of [FC1] "MMRS Integration" and of
 *    the [910C] operator's guard: an unsupported call leaves the caller free to
 *    run the unfused composition instead).  Faults of an enqueued kernel, if
 *    any, surface at the caller's next synchronisation of the stream.
 */
#ifndef RPL_H
#define RPL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t rpl_bf16; /* bfloat16 bit pattern */

typedef enum {
    RPL_OK = 0,
    RPL_ERR_NULL = 1,        /* a required pointer is NULL                          */
    RPL_ERR_INVALID = 2,     /* bad size / stride / eps, or overlapping outputs     */
    RPL_ERR_UNSUPPORTED = 3, /* valid but outside what the kernels handle: see each */
    RPL_ERR_LAUNCH = 4       /* the HIP launch itself reported an error             */
} rpl_status;

/* Largest tensor-parallel degree accepted by every call. */
#define RPL_MAX_TP 16

/*
 * rpl_partial -- one rank's bf16 partial product over its K-shard.
 *
 * [FC1] review thread (RowParallelLinear MMRS path): the rank's input is
 * [tokens, K_shard], its weight is stored [N, K_shard] and the output has
 * N = weight.size(0) columns; [MMAR] PR description: the partials of all ranks
 * are summed (all-reduce) -- see rpl_reduce_chunk_rmsnorm.
 *
 *   out[r, j] = bf16_rne( sum_{k < K} x[r, k] * w[j, k] )   for r < m
 *   out[r, j] = 0                                           for m <= r < M_pad
 * accumulated in fp32 (any summation order), rounded once to bf16, nearest-even.
 *
 * x    [m, k] bf16, row stride ldx >= k     (the rank's activation shard)
 * w    [n, k] bf16, row stride ldw >= k     (nn.Linear weight shard, K-contiguous)
 * out  [M_pad, n] bf16, contiguous (row stride n) = [tp][M_pad/tp][n] chunks;
 *      must not overlap x or w
 * m >= 0 tokens; n >= 1; k >= 1; 1 <= tp <= RPL_MAX_TP.
 *
 * RPL_ERR_NULL        w is NULL, or m > 0 and x or out is NULL
 * RPL_ERR_INVALID     m < 0, n < 1, k < 1, tp < 1, ldx < k, ldw < k, out overlaps x/w
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; k, n, ldx or ldw not a multiple of 8;
 *                     any pointer not 16-byte aligned; m, n or k >= 2^31;
 *                     a row stride of 8 MiB or more (ldx or ldw >= 2^22)
 * RPL_ERR_LAUNCH      the kernel launch failed (e.g. no gfx950 device)
 */
rpl_status rpl_partial(const rpl_bf16 *x, int64_t ldx,
                       const rpl_bf16 *w, int64_t ldw,
                       rpl_bf16 *out,
                       int64_t m, int64_t n, int64_t k, int32_t tp,
                       void *stream);

/*
 * rpl_reduce_chunk_rmsnorm -- what rank c does with the token chunk it
 * receives: the sum of every rank's partial for that chunk, residual add,
 * RMSNorm.
 *
 * [FC1] Summary and review thread: with sequence parallelism the row-parallel
 * reduction is a reduce-scatter along tokens, the residual is sharded the same
 * way, and add + RMSNorm run on the local token chunk only.  [910C]
 * communication-fusion section: after the cross-rank sum, the residual is
 * added, the sum becomes the next residual, and RMSNorm takes the row's sum of
 * squares, its reciprocal root, and scales by the weight.  For the Gemma form
 * whose weight is 1+w ([910C] "small ops"), pass gamma = 1+w.
 *
 *   h[i, j]            = sum_{s < tp} partials[s][i, j] + residual[i, j]   (fp32)
 *   residual_out[i, j] = bf16_rne(h[i, j])
 *   y[i, j]            = bf16_rne( gamma[j] * h[i, j] / sqrt(mean_j(h[i, :]^2) + eps) )
 * h is not rounded before the norm.  With m_chunk = M_pad (tp partials of all
 * rows) this is the all-reduce form of [MMAR].
 *
 * partials      HOST array of tp DEVICE pointers, each -> [m_chunk, n] bf16,
 *               contiguous (rank s's chunk: &out_s[c * m_chunk * n])
 * residual      [m_chunk, n] bf16 contiguous
 * gamma         [n] bf16
 * eps           >= 0, finite (e.g. 1e-6)
 * y             [m_chunk, n] bf16; must not overlap any input or residual_out
 * residual_out  [m_chunk, n] bf16; may be exactly residual (in place), must
 *               not otherwise overlap an input
 *
 * RPL_ERR_NULL        partials or gamma is NULL, or m_chunk > 0 and residual,
 *                     y, residual_out or one of partials[0..tp-1] is NULL
 *                     (entries are read only for tp <= RPL_MAX_TP)
 * RPL_ERR_INVALID     tp < 1, m_chunk < 0, n < 1, eps < 0 or not finite,
 *                     y overlaps an input or residual_out, residual_out
 *                     partially overlaps residual or overlaps another input
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; n not a multiple of 8; n > 16384;
 *                     any pointer not 16-byte aligned; m_chunk >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_reduce_chunk_rmsnorm(const rpl_bf16 *const *partials, int32_t tp,
                                    int64_t m_chunk, int64_t n,
                                    const rpl_bf16 *residual,
                                    const rpl_bf16 *gamma, float eps,
                                    rpl_bf16 *y, rpl_bf16 *residual_out,
                                    void *stream);

/*
 * rpl_w8a8_partial -- the w8a8 (dynamic-quant) rank partial.
 *
 * [FC1] review thread (w8a8_dynamic quant matmul): int8 activations carry a
 * per-token scale, int8 weights a per-output-channel weight_scale, which is
 * required; the integer product is dequantised.
 *
 *   acc[r, j] = sum_{k < K} xq[r, k] * wq[j, k]                   (exact int32)
 *   out[r, j] = bf16_rne( (float(acc[r, j]) * x_scale[r]) * w_scale[j] )
 * with int -> fp32 nearest-even and two fp32 multiplies in exactly this order
 * (no fused multiply-add); rows m <= r < M_pad give acc = 0 and out = 0.
 * The caller guarantees |acc| < 2^31 (always true for k < 131072; with codes
 * in [-127, 127] for k <= 133143).
 *
 * xq       [m, k] int8, row stride ldx >= k
 * x_scale  [m] fp32 per-token scale
 * wq       [n, k] int8, row stride ldw >= k
 * w_scale  [n] fp32 per-channel scale (required)
 * out      [M_pad, n] bf16 contiguous, chunk layout as rpl_partial
 * acc      optional [M_pad, n] int32 contiguous (NULL = not stored)
 * out and acc must not overlap each other or any input.
 *
 * RPL_ERR_NULL        wq or w_scale is NULL, or m > 0 and xq, x_scale or out
 *                     is NULL
 * RPL_ERR_INVALID     m < 0, n < 1, k < 1, tp < 1, ldx < k, ldw < k, overlaps
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; k, ldx or ldw not a multiple of 16;
 *                     n not a multiple of 8; xq, wq, out, acc not 16-byte
 *                     aligned or scales not 4-byte aligned; m, n or k >= 2^31;
 *                     a row stride of 8 MiB or more (ldx or ldw >= 2^23)
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_w8a8_partial(const int8_t *xq, int64_t ldx, const float *x_scale,
                            const int8_t *wq, int64_t ldw, const float *w_scale,
                            rpl_bf16 *out, int32_t *acc,
                            int64_t m, int64_t n, int64_t k, int32_t tp,
                            void *stream);

/*
 * rpl_sum_partials -- the all-reduce form of the cross-rank sum (no epilogue).
 *
 * [MMAR] PR description: RowParallelLinear's matmul is fused with its
 * all-reduce, after which every rank holds the sum of all ranks' partials for
 * all token rows.  On one GPU the tp partials are given directly:
 *   out[i, j] = bf16_rne( sum_s partials[s][i, j] )        (fp32 sum, shard order)
 *
 * partials  HOST array of tp DEVICE pointers, each -> [m, n] bf16, row stride ldp
 * out       [m, n] bf16 contiguous; must not overlap a partial
 *
 * RPL_ERR_NULL        partials is NULL, or m > 0 and out or a partials[s] is NULL
 * RPL_ERR_INVALID     tp < 1, m < 0, n < 1, ldp < n, out overlaps a partial
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; n or ldp not a multiple of 8; pointers
 *                     not 16-byte aligned; m or n >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_sum_partials(const rpl_bf16 *const *partials, int32_t tp, int64_t m, int64_t n,
                            int64_t ldp, rpl_bf16 *out, void *stream);

/*
 * rpl_reduce_slice_sumsq / rpl_rmsnorm_slice_apply -- the hidden-split epilogue
 * of the 910C layout, where each rank owns a column slice of every token row.
 *
 * [910C] communication-fusion section: after the cross-rank reduce-add each
 * rank takes the sum of squares of its part of the row, those partial sums are
 * summed across ranks, then the reciprocal root and the normalised output.
 *
 * Step 1, rank r on its slice (columns c0 .. c0 + n_slice - 1):
 *   h[i, j]      = sum_s partials[s][i, j] + residual[i, j]     (fp32)
 *   residual_out = bf16_rne(h);   h_out[i, j] = h (fp32);   sumsq[i] = sum_j h[i, j]^2
 * partials[s], residual, residual_out point at the slice's first column of
 * [m, *] arrays with row stride ld; h_out [m, n_slice] fp32 contiguous; sumsq
 * [m] fp32.  residual_out may be exactly residual.
 *
 * Step 2, after the cross-rank sum (emulated here: the tp ranks' sumsq arrays
 * are summed by the kernel):
 *   ss[i] = sum_r sumsq_parts[r][i];   y[i, j] = bf16_rne(gamma[j] * h[i, j] / sqrt(ss[i] / n_total + eps))
 * h [m, n_slice] fp32 from step 1; gamma -> the slice's n_slice weights; y
 * points at the slice's first column, row stride ld; n_total is the full
 * hidden size.  Over all ranks' slices this equals rpl_reduce_chunk_rmsnorm's
 * outputs (to fp32 summation order).
 *
 * RPL_ERR_NULL        an array or required pointer is NULL (m > 0)
 * RPL_ERR_INVALID     tp < 1, m < 0, n_slice < 1, ld < n_slice, n_total < n_slice,
 *                     eps < 0 or not finite, an output overlaps an input or
 *                     another output (residual_out == residual allowed)
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; n_slice or ld not a multiple of 8;
 *                     n_slice > 16384; bf16 and fp32 row pointers not 16-byte
 *                     aligned (sumsq arrays: 4-byte); m >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_reduce_slice_sumsq(const rpl_bf16 *const *partials, int32_t tp, int64_t m,
                                  int64_t n_slice, int64_t ld, const rpl_bf16 *residual,
                                  rpl_bf16 *residual_out, float *h_out, float *sumsq,
                                  void *stream);

rpl_status rpl_rmsnorm_slice_apply(const float *h, const float *const *sumsq_parts, int32_t tp,
                                   int64_t m, int64_t n_slice, int64_t n_total,
                                   const rpl_bf16 *gamma, float eps, rpl_bf16 *y, int64_t ld,
                                   void *stream);

/*
 * rpl_quant_per_token -- per-token dynamic int8 quantisation of a bf16
 * activation, the producer of rpl_w8a8_partial's xq and x_scale.
 *
 * [FC1] review thread (RowParallelLinear forward on the w8a8_dynamic path):
 * the scattered activation is quantised at run time before the int8 matmul.
 * The page does not spell out the arithmetic; the symmetric per-row form is
 * used, with every operation in fp32:
 *   amax[r]    = max_k |x[r, k]|
 *   x_scale[r] = amax[r] / 127                       (IEEE division, nearest-even)
 *   xq[r, k]   = clamp(rint(x[r, k] / x_scale[r]), -127, 127)
 * rint rounds half to even; an all-zero row gets x_scale 0 and all codes 0.
 * Every code equals the one from the correctly rounded quotient x / x_scale,
 * so codes are exact functions of the input (the kernel may form the quotient
 * another way where that cannot change a code).  Inputs
 * must be finite: a row holding Inf or NaN gets unspecified codes and scale.
 *
 * x        [m, k] bf16, row stride ldx >= k
 * xq       [m, k] int8, row stride ldq >= k (columns k..ldq-1 are not written)
 * x_scale  [m] fp32
 * xq and x_scale must not overlap each other or x.
 *
 * RPL_ERR_NULL        m > 0 and x, xq or x_scale is NULL
 * RPL_ERR_INVALID     m < 0, k < 1, ldx < k, ldq < k, overlaps
 * RPL_ERR_UNSUPPORTED k, ldx or ldq not a multiple of 8; x or xq not 16-byte
 *                     aligned or x_scale not 4-byte aligned; m or k >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_quant_per_token(const rpl_bf16 *x, int64_t ldx,
                               int8_t *xq, int64_t ldq, float *x_scale,
                               int64_t m, int64_t k, void *stream);

/*
 * rpl_matmul_reduce_rmsnorm -- the whole path for a decode-sized block of token
 * rows in one launch: every shard's product, their sum, residual add, RMSNorm.
 *
 * [910C] communication-fusion section: one operator holds o_proj matmul +
 * AllReduce + residual add + RMSNorm for up to 40 rows (a decode step with
 * speculative tokens); its fallback is matmul + all_reduce + add_rms_norm.  On
 * one GPU all tp shards' products for the rows are computed in the same launch:
 *   P_s[i, j]    = bf16_rne( sum_k x_shards[s][i, k] * w_shards[s][j, k] )
 *                  (rows m_valid <= i < m are padding: P_s = 0)
 *   h[i, j]      = sum_s P_s[i, j] + residual[i, j]                (fp32)
 *   residual_out = bf16_rne(h);  y = bf16_rne(gamma * h / sqrt(mean_j h^2 + eps))
 * Each shard's product is rounded to bf16 before the sum, as a partial crossing
 * the wire would be, so the result equals rpl_partial per shard followed by
 * rpl_reduce_chunk_rmsnorm on these rows (within the bf16 rule: fp32 sums).
 * With the rows of one reduce-scatter chunk this is rank c's step; with all M
 * rows it is the all-reduce form of [MMAR] plus the epilogue.
 *
 * x_shards   HOST array of tp DEVICE pointers, each -> [m_valid, k] bf16 (shard
 *            s's activation rows of the block), row stride ldx >= k
 * w_shards   HOST array of tp DEVICE pointers, each -> [n, k] bf16, stride ldw >= k
 * residual   [m, n] bf16 contiguous; residual_out [m, n] bf16 (may be exactly
 *            residual); y [m, n] bf16; gamma [n] bf16; eps >= 0, finite
 * workspace  device buffer of at least
 *            rpl_matmul_reduce_rmsnorm_workspace_size(m, n, tp) bytes, 256-byte
 *            aligned, ZERO-FILLED before its first use; a call leaves it ready
 *            for the next one (nothing to reset).  It carries the shards'
 *            rounded products from the launch's product workgroups to its
 *            row workgroups, one call count per workgroup and, at byte offset 8, a 32-bit
 *            status word: 0, or nonzero once a workgroup of some call waited
 *            past its bound for another (the launch is cooperative, so every
 *            workgroup is resident and this does not happen in a correct launch;
 *            that call's y is then NaN).  The word at byte offset 12 bounds the
 *            waits in polls (0 = the default, about 2^22).  Calls that share a
 *            workspace must not overlap in time (same stream is fine).
 * y, residual_out and workspace must not overlap inputs or each other (except
 * residual_out == residual).
 *
 * RPL_ERR_NULL        m > 0 and a pointer (or an entry x_shards[s], w_shards[s],
 *                     s < tp <= RPL_MAX_TP) is NULL
 * RPL_ERR_INVALID     m < 0, m_valid < 0 or > m, n < 1, k < 1, tp < 1, ldx < k,
 *                     ldw < k, eps < 0 or not finite, workspace too small,
 *                     overlaps
 * RPL_ERR_UNSUPPORTED tp > RPL_MAX_TP; m > 64; n > 8192; n, k, ldx or ldw not a
 *                     multiple of 8; bf16 pointers not 16-byte aligned, workspace
 *                     not 256-byte aligned; k >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed, or the device cannot hold the
 *                     m row workgroups and one product workgroup at once
 *
 * rpl_matmul_reduce_rmsnorm_workspace_size returns the bytes for m rows, n
 * columns and tp shards (4 * m * tp * n plus a 4352-byte header), or -1
 * outside 0 <= m <= 64, 1 <= n <= 8192, 1 <= tp <= RPL_MAX_TP.
 */
int64_t rpl_matmul_reduce_rmsnorm_workspace_size(int64_t m, int64_t n, int32_t tp);

rpl_status rpl_matmul_reduce_rmsnorm(const rpl_bf16 *const *x_shards, int64_t ldx,
                                     const rpl_bf16 *const *w_shards, int64_t ldw,
                                     int32_t tp, int64_t m, int64_t m_valid,
                                     int64_t n, int64_t k,
                                     const rpl_bf16 *residual, const rpl_bf16 *gamma,
                                     float eps, rpl_bf16 *y, rpl_bf16 *residual_out,
                                     void *workspace, int64_t workspace_bytes,
                                     void *stream);

/*
 * rpl_matmul_reduce_rmsnorm_noalloc -- rpl_matmul_reduce_rmsnorm for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and checks
 * without the workspace: the hand-offs between the launch's workgroups use a
 * device array inside the library (4 MiB, each GPU the library runs on holds
 * its own copy until the process ends; it starts zero-filled and every call
 * leaves it ready for the next, so nothing needs clearing).  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine); the
 * caller passes the inputs and outputs.  All calls of this function on one GPU
 * share that GPU's array: calls that overlap in time on one GPU (on different
 * streams) race, so the caller must order them (one stream is enough).  Calls
 * of rpl_matmul_reduce_rmsnorm with their own workspaces do not touch it.
 *
 * RPL_ERR_UNSUPPORTED also when the hand-off memory the shape needs,
 *                     rpl_matmul_reduce_rmsnorm_workspace_size(m, n, tp),
 *                     exceeds 4 MiB (e.g. m = 8, n = 3584, tp = 2 needs
 *                     233,728 bytes; with m = 64, n * tp may be at most 16,367)
 * RPL_ERR_LAUNCH      also when the array's device address cannot be looked up
 *                     on the current device
 */
rpl_status rpl_matmul_reduce_rmsnorm_noalloc(const rpl_bf16 *const *x_shards, int64_t ldx,
                                             const rpl_bf16 *const *w_shards, int64_t ldw,
                                             int32_t tp, int64_t m, int64_t m_valid,
                                             int64_t n, int64_t k,
                                             const rpl_bf16 *residual, const rpl_bf16 *gamma,
                                             float eps, rpl_bf16 *y, rpl_bf16 *residual_out,
                                             void *stream);

/*
 * rpl_shard_rows / rpl_gather_rows -- the token-row movement around the
 * exchange in the FlashComm1 layout.
 *
 * [FC1] review thread (sequence pad/shard helpers): the M token rows are padded
 * at the end to M_pad = tp * M_c rows, M_c = ceil(M / tp); rank r keeps the
 * block of padded rows starting at r * M_c; after the layer all ranks' blocks
 * are gathered in rank order and cut back to the first M rows.  Pad rows are
 * zero.
 *
 * rpl_shard_rows:   out[i, :] = x[rank * M_c + i, :] if rank * M_c + i < m, else 0
 *   x    [m, n] bf16, row stride ldx >= n
 *   out  [M_c, n] bf16 contiguous, must not overlap x
 *   The rank's block is written in one pass, with no padded copy of x.
 *
 * rpl_gather_rows:  out[i, :] = chunks[i / m_chunk][i % m_chunk, :]   for i < m
 *   chunks  HOST array of tp DEVICE pointers, each -> [m_chunk, n] bf16 with
 *           row stride ld (on one GPU every rank's block is given directly)
 *   out     [m, n] bf16 contiguous, m <= tp * m_chunk (rows past m are the pad
 *           rows and are dropped); must not overlap a block
 *
 * RPL_ERR_NULL        shard: m > 0 and x or out is NULL; gather: chunks is
 *                     NULL, or m > 0 and out or a chunks[s] is NULL
 * RPL_ERR_INVALID     m < 0, n < 1, tp < 1, shard: rank outside [0, tp);
 *                     gather: m_chunk < 0 or m > tp * m_chunk; ld < n; overlaps
 * RPL_ERR_UNSUPPORTED n or the row stride not a multiple of 8; pointers not
 *                     16-byte aligned; gather: tp > RPL_MAX_TP; sizes >= 2^31
 * RPL_ERR_LAUNCH      the kernel launch failed
 */
rpl_status rpl_shard_rows(const rpl_bf16 *x, int64_t ldx, int64_t m, int64_t n, int32_t tp,
                          int32_t rank, rpl_bf16 *out, void *stream);

rpl_status rpl_gather_rows(const rpl_bf16 *const *chunks, int32_t tp, int64_t m_chunk, int64_t ld,
                           int64_t m, int64_t n, rpl_bf16 *out, void *stream);

/* Static, NUL-terminated name of a status code ("RPL_OK", ...; "unknown"). */
const char *rpl_status_string(rpl_status s);

/* Library ABI version: (major << 16) | minor.  Currently 2.2. */
int32_t rpl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RPL_H */
