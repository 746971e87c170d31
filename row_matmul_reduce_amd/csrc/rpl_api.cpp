// rpl_api.cpp -- the C ABI of librpl: host-side argument checks, then launch.
//
// Every check runs on the host, in the order of the status codes (NULL, then
// INVALID, then UNSUPPORTED), before any HIP call, so a rejected call touches
// neither the device nor the outputs.  This mirrors the fallback convention of
// the pages' fused operators: xLLM pull request #1890, "feat: add FlashComm1 and
// MMRS fusion support for Qwen3.5 NPU" ("MMRS Integration": unsupported inputs
// return nothing and the caller keeps its unfused matmul + reduce path), and the
// Dewu 910C blog's fused o_proj operator (communication-fusion section: a guard
// declines unsupported shapes so the unfused composition runs instead).
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "../../include/rpl.h"
#include "rpl_launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Operand row strides (bytes) must stay below 8 MiB: the tile engine addresses a
// 256-row tile with 32-bit buffer offsets.
constexpr int64_t kMaxLdBytes = int64_t(1) << 23;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [p, p + bytes) overlap?
bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

// Saturating arithmetic on non-negative sizes, so absurd arguments cannot overflow
// before they are rejected.
int64_t smul(int64_t a, int64_t b) {
    const __int128 r = (__int128)a * b;
    return r > INT64_MAX ? INT64_MAX : (int64_t)r;
}
int64_t sadd(int64_t a, int64_t b) { return a > INT64_MAX - b ? INT64_MAX : a + b; }

// Bytes spanned by a row-major [rows, cols] matrix with row stride ld elements.
int64_t span(int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
    return rows <= 0 ? 0 : smul(sadd(smul(rows - 1, ld), cols), esize);
}

int64_t padded_rows(int64_t m, int32_t tp) { return m > kMaxDim ? m : (m + tp - 1) / tp * tp; }

rpl_status launch_status(hipError_t e) { return e == hipSuccess ? RPL_OK : RPL_ERR_LAUNCH; }

}  // namespace

extern "C" {

rpl_status rpl_partial(const rpl_bf16 *x, int64_t ldx, const rpl_bf16 *w, int64_t ldw, rpl_bf16 *out, int64_t m,
                       int64_t n, int64_t k, int32_t tp, void *stream) {
    if (!w || (m != 0 && (!x || !out))) return RPL_ERR_NULL;
    if (m < 0 || n < 1 || k < 1 || tp < 1 || ldx < k || ldw < k) return RPL_ERR_INVALID;
    const int64_t m_pad = padded_rows(m, tp);
    const int64_t out_bytes = span(m_pad, n, n, 2);
    if (overlap(out, out_bytes, x, span(m, k, ldx, 2)) || overlap(out, out_bytes, w, span(n, k, ldw, 2)))
        return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || k % 8 || n % 8 || ldx % 8 || ldw % 8) return RPL_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(out, 16)) return RPL_ERR_UNSUPPORTED;
    if (m_pad > kMaxDim || n > kMaxDim || k > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (ldx * 2 >= kMaxLdBytes || ldw * 2 >= kMaxLdBytes) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    return launch_status(rpl::launch_partial_bf16(x, ldx, w, ldw, out, (int)m, (int)m_pad, (int)n, (int)k,
                                                  static_cast<hipStream_t>(stream)));
}

rpl_status rpl_reduce_chunk_rmsnorm(const rpl_bf16 *const *partials, int32_t tp, int64_t m_chunk, int64_t n,
                                    const rpl_bf16 *residual, const rpl_bf16 *gamma, float eps, rpl_bf16 *y,
                                    rpl_bf16 *residual_out, void *stream) {
    if (!partials || !gamma) return RPL_ERR_NULL;
    if (m_chunk != 0) {
        if (!residual || !y || !residual_out) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!partials[s]) return RPL_ERR_NULL;
    }
    if (tp < 1 || m_chunk < 0 || n < 1 || !(eps >= 0.0f) || !std::isfinite(eps)) return RPL_ERR_INVALID;
    const int64_t mat = span(m_chunk, n, n, 2);
    const int64_t gbytes = span(1, n, n, 2);
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    // y must not overlap any input nor residual_out.
    if (overlap(y, mat, residual, mat) || overlap(y, mat, gamma, gbytes) || overlap(y, mat, residual_out, mat))
        return RPL_ERR_INVALID;
    for (int s = 0; s < np; ++s)
        if (overlap(y, mat, partials[s], mat)) return RPL_ERR_INVALID;
    // residual_out may be exactly residual, but must not otherwise overlap an input.
    if (residual_out != residual && overlap(residual_out, mat, residual, mat)) return RPL_ERR_INVALID;
    if (overlap(residual_out, mat, gamma, gbytes)) return RPL_ERR_INVALID;
    for (int s = 0; s < np; ++s)
        if (overlap(residual_out, mat, partials[s], mat)) return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || n % 8 || n > 16384) return RPL_ERR_UNSUPPORTED;
    if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(y, 16) || !aligned(residual_out, 16))
        return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s)
        if (!aligned(partials[s], 16)) return RPL_ERR_UNSUPPORTED;
    if (m_chunk > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m_chunk == 0) return RPL_OK;
    rpl::PartialPtrs p{};
    for (int s = 0; s < tp; ++s) p.p[s] = partials[s];
    return launch_status(rpl::launch_reduce_rmsnorm(p, tp, (int)m_chunk, (int)n, residual, gamma, eps, y,
                                                    residual_out, static_cast<hipStream_t>(stream)));
}

rpl_status rpl_w8a8_partial(const int8_t *xq, int64_t ldx, const float *x_scale, const int8_t *wq, int64_t ldw,
                            const float *w_scale, rpl_bf16 *out, int32_t *acc, int64_t m, int64_t n, int64_t k,
                            int32_t tp, void *stream) {
    if (!wq || !w_scale || (m != 0 && (!xq || !x_scale || !out))) return RPL_ERR_NULL;
    if (m < 0 || n < 1 || k < 1 || tp < 1 || ldx < k || ldw < k) return RPL_ERR_INVALID;
    const int64_t m_pad = padded_rows(m, tp);
    const int64_t ob = span(m_pad, n, n, 2), ab = span(m_pad, n, n, 4);
    const int64_t xb = span(m, k, ldx, 1), wb = span(n, k, ldw, 1);
    if (overlap(out, ob, xq, xb) || overlap(out, ob, wq, wb) || overlap(out, ob, x_scale, span(1, m, m, 4)) ||
        overlap(out, ob, w_scale, span(1, n, n, 4)))
        return RPL_ERR_INVALID;
    if (acc && (overlap(acc, ab, out, ob) || overlap(acc, ab, xq, xb) || overlap(acc, ab, wq, wb) ||
                overlap(acc, ab, x_scale, span(1, m, m, 4)) || overlap(acc, ab, w_scale, span(1, n, n, 4))))
        return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || k % 16 || ldx % 16 || ldw % 16 || n % 8) return RPL_ERR_UNSUPPORTED;
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(out, 16) || (acc && !aligned(acc, 16)) ||
        !aligned(x_scale, 4) || !aligned(w_scale, 4))
        return RPL_ERR_UNSUPPORTED;
    if (m_pad > kMaxDim || n > kMaxDim || k > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (ldx >= kMaxLdBytes || ldw >= kMaxLdBytes) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    return launch_status(rpl::launch_partial_w8a8(xq, ldx, x_scale, wq, ldw, w_scale, out, acc, (int)m, (int)m_pad,
                                                  (int)n, (int)k, static_cast<hipStream_t>(stream)));
}

rpl_status rpl_sum_partials(const rpl_bf16 *const *partials, int32_t tp, int64_t m, int64_t n, int64_t ldp,
                            rpl_bf16 *out, void *stream) {
    if (!partials) return RPL_ERR_NULL;
    if (m != 0) {
        if (!out) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!partials[s]) return RPL_ERR_NULL;
    }
    if (tp < 1 || m < 0 || n < 1 || ldp < n) return RPL_ERR_INVALID;
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    const int64_t ob = span(m, n, n, 2), pb = span(m, n, ldp, 2);
    for (int s = 0; s < np; ++s)
        if (overlap(out, ob, partials[s], pb)) return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || n % 8 || ldp % 8 || !aligned(out, 16)) return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s)
        if (!aligned(partials[s], 16)) return RPL_ERR_UNSUPPORTED;
    if (m > kMaxDim || n > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    rpl::PartialPtrs p{};
    for (int s = 0; s < tp; ++s) p.p[s] = partials[s];
    return launch_status(rpl::launch_sum_partials(p, tp, (int)m, (int)n, ldp, out, static_cast<hipStream_t>(stream)));
}

rpl_status rpl_shard_rows(const rpl_bf16 *x, int64_t ldx, int64_t m, int64_t n, int32_t tp, int32_t rank,
                          rpl_bf16 *out, void *stream) {
    if (m > 0 && (!x || !out)) return RPL_ERR_NULL;
    if (m < 0 || n < 1 || tp < 1 || rank < 0 || rank >= tp || ldx < n) return RPL_ERR_INVALID;
    const int64_t mc = (m + tp - 1) / tp;
    if (m > 0 && overlap(out, span(mc, n, n, 2), x, span(m, n, ldx, 2))) return RPL_ERR_INVALID;
    if (n % 8 || ldx % 8 || !aligned(x, 16) || !aligned(out, 16)) return RPL_ERR_UNSUPPORTED;
    if (m > kMaxDim || n > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    return launch_status(rpl::launch_shard_rows(x, ldx, (int)m, (int)n, tp, rank, out,
                                                static_cast<hipStream_t>(stream)));
}

rpl_status rpl_gather_rows(const rpl_bf16 *const *chunks, int32_t tp, int64_t m_chunk, int64_t ld, int64_t m,
                           int64_t n, rpl_bf16 *out, void *stream) {
    if (!chunks) return RPL_ERR_NULL;
    if (m > 0) {
        if (!out) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!chunks[s]) return RPL_ERR_NULL;
    }
    if (tp < 1 || m_chunk < 0 || m < 0 || n < 1 || ld < n || m > (int64_t)tp * m_chunk) return RPL_ERR_INVALID;
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    const int64_t ob = span(m, n, n, 2), cb = span(m_chunk, n, ld, 2);
    for (int s = 0; s < np && m > 0; ++s)
        if (overlap(out, ob, chunks[s], cb)) return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || n % 8 || ld % 8 || (m > 0 && !aligned(out, 16))) return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp && m > 0; ++s)
        if (!aligned(chunks[s], 16)) return RPL_ERR_UNSUPPORTED;
    if (m_chunk > kMaxDim || n > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    rpl::PartialPtrs p{};
    for (int s = 0; s < tp; ++s) p.p[s] = chunks[s];
    return launch_status(rpl::launch_gather_rows(p, (int)m_chunk, ld, (int)m, (int)n, out,
                                                 static_cast<hipStream_t>(stream)));
}

rpl_status rpl_reduce_slice_sumsq(const rpl_bf16 *const *partials, int32_t tp, int64_t m, int64_t n_slice,
                                  int64_t ld, const rpl_bf16 *residual, rpl_bf16 *residual_out, float *h_out,
                                  float *sumsq, void *stream) {
    if (!partials) return RPL_ERR_NULL;
    if (m != 0) {
        if (!residual || !residual_out || !h_out || !sumsq) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!partials[s]) return RPL_ERR_NULL;
    }
    if (tp < 1 || m < 0 || n_slice < 1 || ld < n_slice) return RPL_ERR_INVALID;
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    const int64_t sl = span(m, n_slice, ld, 2), hb = span(m, n_slice, n_slice, 4), sb = span(1, m, m, 4);
    const void *outs[3] = {residual_out, h_out, sumsq};
    const int64_t osz[3] = {sl, hb, sb};
    for (int o = 0; o < 3; ++o) {
        if (o != 0 || residual_out != residual)
            if (overlap(outs[o], osz[o], residual, sl)) return RPL_ERR_INVALID;
        for (int s = 0; s < np; ++s)
            if (overlap(outs[o], osz[o], partials[s], sl)) return RPL_ERR_INVALID;
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], osz[o], outs[q], osz[q])) return RPL_ERR_INVALID;
    }
    if (tp > RPL_MAX_TP || n_slice % 8 || ld % 8 || n_slice > 16384) return RPL_ERR_UNSUPPORTED;
    if (!aligned(residual, 16) || !aligned(residual_out, 16) || !aligned(h_out, 16) || !aligned(sumsq, 4))
        return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s)
        if (!aligned(partials[s], 16)) return RPL_ERR_UNSUPPORTED;
    if (m > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    rpl::PartialPtrs p{};
    for (int s = 0; s < tp; ++s) p.p[s] = partials[s];
    return launch_status(rpl::launch_slice_sumsq(p, tp, (int)m, (int)n_slice, ld, residual, residual_out, h_out,
                                                 sumsq, static_cast<hipStream_t>(stream)));
}

rpl_status rpl_rmsnorm_slice_apply(const float *h, const float *const *sumsq_parts, int32_t tp, int64_t m,
                                   int64_t n_slice, int64_t n_total, const rpl_bf16 *gamma, float eps, rpl_bf16 *y,
                                   int64_t ld, void *stream) {
    if (!sumsq_parts || !gamma) return RPL_ERR_NULL;
    if (m != 0) {
        if (!h || !y) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!sumsq_parts[s]) return RPL_ERR_NULL;
    }
    if (tp < 1 || m < 0 || n_slice < 1 || ld < n_slice || n_total < n_slice || !(eps >= 0.0f) ||
        !std::isfinite(eps))
        return RPL_ERR_INVALID;
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    const int64_t yb = span(m, n_slice, ld, 2);
    if (overlap(y, yb, h, span(m, n_slice, n_slice, 4)) || overlap(y, yb, gamma, span(1, n_slice, n_slice, 2)))
        return RPL_ERR_INVALID;
    for (int s = 0; s < np; ++s)
        if (overlap(y, yb, sumsq_parts[s], span(1, m, m, 4))) return RPL_ERR_INVALID;
    if (tp > RPL_MAX_TP || n_slice % 8 || ld % 8 || n_slice > 16384) return RPL_ERR_UNSUPPORTED;
    if (!aligned(h, 16) || !aligned(gamma, 16) || !aligned(y, 16)) return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s)
        if (!aligned(sumsq_parts[s], 4)) return RPL_ERR_UNSUPPORTED;
    if (m > kMaxDim || n_total > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    rpl::SumsqPtrs sp{};
    for (int s = 0; s < tp; ++s) sp.p[s] = sumsq_parts[s];
    return launch_status(rpl::launch_slice_apply(h, sp, tp, (int)m, (int)n_slice, (int)n_total, gamma, eps, y, ld,
                                                 static_cast<hipStream_t>(stream)));
}

rpl_status rpl_quant_per_token(const rpl_bf16 *x, int64_t ldx, int8_t *xq, int64_t ldq, float *x_scale, int64_t m,
                               int64_t k, void *stream) {
    if (m != 0 && (!x || !xq || !x_scale)) return RPL_ERR_NULL;
    if (m < 0 || k < 1 || ldx < k || ldq < k) return RPL_ERR_INVALID;
    const int64_t xb = span(m, k, ldx, 2), qb = span(m, k, ldq, 1), sb = span(1, m, m, 4);
    if (overlap(xq, qb, x, xb) || overlap(x_scale, sb, x, xb) || overlap(xq, qb, x_scale, sb))
        return RPL_ERR_INVALID;
    if (k % 8 || ldx % 8 || ldq % 8) return RPL_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(x_scale, 4)) return RPL_ERR_UNSUPPORTED;
    if (m > kMaxDim || k > kMaxDim) return RPL_ERR_UNSUPPORTED;
    if (m == 0) return RPL_OK;
    return launch_status(rpl::launch_quant_per_token(x, ldx, xq, ldq, x_scale, (int)m, (int)k,
                                                     static_cast<hipStream_t>(stream)));
}

int64_t rpl_matmul_reduce_rmsnorm_workspace_size(int64_t m, int64_t n, int32_t tp) {
    if (m < 0 || n < 1 || tp < 1 || m > 64 || n > rpl::FD_MAX_N || tp > RPL_MAX_TP) return -1;
    return rpl::fused_decode_workspace_bytes(m, n, tp);
}

}  // extern "C"

namespace {

// Checks of the single-launch decode path shared by its two entry points (workspace != NULL:
// the caller's workspace of workspace_bytes; NULL: the library's static hand-off memory, which
// needs fused_decode_workspace_bytes <= FD_SCRATCH_BYTES).  Fills the kernel arguments except
// the hand-off pointers.
rpl_status fused_check(const rpl_bf16 *const *x_shards, int64_t ldx, const rpl_bf16 *const *w_shards, int64_t ldw,
                       int32_t tp, int64_t m, int64_t m_valid, int64_t n, int64_t k, const rpl_bf16 *residual,
                       const rpl_bf16 *gamma, float eps, rpl_bf16 *y, rpl_bf16 *residual_out, const void *workspace,
                       int64_t workspace_bytes, bool own_scratch, rpl::FusedDecodeArgs &a) {
    if (!x_shards || !w_shards || !gamma) return RPL_ERR_NULL;
    if (m != 0) {
        if (!residual || !y || !residual_out || (!own_scratch && !workspace)) return RPL_ERR_NULL;
        if (tp >= 1 && tp <= RPL_MAX_TP)
            for (int s = 0; s < tp; ++s)
                if (!w_shards[s] || (m_valid > 0 && !x_shards[s])) return RPL_ERR_NULL;
    }
    if (m < 0 || m_valid < 0 || m_valid > m || n < 1 || k < 1 || tp < 1 || ldx < k || ldw < k ||
        !(eps >= 0.0f) || !std::isfinite(eps))
        return RPL_ERR_INVALID;
    const int np = tp <= RPL_MAX_TP ? tp : 0;
    const int64_t mat = span(m, n, n, 2), gb = span(1, n, n, 2);
    const int64_t xb = span(m_valid, k, ldx, 2), wb = span(n, k, ldw, 2);
    const int64_t need = (m <= 64 && n <= rpl::FD_MAX_N && np) ? rpl::fused_decode_workspace_bytes(m, n, tp) : 0;
    if (!own_scratch && m != 0 && workspace_bytes < need) return RPL_ERR_INVALID;
    const int64_t wsb = own_scratch || workspace_bytes < 0 ? 0 : workspace_bytes;
    // outputs and workspace against the inputs and each other
    const void *outs[3] = {y, residual_out, workspace};
    const int64_t osz[3] = {mat, mat, wsb};
    for (int o = 0; o < 3; ++o) {
        if (o != 1 || residual_out != residual)
            if (overlap(outs[o], osz[o], residual, mat)) return RPL_ERR_INVALID;
        if (overlap(outs[o], osz[o], gamma, gb)) return RPL_ERR_INVALID;
        for (int s = 0; s < np; ++s)
            if (overlap(outs[o], osz[o], x_shards[s], xb) || overlap(outs[o], osz[o], w_shards[s], wb))
                return RPL_ERR_INVALID;
        for (int q = o + 1; q < 3; ++q)
            if (overlap(outs[o], osz[o], outs[q], osz[q])) return RPL_ERR_INVALID;
    }
    if (tp > RPL_MAX_TP || m > 64 || n > rpl::FD_MAX_N || n % 8 || k % 8 || ldx % 8 || ldw % 8)
        return RPL_ERR_UNSUPPORTED;
    if (own_scratch && need > rpl::FD_SCRATCH_BYTES) return RPL_ERR_UNSUPPORTED;
    if (!aligned(residual, 16) || !aligned(gamma, 16) || !aligned(y, 16) || !aligned(residual_out, 16) ||
        (!own_scratch && !aligned(workspace, 256)))
        return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s)
        if (!aligned(w_shards[s], 16) || !aligned(x_shards[s], 16)) return RPL_ERR_UNSUPPORTED;
    if (k > kMaxDim) return RPL_ERR_UNSUPPORTED;
    for (int s = 0; s < tp; ++s) {
        a.x[s] = x_shards[s];
        a.w[s] = w_shards[s];
    }
    a.ldx = ldx;
    a.ldw = ldw;
    a.tp = tp;
    a.m = (int)m;
    a.m_valid = (int)m_valid;
    a.n = (int)n;
    a.k = (int)k;
    a.residual = residual;
    a.gamma = gamma;
    a.eps = eps;
    a.y = y;
    a.residual_out = residual_out;
    return RPL_OK;
}

void fused_handoff(rpl::FusedDecodeArgs &a, void *mem) {
    uint8_t *ws = static_cast<uint8_t *>(mem);
    a.calls = reinterpret_cast<unsigned *>(ws + 256);
    a.status = reinterpret_cast<unsigned *>(ws + 8);
    a.poll_limit = reinterpret_cast<const unsigned *>(ws + 12);
    a.p_slots = reinterpret_cast<unsigned long long *>(ws + rpl::FD_WS_HEADER);
}

}  // namespace

extern "C" {

rpl_status rpl_matmul_reduce_rmsnorm(const rpl_bf16 *const *x_shards, int64_t ldx, const rpl_bf16 *const *w_shards,
                                     int64_t ldw, int32_t tp, int64_t m, int64_t m_valid, int64_t n, int64_t k,
                                     const rpl_bf16 *residual, const rpl_bf16 *gamma, float eps, rpl_bf16 *y,
                                     rpl_bf16 *residual_out, void *workspace, int64_t workspace_bytes,
                                     void *stream) {
    rpl::FusedDecodeArgs a{};
    const rpl_status st = fused_check(x_shards, ldx, w_shards, ldw, tp, m, m_valid, n, k, residual, gamma, eps, y,
                                      residual_out, workspace, workspace_bytes, false, a);
    if (st != RPL_OK || m == 0) return st;
    fused_handoff(a, workspace);
    return launch_status(rpl::launch_decode_fused(a, static_cast<hipStream_t>(stream)));
}

rpl_status rpl_matmul_reduce_rmsnorm_noalloc(const rpl_bf16 *const *x_shards, int64_t ldx,
                                             const rpl_bf16 *const *w_shards, int64_t ldw, int32_t tp, int64_t m,
                                             int64_t m_valid, int64_t n, int64_t k, const rpl_bf16 *residual,
                                             const rpl_bf16 *gamma, float eps, rpl_bf16 *y, rpl_bf16 *residual_out,
                                             void *stream) {
    rpl::FusedDecodeArgs a{};
    const rpl_status st = fused_check(x_shards, ldx, w_shards, ldw, tp, m, m_valid, n, k, residual, gamma, eps, y,
                                      residual_out, nullptr, 0, true, a);
    if (st != RPL_OK || m == 0) return st;
    void *mem = nullptr;
    if (rpl::fused_decode_scratch(&mem) != hipSuccess) return RPL_ERR_LAUNCH;
    fused_handoff(a, mem);
    return launch_status(rpl::launch_decode_fused(a, static_cast<hipStream_t>(stream)));
}

const char *rpl_status_string(rpl_status s) {
    switch (s) {
        case RPL_OK: return "RPL_OK";
        case RPL_ERR_NULL: return "RPL_ERR_NULL";
        case RPL_ERR_INVALID: return "RPL_ERR_INVALID";
        case RPL_ERR_UNSUPPORTED: return "RPL_ERR_UNSUPPORTED";
        case RPL_ERR_LAUNCH: return "RPL_ERR_LAUNCH";
    }
    return "unknown";
}

int32_t rpl_version(void) { return (2 << 16) | 2; }

}  // extern "C"
