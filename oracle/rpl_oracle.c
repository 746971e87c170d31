/*
 * rpl_oracle.c -- plain, slow, obviously correct CPU oracle for the row-parallel
 * matmul + reduce hot path.  TEST INFRASTRUCTURE ONLY: nothing on the product
 * path (the HIP library and its Python binding) may link, load or call this.
 * It shares no code, header or table with the HIP sources.
 *
 * Sources (web pages; cited by title and section):
 *   [FC1]  xLLM pull request #1890, "feat: add FlashComm1 and MMRS fusion support
 *          for Qwen3.5 NPU" -- the Summary, the "MMRS Integration" notes and the
 *          review thread's diff excerpts (RowParallelLinear MMRS output shape,
 *          sequence pad/shard helpers, w8a8_dynamic weight_scale requirement).
 *   [MMAR] vllm-ascend pull request #1926, "[Feature]: implement the fusion of
 *          allreduce and matmul in prefill phase when tp is enabled" -- the PR
 *          description (RowParallelLinear matmul fused with its all-reduce).
 *   [910C] Dewu tech blog, "国产算力·昇腾 910C 大模型推理优化（下）：源码修改与算子优化",
 *          section on communication fusion (the self-built 910C operator
 *          o_proj matmul + AllReduce + residual add + RMSNorm(1+w), and its
 *          unfused fallback composition matmul + all_reduce + add_rms_norm),
 *          and the "small ops" section (Gemma-style RMSNorm weight 1+w).
 *
 * What is computed is the UNFUSED composition the fused operators must equal
 * ([910C], fallback paragraph): a matmul per tensor-parallel rank over its
 * K-shard, the sum of those partials over ranks (all-reduce, or its
 * reduce-scatter restriction to one token chunk [FC1]), then residual add and
 * RMSNorm.  Everything is in fp64 except where a reading pins a precision.
 *
 * Readings taken where the pages leave a step open (each also listed in the
 * design notes):
 *   R1  a rank's partial is delivered as bfloat16, rounded to nearest-even from
 *       the exact (fp64) dot product -- one rounding;
 *   R2  the receiving rank sums the bf16 partials of all ranks (fp64 here);
 *   R3  h = sum + residual is NOT rounded before RMSNorm; only the new residual
 *       is rounded to bf16;
 *   R4  RMSNorm: y = gamma * h / sqrt(mean_n(h^2) + eps), mean over the full
 *       hidden size, eps inside the square root; gamma is a plain multiplier
 *       (pass 1+w for the Gemma form);
 *   R5  w8a8: exact integer dot product (int64 here, must fit int32), then the
 *       dequantisation (float(acc) * s_x[m]) * s_w[n] done as two fp32
 *       multiplies in that order, then bf16 round-to-nearest-even of the fp32;
 *   R6  per-token dynamic int8 quantisation of the activation: scale = row
 *       absmax / 127 in fp32, code = round-to-nearest-even of x / scale in fp32,
 *       clamped to [-127, 127]; an all-zero row has scale 0 and codes 0;
 *   R7  the 910C layout splits the hidden dimension over ranks: each rank
 *       reduces a column slice of every row and contributes the slice's sum of
 *       squares; the full-row sum is their cross-rank sum;
 *   R8  FC1 pad rows are zero and sit after the M real rows; the gathered
 *       chunks are cut back to their first M rows.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 * OpenMP only splits independent output rows across threads; every dot
 * product is a single sequential loop over k.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_OVERFLOW 2

/* ---------------------------------------------------------------- bf16 codec
 * bfloat16 = the top 16 bits of an IEEE binary32: 1 sign, 8 exponent, 7
 * fraction bits.  Decoding is exact.  Encoding from fp64 rounds ONCE, to
 * nearest, ties to even, with the bf16 quantum of the value's binade:
 *   normal  |v| in [2^e, 2^(e+1)), e >= -126: quantum 2^(e-7)
 *   subnormal |v| < 2^-126:                   quantum 2^-133
 * A result of 2^128 or more is infinity.                                    */

double orc_bf16_to_f64(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t f32_bits_hi(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

uint16_t orc_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    if (isinf(v)) return v > 0 ? 0x7F80 : 0xFF80;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    int e;
    (void)frexp(a, &e);           /* a = f * 2^e, f in [0.5, 1): binade exponent e-1 */
    int binade = e - 1;
    if (binade < -126) binade = -126;        /* subnormal range shares the 2^-133 quantum */
    double quantum = ldexp(1.0, binade - 7);
    double q = a / quantum;                  /* exact: division by a power of two */
    double r = nearbyint(q);                 /* default mode: nearest, ties to even */
    double res = r * quantum;                /* exact */
    if (res >= ldexp(1.0, 128)) return v > 0 ? 0x7F80 : 0xFF80;
    float f = (float)res;                    /* exact: res has <= 8 significant bits */
    uint16_t h = f32_bits_hi(f);
    return v < 0 ? (uint16_t)(h | 0x8000) : h;
}

uint16_t orc_f32_to_bf16(float v)
{
    return orc_f64_to_bf16((double)v);       /* a float is exact in fp64: one rounding */
}

/* ------------------------------------------------------------ partial (a2/a3)
 * [FC1] review thread, RowParallelLinear MMRS path: the rank's output has
 * padded_local_num_tokens rows per rank and weight.size(0) = N columns, the
 * weight being stored [N, K_shard] (nn.Linear layout); [MMAR] PR description:
 * RowParallelLinear computes the rank's matmul whose partial results are then
 * summed across tensor-parallel ranks.
 * [FC1] review thread, pad/shard helpers: the token count is padded up to a
 * multiple of the TP size by appending rows; the padded rows carry zeros, so
 * their products are zero.
 *
 * For each requested output row r (an index into the padded [M_pad, N] output):
 *     out[i, j] = bf16( sum_k x[r, k] * w[j, k] )   if r <  m
 *     out[i, j] = 0                                 if m <= r < M_pad
 * The sum is exact to fp64 rounding; when out_f64 != NULL the unrounded fp64
 * value is also returned (0 for pad rows).                                    */
int orc_partial_rows(const uint16_t *x, int64_t ldx,
                     const uint16_t *w, int64_t ldw,
                     int64_t m, int64_t n, int64_t k,
                     const int64_t *rows, int64_t nrows,
                     uint16_t *out, double *out_f64)
{
    if (!x || !w || !rows || (!out && !out_f64)) return ORC_ERR_ARG;
    if (m < 0 || n < 0 || k < 0 || ldx < k || ldw < k || nrows < 0) return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        if (r < 0) { bad = 1; continue; }
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            if (r < m) {
                const uint16_t *xr = x + r * ldx;
                const uint16_t *wr = w + j * ldw;
                for (int64_t kk = 0; kk < k; ++kk)
                    s += orc_bf16_to_f64(xr[kk]) * orc_bf16_to_f64(wr[kk]);
            }
            if (out) out[i * n + j] = orc_f64_to_bf16(s);
            if (out_f64) out_f64[i * n + j] = s;
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* -------------------------------------------- received chunk + epilogue (a4-a6)
 * [FC1] Summary and review thread: with sequence parallelism the reduction is a
 * reduce-scatter along tokens, rank r receiving chunk r = rows
 * [r*M_c, (r+1)*M_c) of the summed output; the residual is sharded the same way
 * and the add + RMSNorm run on the local rows only.
 * [910C] communication-fusion section: the epilogue after the cross-rank sum is
 * residual add, then RMSNorm computed as a sum of squares, its reciprocal root,
 * and the normalised, weighted output; the new residual is the pre-norm sum.
 *
 *   S[i, j]   = sum_s partials[s][i, j]                 (fp64, R2)
 *   h[i, j]   = S[i, j] + residual[i, j]                (fp64, R3)
 *   resid_out = bf16(h)
 *   ms[i]     = (1/n) sum_j h[i, j]^2
 *   y[i, j]   = bf16( gamma[j] * h[i, j] / sqrt(ms[i] + eps) )   (R4)
 * Optional fp64 outputs: h_f64 = h, y_f64 = the unrounded y.
 * partials[s] points to an [m_chunk, n] bf16 block with row stride ldp.       */
int orc_reduce_chunk_rmsnorm(const uint16_t *const *partials, int tp, int64_t ldp,
                             int64_t m_chunk, int64_t n,
                             const uint16_t *residual, const uint16_t *gamma, float eps,
                             uint16_t *y, uint16_t *residual_out,
                             double *h_f64, double *y_f64)
{
    if (!partials || !residual || !gamma || tp < 1 || m_chunk < 0 || n < 0 || ldp < n)
        return ORC_ERR_ARG;
    for (int s = 0; s < tp; ++s)
        if (!partials[s]) return ORC_ERR_ARG;
    if (!(eps >= 0.0f)) return ORC_ERR_ARG;
    const double deps = (double)eps;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m_chunk; ++i) {
        double sumsq = 0.0;
        /* first pass: h and its sum of squares */
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int s = 0; s < tp; ++s)
                acc += orc_bf16_to_f64(partials[s][i * ldp + j]);
            double h = acc + orc_bf16_to_f64(residual[i * n + j]);
            sumsq += h * h;
            if (residual_out) residual_out[i * n + j] = orc_f64_to_bf16(h);
            if (h_f64) h_f64[i * n + j] = h;
        }
        double ms = sumsq / (double)n;
        double denom = sqrt(ms + deps);
        /* second pass: normalise (h recomputed with the identical sum order) */
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int s = 0; s < tp; ++s)
                acc += orc_bf16_to_f64(partials[s][i * ldp + j]);
            double h = acc + orc_bf16_to_f64(residual[i * n + j]);
            double v = orc_bf16_to_f64(gamma[j]) * h / denom;
            if (y) y[i * n + j] = orc_f64_to_bf16(v);
            if (y_f64) y_f64[i * n + j] = v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ w8a8 partial (a7)
 * [FC1] review thread, w8a8_dynamic quant matmul: int8 activations with a
 * per-token dynamic scale, int8 weights with a required per-channel
 * weight_scale; the product is accumulated in integers and dequantised.
 *
 *   acc[i, j] = sum_k xq[r, k] * wq[j, k]        exact (int64), must fit int32
 *   out[i, j] = bf16( (float(acc) * sx[r]) * sw[j] )   two fp32 multiplies (R5)
 * Pad rows (m <= r < M_pad) give acc = 0 and out = 0.
 * Returns ORC_ERR_OVERFLOW if any accumulator leaves the int32 range.         */
int orc_w8a8_rows(const int8_t *xq, int64_t ldx, const float *sx,
                  const int8_t *wq, int64_t ldw, const float *sw,
                  int64_t m, int64_t n, int64_t k,
                  const int64_t *rows, int64_t nrows,
                  uint16_t *out, int32_t *acc)
{
    if (!xq || !sx || !wq || !sw || !rows || (!out && !acc)) return ORC_ERR_ARG;
    if (m < 0 || n < 0 || k < 0 || ldx < k || ldw < k || nrows < 0) return ORC_ERR_ARG;
    int bad = 0, ovf = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad, ovf)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows[i];
        if (r < 0) { bad = 1; continue; }
        for (int64_t j = 0; j < n; ++j) {
            int64_t s = 0;
            if (r < m) {
                const int8_t *xr = xq + r * ldx;
                const int8_t *wr = wq + j * ldw;
                for (int64_t kk = 0; kk < k; ++kk)
                    s += (int64_t)xr[kk] * (int64_t)wr[kk];
            }
            if (s > INT32_MAX || s < INT32_MIN) { ovf = 1; continue; }
            int32_t a32 = (int32_t)s;
            if (acc) acc[i * n + j] = a32;
            if (out) {
                volatile float t = (float)a32;            /* int -> fp32, nearest-even */
                volatile float u = t * ((r < m) ? sx[r] : 0.0f);
                volatile float v = u * sw[j];
                out[i * n + j] = orc_f32_to_bf16(v);
            }
        }
    }
    if (bad) return ORC_ERR_ARG;
    return ovf ? ORC_ERR_OVERFLOW : ORC_OK;
}

/* ------------------------------------------------- all-reduce form (sum only)
 * [MMAR] PR description: RowParallelLinear's matmul is fused with its
 * all-reduce, after which every rank holds the sum of all ranks' partials for
 * all token rows (no epilogue).  The partials travel as bf16 (R1) and the sum
 * is delivered as bf16:
 *   out[i, j] = bf16( sum_s partials[s][i * ldp + j] )      (fp64 sum)
 * When out_f64 != NULL the unrounded sum is returned too.                    */
int orc_sum_partials(const uint16_t *const *partials, int tp, int64_t ldp,
                     int64_t m, int64_t n, uint16_t *out, double *out_f64)
{
    if (!partials || tp < 1 || m < 0 || n < 0 || ldp < n || (!out && !out_f64)) return ORC_ERR_ARG;
    for (int s = 0; s < tp; ++s)
        if (!partials[s]) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int s = 0; s < tp; ++s)
                acc += orc_bf16_to_f64(partials[s][i * ldp + j]);
            if (out) out[i * n + j] = orc_f64_to_bf16(acc);
            if (out_f64) out_f64[i * n + j] = acc;
        }
    return ORC_OK;
}

/* --------------------------------------- hidden-split RMSNorm (910C layout)
 * [910C] communication-fusion section: after the cross-rank reduce-add each
 * rank computes the sum of squares of its own part of the row, the partial
 * sums are summed across ranks, then the reciprocal root and the normalised
 * output follow.  Reading R7: rank r owns the column slice [c0, c0 + n_slice)
 * of every row (the hidden dimension split over ranks), so
 *   step 1 (per rank):  h[i, j]      = sum_s P_s[i, c0 + j] + residual[i, c0 + j]
 *                       residual_out = bf16(h)
 *                       sumsq[i]     = sum_j h[i, j]^2            over the slice
 *   step 2 (all ranks): ss[i]        = sum_r sumsq_r[i]
 *                       y[i, j]      = bf16( gamma[c0 + j] * h[i, j] / sqrt(ss[i] / n + eps) )
 * with n the full hidden size.  Slices taken over all ranks give exactly the
 * token-chunk epilogue above up to fp64 summation order.
 * Step 1: partials[s] and residual point at the slice's first column (row stride
 * ld); residual_out likewise; h_f64 [m][n_slice] and sumsq [m] are outputs.    */
int orc_reduce_slice_sumsq(const uint16_t *const *partials, int tp, int64_t ld,
                           int64_t m, int64_t n_slice, const uint16_t *residual,
                           uint16_t *residual_out, double *h_f64, double *sumsq)
{
    if (!partials || tp < 1 || m < 0 || n_slice < 0 || ld < n_slice || !residual || !h_f64 || !sumsq)
        return ORC_ERR_ARG;
    for (int s = 0; s < tp; ++s)
        if (!partials[s]) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        double ss = 0.0;
        for (int64_t j = 0; j < n_slice; ++j) {
            double acc = 0.0;
            for (int s = 0; s < tp; ++s)
                acc += orc_bf16_to_f64(partials[s][i * ld + j]);
            double h = acc + orc_bf16_to_f64(residual[i * ld + j]);
            h_f64[i * n_slice + j] = h;
            if (residual_out) residual_out[i * ld + j] = orc_f64_to_bf16(h);
            ss += h * h;
        }
        sumsq[i] = ss;
    }
    return ORC_OK;
}

/* Step 2: sumsq_parts[r] are the tp ranks' per-row partial sums; gamma points at
 * the slice's first column; y has row stride ld.                            */
int orc_rmsnorm_slice_apply(const double *h_f64, const double *const *sumsq_parts, int tp,
                            int64_t m, int64_t n_slice, int64_t n_total,
                            const uint16_t *gamma, float eps, uint16_t *y, int64_t ld,
                            double *y_f64)
{
    if (!h_f64 || !sumsq_parts || tp < 1 || m < 0 || n_slice < 0 || n_total < 1 || !gamma ||
        !(eps >= 0.0f) || ld < n_slice || (!y && !y_f64))
        return ORC_ERR_ARG;
    for (int r = 0; r < tp; ++r)
        if (!sumsq_parts[r]) return ORC_ERR_ARG;
    const double deps = (double)eps;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i) {
        double ss = 0.0;
        for (int r = 0; r < tp; ++r) ss += sumsq_parts[r][i];
        const double denom = sqrt(ss / (double)n_total + deps);
        for (int64_t j = 0; j < n_slice; ++j) {
            double v = orc_bf16_to_f64(gamma[j]) * h_f64[i * n_slice + j] / denom;
            if (y) y[i * ld + j] = orc_f64_to_bf16(v);
            if (y_f64) y_f64[i * n_slice + j] = v;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------- per-token dynamic int8 quantiser
 * [FC1] review thread, RowParallelLinear forward: on the w8a8_dynamic path the
 * (already sequence-scattered) bf16 activation is quantised before the int8
 * matmul ("dynamic" = the activation scale is computed from the data at run
 * time, one scale per token row, while the weight carries a fixed per-channel
 * weight_scale).  The page names the step but not its arithmetic; reading R6:
 *
 *   amax[r] = max_k |x[r, k]|                       (exact: bf16 -> fp32)
 *   sx[r]   = amax[r] / 127                          one fp32 division, nearest-even
 *   xq[r,k] = clamp(rint(x[r,k] / sx[r]), -127, 127) fp32 division, then round to
 *                                                    the nearest integer, ties to even
 *   a row of zeros (amax = 0): sx = 0 and every code 0 (the quotient is undefined).
 *
 * Symmetric, so the int8 code -128 never occurs.  Codes are integers decided
 * in fp32, the precision the reading fixes, so both this oracle and the GPU
 * take the same decision.  Inputs must be finite.                            */
int orc_quant_per_token(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                        int8_t *xq, int64_t ldq, float *sx)
{
    if (!x || !xq || !sx) return ORC_ERR_ARG;
    if (m < 0 || k < 0 || ldx < k || ldq < k) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < m; ++r) {
        const uint16_t *xr = x + r * ldx;
        float amax = 0.0f;
        for (int64_t kk = 0; kk < k; ++kk) {
            float a = fabsf((float)orc_bf16_to_f64(xr[kk]));   /* exact */
            if (a > amax) amax = a;
        }
        volatile float s = amax / 127.0f;
        sx[r] = s;
        for (int64_t kk = 0; kk < k; ++kk) {
            int8_t q = 0;
            if (amax > 0.0f) {
                volatile float t = (float)orc_bf16_to_f64(xr[kk]) / s;
                float v = nearbyintf(t);                        /* ties to even */
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                q = (int8_t)v;
            }
            xq[r * ldq + kk] = q;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------- token rows around the exchange
 * [FC1] review thread, sequence pad/shard helpers: the M token rows are padded
 * with rows at the end to M_pad = tp * M_c, M_c = ceil(M / tp); rank r keeps the
 * contiguous block of padded rows starting at r * M_c; after the layer every
 * rank's block is gathered in rank order and the gathered rows are cut back to
 * the first M.  Reading R8: the pad rows are zero (they stand for tokens that
 * do not exist), and the cut keeps rows 0 .. M-1 of the gathered rows.
 *   shard:  out[i, :] = x[r * M_c + i, :]  if r * M_c + i < M,  else 0
 *   gather: out[i, :] = chunk[i / M_c][i mod M_c, :]            for i < M
 * Both only move bf16 bit patterns.                                          */
int orc_shard_rows(const uint16_t *x, int64_t ldx, int64_t m, int64_t n, int tp, int rank,
                   uint16_t *out)
{
    if (tp < 1 || rank < 0 || rank >= tp || m < 0 || n < 0 || ldx < n) return ORC_ERR_ARG;
    const int64_t mc = (m + tp - 1) / tp;
    if (mc > 0 && (!out || (m > 0 && !x))) return ORC_ERR_ARG;
    for (int64_t i = 0; i < mc; ++i) {
        const int64_t src = (int64_t)rank * mc + i;  /* row of the padded rows */
        for (int64_t j = 0; j < n; ++j)
            out[i * n + j] = src < m ? x[src * ldx + j] : (uint16_t)0;
    }
    return ORC_OK;
}

int orc_gather_rows(const uint16_t *const *chunks, int tp, int64_t m_chunk, int64_t ld,
                    int64_t m, int64_t n, uint16_t *out)
{
    if (!chunks || tp < 1 || m_chunk < 0 || m < 0 || m > (int64_t)tp * m_chunk || n < 0 || ld < n)
        return ORC_ERR_ARG;
    if (m > 0 && !out) return ORC_ERR_ARG;
    for (int64_t i = 0; i < m; ++i) {
        const int64_t c = i / m_chunk, r = i % m_chunk;  /* rank c's row r */
        if (!chunks[c]) return ORC_ERR_ARG;
        for (int64_t j = 0; j < n; ++j) out[i * n + j] = chunks[c][r * ld + j];
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ plumbing */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int t)
{
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}
