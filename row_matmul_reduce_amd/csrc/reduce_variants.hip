// reduce_variants.hip -- the other two forms of the cross-rank reduction on
// gfx950, both HBM-bound streaming kernels.
//
// All-reduce form (vllm-ascend pull request #1926, "[Feature]: implement the
// fusion of allreduce and matmul in prefill phase when tp is enabled", PR
// description: RowParallelLinear's matmul fused with its all-reduce, after
// which every rank holds the sum over ranks for all token rows):
//   out[i, j] = bf16( sum_s P_s[i, j] )                               (fp32 sum)
//
// Hidden-split RMSNorm (Dewu tech blog "国产算力·昇腾 910C 大模型推理优化（下）：源码修改与
// 算子优化", communication-fusion section: after the reduce-add each rank takes
// the sum of squares of its own part, the parts are summed across ranks, then
// reciprocal root and normalisation).  Rank r owns a column slice of every row:
//   step 1: h = sum_s P_s[:, slice] + residual[:, slice]; residual_out = bf16(h);
//           h kept in fp32; sumsq[i] = sum over the slice of h[i, :]^2
//   step 2: ss[i] = sum_r sumsq_r[i];  y = bf16(gamma * h * rsqrt(ss / n + eps))
//
// Layout as the chunk epilogue: a row per team of RW wavefronts, lane t of the
// team holding 16-byte chunks t, t + 64*RW, ... (CPL of them); every load of a
// row is issued before any is consumed.
#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ------------------------------------------------------------- all-reduce sum
// Grid-stride over 16-byte chunks of the [m, n] result; all tp partial chunks of
// a lane are loaded before they are summed (in shard order).
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
sum_partials_kernel(PartialPtrs P, int tp, int m, int n, int64_t ldp, uint16_t *__restrict__ out) {
    const int nch = n >> 3;
    const int64_t total = (int64_t)m * nch;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < total; c += (int64_t)gridDim.x * 256) {
        const int64_t row = c / nch, col = (c - row * nch) * 8;
        float h[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < tp; s0 += 4) {
            u32x4 v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = s0 + q < tp ? ld16(P.p[s0 + q] + row * ldp + col) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[2 * e] += bf16_lo(v[q][e]);
                    h[2 * e + 1] += bf16_hi(v[q][e]);
                }
        }
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(h[2 * e], h[2 * e + 1]);
        st16(out + row * n + col, o);  // its consumer reads it next: ordinary stores keep it cached
    }
}

// ------------------------------------------------- hidden split, step 1
template <int CPL, int RW, int ROWS = 4 / RW, int G = 2>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * RW * ROWS, 64 * RW * ROWS)))
slice_sumsq_kernel(PartialPtrs P, int tp, int m, int ns, int64_t ld, const uint16_t *__restrict__ residual,
                   uint16_t *residual_out, float *__restrict__ hout, float *__restrict__ sumsq) {
    __shared__ float team_sum[RW * ROWS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * ROWS + wave / RW;
    const int t = (wave % RW) * 64 + lane;
    const int nch = ns >> 3;
    const bool row_ok = row < m;
    const int64_t rbase = (int64_t)row * ld;

    float h[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
    if (row_ok) {
        u32x4 rv[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = t + j * 64 * RW;
            rv[j] = c < nch ? ld16(residual + rbase + c * 8) : u32x4{0, 0, 0, 0};
        }
        for (int s0 = 0; s0 < tp; s0 += G) {
            u32x4 v[G][CPL];
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = t + j * 64 * RW;
                    v[q][j] = (s0 + q < tp && c < nch) ? ld16(P.p[s0 + q] + rbase + c * 8) : u32x4{0, 0, 0, 0};
                }
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int j = 0; j < CPL; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        h[j][2 * e] += bf16_lo(v[q][j][e]);
                        h[j][2 * e + 1] += bf16_hi(v[q][j][e]);
                    }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[j][2 * e] += bf16_lo(rv[j][e]);
                h[j][2 * e + 1] += bf16_hi(rv[j][e]);
            }
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += h[j][e] * h[j][e];
    ss = wave_sum_f(ss);
    if (RW > 1) {
        if (lane == 0) team_sum[wave] = ss;
        __syncthreads();
        ss = 0.f;
        const int tb = (wave / RW) * RW;
#pragma unroll
        for (int v = 0; v < RW; ++v) ss += team_sum[tb + v];
    }
    if (!row_ok) return;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        if (c < nch) {
            u32x4 ro;
#pragma unroll
            for (int q = 0; q < 4; ++q) ro[q] = pack_bf16x2(h[j][2 * q], h[j][2 * q + 1]);
            st16_nt(residual_out + rbase + c * 8, ro);
            float *hp = hout + (int64_t)row * ns + c * 8;
            *reinterpret_cast<f32x4 *>(hp) = f32x4{h[j][0], h[j][1], h[j][2], h[j][3]};
            *reinterpret_cast<f32x4 *>(hp + 4) = f32x4{h[j][4], h[j][5], h[j][6], h[j][7]};
        }
    }
    if (t == 0) sumsq[row] = ss;
}

// ------------------------------------------------- hidden split, step 2
// Same team layout; the row's factor is computed by every lane from the tp partial
// sums (tp loads of one cached word) before its chunks are scaled.
template <int CPL, int RW, int ROWS = 4 / RW>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * RW * ROWS, 64 * RW * ROWS)))
slice_apply_kernel(const float *__restrict__ hin, SumsqPtrs S, int tp, int m, int ns, int n_total,
                   const uint16_t *__restrict__ gamma, float eps, uint16_t *__restrict__ y, int64_t ld) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * ROWS + wave / RW;
    const int t = (wave % RW) * 64 + lane;
    const int nch = ns >> 3;
    if (row >= m) return;
    f32x4 hv[CPL][2];
    u32x4 gv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        if (c < nch) {
            const float *hp = hin + (int64_t)row * ns + c * 8;
            hv[j][0] = *reinterpret_cast<const f32x4 *>(hp);
            hv[j][1] = *reinterpret_cast<const f32x4 *>(hp + 4);
            gv[j] = ld16(gamma + c * 8);
        }
    }
    float ss = 0.f;
    for (int r = 0; r < tp; ++r) ss += S.p[r][row];
    const float inv = rsqrtf(ss / (float)n_total + eps);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        if (c < nch) {
            u32x4 yo;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float h0 = hv[j][q >> 1][(q & 1) * 2], h1 = hv[j][q >> 1][(q & 1) * 2 + 1];
                yo[q] = pack_bf16x2(bf16_lo(gv[j][q]) * (h0 * inv), bf16_hi(gv[j][q]) * (h1 * inv));
            }
            st16_nt(y + (int64_t)row * ld + c * 8, yo);
        }
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_sum_partials(const PartialPtrs &p, int tp, int m, int n, int64_t ldp, uint16_t *out,
                               hipStream_t st) {
    const int64_t chunks = (int64_t)m * (n / 8);
    const int64_t blocks = (chunks + 255) / 256;
    const int grid = (int)(blocks < 4 * 2048 ? blocks : 4 * 2048);
    hipLaunchKernelGGL(sum_partials_kernel, dim3(grid), dim3(256), 0, st, p, tp, m, n, ldp, out);
    return hipGetLastError();
}

// Team shape per slice width: the fewest waves per row that keep each lane at <= 4
// chunks, or 4 waves with up to 8 chunks (slices of at most 16384 columns).
#define RV_DISPATCH(LAUNCH)                                                      \
    const int nch = ns / 8;                                                      \
    if (nch <= 64 * 4) {                                                         \
        switch ((nch + 63) / 64) {                                               \
            LAUNCH(1, 1) LAUNCH(2, 1) LAUNCH(3, 1) LAUNCH(4, 1)                  \
        }                                                                        \
    } else if (nch <= 128 * 4) {                                                 \
        switch ((nch + 127) / 128) { LAUNCH(3, 2) LAUNCH(4, 2) }                 \
    } else {                                                                     \
        switch ((nch + 255) / 256) {                                             \
            LAUNCH(3, 4) LAUNCH(4, 4) LAUNCH(5, 4) LAUNCH(6, 4) LAUNCH(7, 4) LAUNCH(8, 4) \
        }                                                                        \
    }                                                                            \
    return hipErrorInvalidValue;

// Step 1 reads tp partials per chunk: more waves per row and fewer chunks per lane put
// every partial's load in flight at once (up to 256 chunks a row: one chunk per lane,
// all tp partials together).  Long-prefill slice (2048 x 640, 8 partials): 7.9 -> 6.9 us.
template <int C, int W>
static hipError_t launch_s1(const PartialPtrs &p, int tp, int m, int ns, int64_t ld, const uint16_t *residual,
                            uint16_t *residual_out, float *h, float *sumsq, hipStream_t st) {
    constexpr int ROWS = 4 / W, G = C <= 2 ? 8 : C <= 4 ? 4 : 2;
    hipLaunchKernelGGL((slice_sumsq_kernel<C, W, ROWS, G>), dim3((m + ROWS - 1) / ROWS), dim3(256), 0, st, p, tp, m,
                       ns, ld, residual, residual_out, h, sumsq);
    return hipGetLastError();
}

hipError_t launch_slice_sumsq(const PartialPtrs &p, int tp, int m, int ns, int64_t ld, const uint16_t *residual,
                              uint16_t *residual_out, float *h, float *sumsq, hipStream_t st) {
    const int nch = ns / 8;
    if (nch <= 64) return launch_s1<1, 1>(p, tp, m, ns, ld, residual, residual_out, h, sumsq, st);
    if (nch <= 128) return launch_s1<1, 2>(p, tp, m, ns, ld, residual, residual_out, h, sumsq, st);
    switch ((nch + 255) / 256) {
#define L1(C) \
    case C: return launch_s1<C, 4>(p, tp, m, ns, ld, residual, residual_out, h, sumsq, st);
        L1(1) L1(2) L1(3) L1(4) L1(5) L1(6) L1(7) L1(8)
#undef L1
    }
    return hipErrorInvalidValue;
}

hipError_t launch_slice_apply(const float *h, const SumsqPtrs &s, int tp, int m, int ns, int n_total,
                              const uint16_t *gamma, float eps, uint16_t *y, int64_t ld, hipStream_t st) {
#define L2(C, W)                                                                                           \
    case C:                                                                                                \
        hipLaunchKernelGGL((slice_apply_kernel<C, W>), dim3((m + 4 / W - 1) / (4 / W)), dim3(256), 0, st, h, s, tp, m, \
                           ns, n_total, gamma, eps, y, ld);                                                \
        return hipGetLastError();
    RV_DISPATCH(L2)
#undef L2
}
#undef RV_DISPATCH

}  // namespace rpl
