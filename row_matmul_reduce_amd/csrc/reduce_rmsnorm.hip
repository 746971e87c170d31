// reduce_rmsnorm.hip -- the receiving rank's epilogue on gfx950: sum of all
// tensor-parallel partials for its token chunk, residual add, RMSNorm.
//
// What it computes (xLLM pull request #1890, "feat: add FlashComm1 and MMRS
// fusion support for Qwen3.5 NPU", Summary and review thread: the
// sequence-parallel reduction is a reduce-scatter over tokens and the residual
// add + RMSNorm run on the local chunk; Dewu tech blog
// "国产算力·昇腾 910C 大模型推理优化（下）：源码修改与算子优化", communication-
// fusion section: after the cross-rank sum the residual is added, that sum is
// the next residual, and RMSNorm takes the sum of squares, its reciprocal root
// and the weighted product):
//   h            = sum_s P_s[i, :] + residual[i, :]          (fp32 registers)
//   residual_out = bf16(h)
//   y            = bf16( gamma * h * rsqrt(mean(h^2) + eps) )
//
// HBM-bound: every byte is read or written once.  A row is owned by a team of
// RW wavefronts (ROWS rows per workgroup); lane t of the team holds 16-byte
// chunks t, t + 64*RW, ... of the row (CPL of them) in fp32 registers, so the row is read once, the sum of
// squares is a wavefront butterfly (plus an LDS exchange between the team's
// waves when RW > 1), and both outputs are written from registers.  All loads
// of a group of G partials (and the residual and gamma up front) are issued
// before any of them is consumed, so a row costs one or a few memory round
// trips instead of one per chunk.  The residual is read before either output
// is written, so residual_out may be the residual buffer itself.
#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// NT: streaming loads of the partials and the residual and streaming stores for both outputs
// (chunks of many rows; see ld16_nt and st16_nt).
template <int CPL, int RW, int ROWS, bool NT>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * RW * ROWS, 64 * RW * ROWS)))
reduce_rmsnorm_kernel(PartialPtrs P, int tp, int m_chunk, int n, const uint16_t *__restrict__ residual,
                      const uint16_t *__restrict__ gamma, float eps, uint16_t *y, uint16_t *residual_out) {
    constexpr int G = CPL <= 4 ? 4 : 2;     // partials whose loads are in flight together
    __shared__ float team_sum[RW * ROWS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * ROWS + wave / RW;
    const int t = (wave % RW) * 64 + lane;
    const int nch = n >> 3;
    const bool row_ok = row < m_chunk;      // RW > 1: the whole workgroup shares one row
    const int64_t rbase = (int64_t)row * n;

    float h[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) h[j][e] = 0.f;
    u32x4 rv[CPL], gv[CPL];
    if (row_ok) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = t + j * 64 * RW;
            rv[j] = c < nch ? (NT ? ld16_nt(residual + rbase + c * 8) : ld16(residual + rbase + c * 8))
                            : u32x4{0, 0, 0, 0};
            gv[j] = c < nch ? ld16(gamma + c * 8) : u32x4{0, 0, 0, 0};
        }
        for (int s0 = 0; s0 < tp; s0 += G) {
            u32x4 v[G][CPL];
#pragma unroll
            for (int q = 0; q < G; ++q)
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    const int c = t + j * 64 * RW;
                    const uint16_t *src = P.p[s0 + q] + rbase + c * 8;
                    v[q][j] = (s0 + q < tp && c < nch) ? (NT ? ld16_nt(src) : ld16(src)) : u32x4{0, 0, 0, 0};
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
    ss = wave_sum(ss);
    if (RW > 1) {
        if (lane == 0) team_sum[wave] = ss;
        __syncthreads();
        ss = 0.f;
        const int tb = (wave / RW) * RW;  // first wave of this row's team
#pragma unroll
        for (int v = 0; v < RW; ++v) ss += team_sum[tb + v];
    }
    if (!row_ok) return;
    const float inv = rsqrtf(ss / (float)n + eps);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        if (c < nch) {
            u32x4 yo, ro;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = h[j][2 * q], b = h[j][2 * q + 1];
                ro[q] = pack_bf16x2(a, b);
                yo[q] = pack_bf16x2(bf16_lo(gv[j][q]) * (a * inv), bf16_hi(gv[j][q]) * (b * inv));
            }
            if constexpr (NT) {
                st16_nt(residual_out + rbase + c * 8, ro);
                st16_nt(y + rbase + c * 8, yo);
            } else {
                st16(residual_out + rbase + c * 8, ro);
                st16(y + rbase + c * 8, yo);
            }
        }
    }
}

template <int CPL, int RW, bool NT, int ROWS = 4 / RW>
static hipError_t launch_rr(const PartialPtrs &p, int tp, int m_chunk, int n, const uint16_t *residual,
                            const uint16_t *gamma, float eps, uint16_t *y, uint16_t *ro, hipStream_t st) {
    hipLaunchKernelGGL((reduce_rmsnorm_kernel<CPL, RW, ROWS, NT>), dim3((m_chunk + ROWS - 1) / ROWS),
                       dim3(64 * RW * ROWS), 0, st, p, tp, m_chunk, n, residual, gamma, eps, y, ro);
    return hipGetLastError();
}

hipError_t launch_reduce_rmsnorm(const PartialPtrs &p, int tp, int m_chunk, int n, const uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y, uint16_t *ro, hipStream_t st) {
    // Few rows (decode steps): the kernel is one memory round trip long, so each row is
    // spread over 8 wavefronts (1-4 chunks per lane).  Many rows: one wavefront per row
    // (up to 8 chunks per lane, no cross-wave exchange), or 4 per row for rows wider than
    // 4096.  Measured on MI355X: decode chunk 3.8 -> 2.4 us, prefill chunk 15.1 -> 13.1 us.
    // The many-row layouts write with streaming stores (long-prefill chunk after its partial
    // product: 47 -> 43 us; prefill chunk 15.2 -> 14.2 us); the few-row one with ordinary ones.
    const int nch = n / 8;
#define RR(C, W, NT) \
    case C: return launch_rr<C, W, NT, 1>(p, tp, m_chunk, n, residual, gamma, eps, y, ro, st);
    if (m_chunk < 512) {
        switch ((nch + 511) / 512) { RR(1, 8, false) RR(2, 8, false) RR(3, 8, false) RR(4, 8, false) }
    } else if (nch <= 64 * 8) {
        switch ((nch + 63) / 64) {
            RR(1, 1, true) RR(2, 1, true) RR(3, 1, true) RR(4, 1, true)
            RR(5, 1, true) RR(6, 1, true) RR(7, 1, true) RR(8, 1, true)
        }
    } else {
        switch ((nch + 255) / 256) { RR(3, 4, true) RR(4, 4, true) RR(5, 4, true) RR(6, 4, true) RR(7, 4, true) RR(8, 4, true) }
    }
#undef RR
    return hipErrorInvalidValue;
}

}  // namespace rpl
