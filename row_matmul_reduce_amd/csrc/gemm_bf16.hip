// gemm_bf16.hip -- one tensor-parallel rank's bf16 partial product on gfx950.
//
// What it computes (vllm-ascend pull request #1926, "[Feature]: implement the
// fusion of allreduce and matmul in prefill phase when tp is enabled", PR
// description; xLLM pull request #1890, "feat: add FlashComm1 and MMRS fusion
// support for Qwen3.5 NPU", review thread on the RowParallelLinear MMRS path):
// the rank multiplies its activation shard [m, K_shard] by its weight shard
// stored [n, K_shard]; the result, rounded to bf16, is what the rank
// contributes to the cross-rank sum.  The output has M_pad = ceil(m/tp)*tp
// rows (the same pull request's sequence pad helper), so it is directly the
// reduce-scatter send layout [tp][M_pad/tp][n]; pad rows are zero.
//
// Two kernels:
//  * prefill: the four-wave form of the MFMA tile engine of gemm_nt.h
//    (256 x 224 tiles, operands DMA'd straight to LDS, double-buffered) with
//    v_mfma_f32_16x16x32_bf16 and fp32 accumulators in accumulation registers;
//  * decode (M_pad <= 16): the weight stream dominates (a few tokens against
//    the whole weight), so each workgroup owns 16 output columns, its waves
//    split K, every wave issues all of its weight loads before its first MFMA,
//    and the per-wave partial sums are added in LDS (no atomics: the result
//    is deterministic).
#include "gemm_nt.h"
#include "rpl_launch.h"

namespace rpl {

struct Bf16Op {
    using Frag = bf16x8;
    using Acc = f32x4;
    static constexpr bool STAGED = false;  // no per-row / per-column epilogue operands
    uint16_t *out;
    int n;
    __device__ static __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
    // MFMA with the accumulators held in accumulation registers
    __device__ static __forceinline__ void mfma_acc(Acc &c, Frag a, Frag b) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
    __device__ __forceinline__ void store(Acc v, int mrow, int ncol) const {
        u32x2 p = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        st8(out + (int64_t)mrow * n + ncol, p);
    }
};

template <int BN, int PF>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_wide_kernel(GemmShape g, uint16_t *out) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (256 + BN) * KT_BYTES + PF_BYTES];
    Bf16Op op{out, g.n};
    gemm_nt_wide<BN, PF>(g, op, smem);  // not staged: no staging area
}

// ---------------------------------------------------------------- decode path
constexpr int DEC_WAVES = 4;
constexpr int DEC_BATCH = 16;  // K steps (32 values each) whose loads are issued together

__global__ void __attribute__((amdgpu_flat_work_group_size(64 * DEC_WAVES, 64 * DEC_WAVES)))
gemm_bf16_decode_kernel(const uint16_t *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ w,
                        int64_t ldw, uint16_t *__restrict__ out, int m, int m_pad, int n, int k) {
    __shared__ f32x4 red[DEC_WAVES - 1][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int steps = (k + 31) / 32;
    const int per = (steps + DEC_WAVES - 1) / DEC_WAVES;
    const int s_begin = wave * per, s_end = min(steps, s_begin + per);

    const int r16 = lane & 15, g = lane >> 4;
    const int wrow = n0 + r16;
    const bool wrow_ok = wrow < n, xrow_ok = r16 < m;
    const uint16_t *wp = w + (int64_t)(wrow_ok ? wrow : 0) * ldw + g * 8;
    const uint16_t *xp = x + (int64_t)(xrow_ok ? r16 : 0) * ldx + g * 8;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_begin; s0 < s_end; s0 += DEC_BATCH) {
        u32x4 wf[DEC_BATCH], xf[DEC_BATCH];
#pragma unroll
        for (int j = 0; j < DEC_BATCH; ++j) {
            const int s = s0 + j;
            const int kel = s * 32 + g * 8;
            const bool live = s < s_end && kel < k;
            wf[j] = (live && wrow_ok) ? ld16(wp + s * 32) : u32x4{0, 0, 0, 0};
            xf[j] = (live && xrow_ok) ? ld16(xp + s * 32) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < DEC_BATCH; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j]),
                                                          __builtin_bit_cast(bf16x8, xf[j]), acc, 0, 0, 0);
    }
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int v = 0; v < DEC_WAVES - 1; ++v) acc += red[v][lane];
        const int mrow = r16, ncol = n0 + g * 4;
        if (mrow < m_pad && ncol < n) {
            u32x2 p = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
            st8(out + (int64_t)mrow * n + ncol, p);
        }
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_partial_bf16(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *out,
                               int m, int m_pad, int n, int k, hipStream_t st) {
    if (m_pad <= 16) {
        hipLaunchKernelGGL(gemm_bf16_decode_kernel, dim3((n + 15) / 16), dim3(64 * DEC_WAVES), 0, st, x, ldx, w,
                           ldw, out, m, m_pad, n, k);
        return hipGetLastError();
    }
    GemmShape g{reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(w),
                ldx * 2, ldw * 2, m, m_pad, n, k * 2, 4};
    const int nt = ((m_pad + 255) / 256) * ((n + 223) / 224);
    hipLaunchKernelGGL((gemm_bf16_wide_kernel<224, 3>), dim3(persistent_grid(nt)), dim3(256), 0, st, g, out);
    return hipGetLastError();
}

}  // namespace rpl
