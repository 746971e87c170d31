// gemm_w8a8.hip -- the w8a8 (int8 x int8) rank partial on gfx950.
//
// What it computes (xLLM pull request #1890, "feat: add FlashComm1 and MMRS
// fusion support for Qwen3.5 NPU", review thread on the w8a8_dynamic quant
// matmul of RowParallelLinear): int8 activation codes with one fp32 scale per
// token, int8 weight codes with a required fp32 scale per output channel; the
// integer product is accumulated exactly and dequantised to the bf16 partial.
//
// Same tile engine as the bf16 partial (gemm_nt.h): a K step stages 128 int8
// values per row, consumed by two v_mfma_i32_16x16x64_i8 per fragment pair
// with exact int32 accumulators.
// Epilogue, in this order and with no fused multiply-add:
//   out = bf16_rne( (float(acc) * x_scale[m]) * w_scale[n] )
// and, when requested, the int32 accumulators themselves.
#include "gemm_nt.h"
#include "rpl_launch.h"

namespace rpl {

struct W8a8Op {
    using Frag = i32x4;
    using Acc = i32x4;
    uint16_t *out;
    int32_t *acc_out;
    const float *sx;
    const float *sw;
    int m, n;
    __device__ static __forceinline__ Acc zero() { return Acc{0, 0, 0, 0}; }
    __device__ static __forceinline__ Acc mfma(Frag a, Frag b, Acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ void store(Acc v, int mrow, int ncol) const {
        const float s = mrow < m ? sx[mrow] : 0.0f;  // pad rows: acc is 0 and so is out
        float d[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float a = (float)v[t];             // v_cvt_f32_i32: nearest-even
            d[t] = __fmul_rn(__fmul_rn(a, s), sw[ncol + t]);
        }
        u32x2 p = {pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3])};
        st8(out + (int64_t)mrow * n + ncol, p);
        if (acc_out) st16(acc_out + (int64_t)mrow * n + ncol, __builtin_bit_cast(u32x4, v));
    }
};

template <int BM, int BN, int WM, int WN, bool PRIO, int PF, int SCHED>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * WM * WN, 64 * WM * WN)))
__attribute__((amdgpu_waves_per_eu((WM * WN + 3) / 4, (WM * WN + 3) / 4)))
gemm_w8a8_kernel(GemmShape g, W8a8Op op) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * (BM + BN) * KT_BYTES + PF_BYTES];
    gemm_nt_persistent<BM, BN, WM, WN, PRIO, PF, SCHED>(g, op, smem);
}

template <int BM, int BN, int WM, int WN, bool PRIO, int PF, int SCHED>
static hipError_t launch_w8a8(const GemmShape &g, const W8a8Op &op, hipStream_t st) {
    const int nt = ((g.m_pad + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, WM, WN, PRIO, PF, SCHED>), dim3(persistent_grid(nt)), dim3(64 * WM * WN), 0, st, g, op);
    return hipGetLastError();
}

hipError_t launch_partial_w8a8(const int8_t *xq, int64_t ldx, const float *sx, const int8_t *wq, int64_t ldw,
                               const float *sw, uint16_t *out, int32_t *acc, int m, int m_pad, int n, int k,
                               hipStream_t st) {
    GemmShape g{reinterpret_cast<const uint8_t *>(xq), reinterpret_cast<const uint8_t *>(wq), ldx, ldw, m, m_pad, n,
                k, 4};
    W8a8Op op{out, acc, sx, sw, m, n};
    if (pick_tile_n(m_pad, n) == 224) return launch_w8a8<256, 224, 4, 2, false, 3, 2>(g, op, st);
    return launch_w8a8<256, 256, 2, 4, true, 3, 3>(g, op, st);
}

}  // namespace rpl
