// gemm_w8a8.hip -- the w8a8 (int8 x int8) rank partial on gfx950.
//
// What it computes (xLLM pull request #1890, "feat: add FlashComm1 and MMRS
// fusion support for Qwen3.5 NPU", review thread on the w8a8_dynamic quant
// matmul of RowParallelLinear): int8 activation codes with one fp32 scale per
// token, int8 weight codes with a required fp32 scale per output channel; the
// integer product is accumulated exactly and dequantised to the bf16 partial.
//
// Same four-wave tile engine as the bf16 partial (gemm_nt.h): a K step stages
// 128 int8 values per row, consumed by two v_mfma_i32_16x16x64_i8 per fragment
// pair with exact int32 accumulators in accumulation registers; the tile's token
// and channel scales are staged in LDS at the start of the tile.
// Epilogue, in this order and with no fused multiply-add:
//   out = bf16_rne( (float(acc) * x_scale[m]) * w_scale[n] )
// and, when requested, the int32 accumulators themselves.
#include "gemm_nt.h"
#include "rpl_launch.h"

namespace rpl {

struct W8a8Op {
    using Frag = i32x4;
    using Acc = i32x4;
    static constexpr bool STAGED = true;  // the engine stages the tile's scales in LDS
    uint16_t *out;
    int32_t *acc_out;
    const float *sx;
    const float *sw;
    int m, n;
    __device__ static __forceinline__ Acc zero() { return Acc{0, 0, 0, 0}; }
    // MFMA with the accumulators held in accumulation registers
    __device__ static __forceinline__ void mfma_acc(Acc &c, Frag a, Frag b) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    }
    // Dequantise and store 4 consecutive columns of one row, given that row's token scale
    // s (staged; 0 for pad rows, which read out of range) and the 4 channel scales w, in
    // the order of the definition (no fused multiply-add).
    __device__ __forceinline__ u32x2 pack_staged(Acc v, float s, f32x4 w) const {
        float d[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float a = (float)v[t];             // v_cvt_f32_i32: nearest-even
            d[t] = __fmul_rn(__fmul_rn(a, s), w[t]);
        }
        return u32x2{pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3])};
    }
    __device__ __forceinline__ void store_staged(Acc v, int mrow, int ncol, float s, f32x4 w) const {
        st8_nt(out + (int64_t)mrow * n + ncol, pack_staged(v, s, w));
        if (acc_out) st16_nt(acc_out + (int64_t)mrow * n + ncol, __builtin_bit_cast(u32x4, v));
    }
    // 8 consecutive bf16 output columns
    __device__ __forceinline__ void store16(int mrow, int ncol, u32x4 v) const { st16_nt(out + (int64_t)mrow * n + ncol, v); }
    // the last tile goes through LDS unless the int32 accumulators are stored as well
    __device__ __forceinline__ bool coalesced_final() const { return acc_out == nullptr; }
    // DMA the token scales of tile rows m0 .. m0+255 (wave 0) and the channel scales of
    // columns n0 .. n0+255 (wave 1) into LDS; entries past m or n read as zero.
    __device__ __forceinline__ void stage(float *rows, float *cols, int m0, int n0, int wave, int lane) const {
        if (wave > 1) return;
        const float *base = wave == 0 ? sx : sw;
        const int lim = wave == 0 ? m : n, o = wave == 0 ? m0 : n0;
        const uint32_t nrec = __builtin_amdgcn_readfirstlane(o < lim ? (uint32_t)(lim - o) * 4u : 0u);
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(base + (o < lim ? o : 0)), (short)0, (int)nrec, RSRC_DWORD3);
        float *dst = wave == 0 ? rows : cols;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + 64 * j), 4, (uint32_t)(lane + 64 * j) * 4u,
                                                     0, 0, 0);
    }
};

template <int BN, int PF, bool KTAIL>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_w8a8_wide_kernel(GemmShape g, W8a8Op op) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[wide_main_bytes(BN, true) + PF_BYTES + WIDE_STAGE_BYTES];
    gemm_nt_wide<BN, PF, KTAIL>(g, op, smem);
}

hipError_t launch_partial_w8a8(const int8_t *xq, int64_t ldx, const float *sx, const int8_t *wq, int64_t ldw,
                               const float *sw, uint16_t *out, int32_t *acc, int m, int m_pad, int n, int k,
                               hipStream_t st) {
    GemmShape g{reinterpret_cast<const uint8_t *>(xq), reinterpret_cast<const uint8_t *>(wq), ldx, ldw, m, m_pad, n,
                k, 4};
    W8a8Op op{out, acc, sx, sw, m, n};
    const int nt = ((m_pad + 255) / 256) * ((n + 223) / 224);
    if (g.kbytes % KT_BYTES)
        hipLaunchKernelGGL((gemm_w8a8_wide_kernel<224, 3, true>), dim3(persistent_grid(nt)), dim3(256), 0, st, g, op);
    else
        hipLaunchKernelGGL((gemm_w8a8_wide_kernel<224, 3, false>), dim3(persistent_grid(nt)), dim3(256), 0, st, g, op);
    return hipGetLastError();
}

}  // namespace rpl
