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
//    (256 x 224 or 256 x 256 tiles, operands DMA'd straight to LDS in rings of K steps) with
//    v_mfma_f32_16x16x32_bf16 and fp32 accumulators in accumulation registers; the
//    output goes out with streaming stores, so it does not sit dirty in the memory-side
//    cache when the chunk reduce streams its inputs;
//  * decode (M_pad <= 16): the weight stream dominates (a few tokens against
//    the whole weight), so each workgroup owns 16 output columns, its waves
//    split K, every wave issues all of its weight loads before its first MFMA,
//    and the per-wave partial sums are added in LDS (no atomics: the result
//    is deterministic).  With 8 or fewer rows one activation load carries
//    two (four) K steps, moved into place with row shifts between lanes.
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
    __device__ static __forceinline__ u32x2 pack(Acc v) { return u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}; }
    __device__ __forceinline__ void store(Acc v, int mrow, int ncol) const { st8_nt(out + (int64_t)mrow * n + ncol, pack(v)); }
    // 8 consecutive output columns
    __device__ __forceinline__ void store16(int mrow, int ncol, u32x4 v) const { st16_nt(out + (int64_t)mrow * n + ncol, v); }
    __device__ static __forceinline__ bool coalesced_final() { return true; }
};

template <int BN, int PF, bool KTAIL>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_bf16_wide_kernel(GemmShape g, uint16_t *out) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[wide_main_bytes(BN, false) + PF_BYTES];
    Bf16Op op{out, g.n};
    gemm_nt_wide<BN, PF, KTAIL>(g, op, smem);  // not staged: no staging area
}

// ---------------------------------------------------------------- decode path
constexpr int DEC_WAVES = 4;
constexpr int DEC_BATCH = 16;  // K steps (32 values each) whose loads are issued together

// XP: K steps per activation load.  The MFMA takes token row r from lanes r, r+16, r+32,
// r+48; with m_pad <= 16/XP rows the other lanes of a load would be idle, so lane row
// r16 loads token row r16 % (16/XP) of step s + r16 / (16/XP), and step s + q reads its
// fragment q*16/XP lanes down.  Output rows >= 16/XP then hold other steps' products;
// they are pad rows past m_pad and never stored.
template <int XP>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * DEC_WAVES, 64 * DEC_WAVES)))
gemm_bf16_decode_kernel(const uint16_t *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ w,
                        int64_t ldw, uint16_t *__restrict__ out, int m, int m_pad, int n, int k) {
    constexpr int XR = 16 / XP;  // token rows one load carries per step
    static_assert(DEC_BATCH % XP == 0, "whole activation loads per batch");
    __shared__ f32x4 red[DEC_WAVES - 1][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int steps = (k + 31) / 32;
    const int per = (steps + DEC_WAVES - 1) / DEC_WAVES;
    const int s_begin = wave * per, s_end = min(steps, s_begin + per);

    const int r16 = lane & 15, g = lane >> 4;
    const int wrow = n0 + r16;
    const int xrow = r16 % XR, xsub = r16 / XR;
    const bool wrow_ok = wrow < n, xrow_ok = xrow < m;
    const uint16_t *wp = w + (int64_t)(wrow_ok ? wrow : 0) * ldw + g * 8;
    const uint16_t *xp = x + (int64_t)(xrow_ok ? xrow : 0) * ldx + g * 8;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = s_begin; s0 < s_end; s0 += DEC_BATCH) {
        // The activation loads go first: they are few, and every MFMA needs one, so the
        // MFMAs can start as the weight loads arrive in order (5.44 -> 5.22 us on decode o_proj).
        u32x4 wf[DEC_BATCH], xf[DEC_BATCH / XP];
#pragma unroll
        for (int j = 0; j < DEC_BATCH / XP; ++j) {
            const int s = s0 + j * XP + xsub;
            const bool live = s < s_end && s * 32 + g * 8 < k;
            xf[j] = (live && xrow_ok) ? ld16(xp + s * 32) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < DEC_BATCH; ++j) {
            const int s = s0 + j;
            const bool live = s < s_end && s * 32 + g * 8 < k;
            wf[j] = (live && wrow_ok) ? ld16(wp + s * 32) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < DEC_BATCH; ++j) {
            u32x4 xv = xf[j / XP];
            if constexpr (XP == 2) {
                if (j % 2) xv = lanes_down<8>(xv);
            } else if constexpr (XP == 4) {
                if (j % 4 == 1) xv = lanes_down<4>(xv);
                if (j % 4 == 2) xv = lanes_down<8>(xv);
                if (j % 4 == 3) xv = lanes_down<12>(xv);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j]),
                                                          __builtin_bit_cast(bf16x8, xv), acc, 0, 0, 0);
        }
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
        const dim3 grid((n + 15) / 16), block(64 * DEC_WAVES);
        if (m_pad <= 4)
            hipLaunchKernelGGL(gemm_bf16_decode_kernel<4>, grid, block, 0, st, x, ldx, w, ldw, out, m, m_pad, n, k);
        else if (m_pad <= 8)
            hipLaunchKernelGGL(gemm_bf16_decode_kernel<2>, grid, block, 0, st, x, ldx, w, ldw, out, m, m_pad, n, k);
        else
            hipLaunchKernelGGL(gemm_bf16_decode_kernel<1>, grid, block, 0, st, x, ldx, w, ldw, out, m, m_pad, n, k);
        return hipGetLastError();
    }
    GemmShape g{reinterpret_cast<const uint8_t *>(x), reinterpret_cast<const uint8_t *>(w),
                ldx * 2, ldw * 2, m, m_pad, n, k * 2, 4};
    // Tile width: each round of tiles (one per CU) costs about the tile's width, so take the width
    // with the fewer rounds x width.  224 gives the prefill share 256 tiles (one round, where 256-wide
    // tiles would leave 32 CUs idle); 256 gives the long-prefill share exactly five rounds instead of
    // 5.75 (408 against 425 us on one box, bit-identical outputs).
    // The 256-wide form is used without a K tail only (its per-lane tail cuts would spill registers).
    const int tm = (m_pad + 255) / 256;
    const int nt224 = tm * ((n + 223) / 224), nt256 = tm * ((n + 255) / 256);
    const bool tail = g.kbytes % KT_BYTES;
    const bool wide256 =
        !tail && (int64_t)((nt256 + NUM_CU - 1) / NUM_CU) * 256 < (int64_t)((nt224 + NUM_CU - 1) / NUM_CU) * 224;
    if (wide256) {
        hipLaunchKernelGGL((gemm_bf16_wide_kernel<256, 3, false>), dim3(persistent_grid(nt256)), dim3(256), 0, st, g, out);
    } else {
        if (tail) hipLaunchKernelGGL((gemm_bf16_wide_kernel<224, 3, true>), dim3(persistent_grid(nt224)), dim3(256), 0, st, g, out);
        else hipLaunchKernelGGL((gemm_bf16_wide_kernel<224, 3, false>), dim3(persistent_grid(nt224)), dim3(256), 0, st, g, out);
    }
    return hipGetLastError();
}

}  // namespace rpl
