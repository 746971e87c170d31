// mfma_ceiling.hip -- matrix-core work alone, for measurement only: what the card
// sustains on the partials' MFMA instruction when nothing else runs, with the operand
// data the caller supplies.  Under the board's power cap the clock (and so this rate)
// depends on how many operand bits toggle; timed on random operands it gives the
// practical ceiling the GEMM partials are judged against beside the published peak.
// It is not a step of the method.
//
// One workgroup of four waves per CU (256 workgroups, each wave alone on its SIMD, as in
// the tile engine).  Each lane holds two sets of 16 operand fragments (its own 512 bytes
// of `ops`) and 64 accumulator blocks in accumulation registers -- the engine's
// 128 x 128 wave tile -- and issues iters x 2 x 64 MFMAs, alternating the two sets so
// consecutive instructions see different data.  Each workgroup records the shader-clock
// ticks (s_memtime) and the 100 MHz ticks (s_memrealtime) its wave 0 spent in the loop,
// from which the host reads each workgroup's clock; workgroup b runs on XCD b mod 8.
#include "../../include/rpl_measure.h"
#include "rpl_device.h"

namespace rpl {

constexpr int MC_GRID = 256, MC_FRAGS = 32;

template <bool I8>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256))) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma_ceiling_kernel(const u32x4 *__restrict__ ops, int iters, uint64_t *__restrict__ clocks, uint32_t never,
                    uint32_t *__restrict__ sink) {
    const int64_t base = ((int64_t)blockIdx.x * 256 + threadIdx.x) * MC_FRAGS;
    u32x4 a[2][8], b[2][8];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[s][i] = ops[base + s * 16 + i];
            b[s][i] = ops[base + s * 16 + 8 + i];
        }
    f32x4 acc[8][8];  // the int8 form keeps int32 bits in the same registers
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            asm volatile("" : "+a"(acc[i][j]));
        }
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 64; ++i) {
                if constexpr (I8)
                    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc[i / 8][i % 8]) : "v"(b[s][i % 8]), "v"(a[s][i / 8]));
                else
                    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i / 8][i % 8]) : "v"(b[s][i % 8]), "v"(a[s][i / 8]));
            }
    }
    // the last eight MFMAs' results are read below: the wait states come after all of them
    // and before any read (the empty statements order the other seven behind the wait)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[7][7]));
#pragma unroll
    for (int j = 0; j < 7; ++j) asm volatile("" : "+a"(acc[7][j]));
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint32_t fold = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) fold ^= __builtin_bit_cast(uint32_t, acc[i][j][0]);
    if (fold == never) sink[0] = fold;
    if (threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
}

}  // namespace rpl

extern "C" rpl_status rpl_mfma_ceiling(const void *ops, int64_t ops_bytes, int32_t kind, int32_t iters,
                                       uint64_t *clocks, uint32_t *sink, void *stream) {
    if (!ops || !clocks || !sink) return RPL_ERR_NULL;
    if (ops_bytes < RPL_MFMA_CEILING_OPS_BYTES || (kind != 0 && kind != 1) || iters < 1 || iters > (1 << 20))
        return RPL_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(ops) % 16 || reinterpret_cast<uintptr_t>(clocks) % 8 ||
        reinterpret_cast<uintptr_t>(sink) % 4)
        return RPL_ERR_UNSUPPORTED;
    const auto *p = static_cast<const rpl::u32x4 *>(ops);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 1)
        hipLaunchKernelGGL(rpl::mfma_ceiling_kernel<true>, dim3(rpl::MC_GRID), dim3(256), 0, st, p, iters, clocks,
                           0x9E3779B9u, sink);
    else
        hipLaunchKernelGGL(rpl::mfma_ceiling_kernel<false>, dim3(rpl::MC_GRID), dim3(256), 0, st, p, iters, clocks,
                           0x9E3779B9u, sink);
    return hipGetLastError() == hipSuccess ? RPL_OK : RPL_ERR_LAUNCH;
}
