/*
 * rpl_measure.h -- measurement helpers of librpl.so, not steps of the method.
 *
 * rpl_read_ceiling -- reads `bytes` bytes at device pointer p once, with `grid`
 * workgroups of 256 threads in a grid-stride loop of 16-byte loads, and writes
 * nothing (sink, a device word, is written only if the folded data equal a fixed
 * 32-bit value: effectively never).  Timed like the decode-shaped kernels on the
 * same bytes, it gives the read rate a standalone launch of that size reaches on
 * the device, the practical ceiling for those kernels.  Asynchronous on stream.
 *
 * RPL_ERR_NULL        p or sink is NULL
 * RPL_ERR_INVALID     bytes < 16 or not a multiple of 16; grid < 1 or > 65536
 * RPL_ERR_UNSUPPORTED p not 16-byte aligned or sink not 4-byte aligned
 * RPL_ERR_LAUNCH      the launch failed
 *
 * rpl_mfma_ceiling -- matrix-core work alone: 256 workgroups of four waves (one per
 * CU, each wave alone on its SIMD), each lane holding its own 512 bytes of `ops` as
 * two sets of 16 MFMA operand fragments and a 128 x 128 wave tile of accumulators in
 * accumulation registers, issue iters x 128 MFMAs per wave, alternating the two
 * sets: v_mfma_f32_16x16x32_bf16 (kind 0, 16384 FLOP each) or v_mfma_i32_16x16x64_i8
 * (kind 1, 32768 OP each) -- the instructions of the bf16 and w8a8 partials.  One
 * launch does 256 * 4 * 128 * iters MFMAs.  Under the board's power cap the clock
 * depends on the operands' bit activity, so timed on random operands this is the
 * rate the card sustains on those instructions with real data, the practical ceiling
 * of the GEMM partials beside the published peak.  Asynchronous on stream.
 *
 * ops     device, at least RPL_MFMA_CEILING_OPS_BYTES bytes (lane g of the 65536
 *         reads bytes [512 g, 512 g + 512)), 16-byte aligned
 * clocks  device uint64[2 * 256]: for workgroup b, the shader-clock ticks
 *         (s_memtime) and the 100 MHz ticks (s_memrealtime) its first wave spent in
 *         the MFMA loop, so its clock is 100 MHz * clocks[2b] / clocks[2b+1];
 *         workgroup b runs on XCD b mod 8
 * sink    device word, written only if the folded accumulators equal a fixed value
 *
 * RPL_ERR_NULL        ops, clocks or sink is NULL
 * RPL_ERR_INVALID     ops_bytes < RPL_MFMA_CEILING_OPS_BYTES; kind not 0 or 1;
 *                     iters < 1 or > 2^20
 * RPL_ERR_UNSUPPORTED ops not 16-byte, clocks not 8-byte or sink not 4-byte aligned
 * RPL_ERR_LAUNCH      the launch failed
 */
#ifndef RPL_MEASURE_H
#define RPL_MEASURE_H

#include "rpl.h"

#ifdef __cplusplus
extern "C" {
#endif

rpl_status rpl_read_ceiling(const void *p, int64_t bytes, int32_t grid, uint32_t *sink, void *stream);

#define RPL_MFMA_CEILING_OPS_BYTES (256LL * 256 * 512)

rpl_status rpl_mfma_ceiling(const void *ops, int64_t ops_bytes, int32_t kind, int32_t iters, uint64_t *clocks,
                            uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RPL_MEASURE_H */
