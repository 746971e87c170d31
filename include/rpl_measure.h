/*
 * rpl_measure.h -- measurement helper of librpl.so, not a step of the method.
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
 */
#ifndef RPL_MEASURE_H
#define RPL_MEASURE_H

#include "rpl.h"

#ifdef __cplusplus
extern "C" {
#endif

rpl_status rpl_read_ceiling(const void *p, int64_t bytes, int32_t grid, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RPL_MEASURE_H */
