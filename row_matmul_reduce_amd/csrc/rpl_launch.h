// rpl_launch.h -- internal launchers of librpl (host side, not part of the ABI).
// Arguments reaching these functions have already been validated by rpl_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpl {

constexpr int MAX_TP = 16;

struct PartialPtrs {
    const uint16_t *p[MAX_TP];
};

hipError_t launch_partial_bf16(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *out,
                               int m, int m_pad, int n, int k, hipStream_t st);

hipError_t launch_partial_w8a8(const int8_t *xq, int64_t ldx, const float *sx, const int8_t *wq, int64_t ldw,
                               const float *sw, uint16_t *out, int32_t *acc, int m, int m_pad, int n, int k,
                               hipStream_t st);

hipError_t launch_reduce_rmsnorm(const PartialPtrs &p, int tp, int m_chunk, int n, const uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y, uint16_t *residual_out,
                                 hipStream_t st);

hipError_t launch_quant_per_token(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq, float *scale, int m,
                                  int k, hipStream_t st);

}  // namespace rpl
