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
struct SumsqPtrs {
    const float *p[MAX_TP];
};

hipError_t launch_partial_bf16(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *out,
                               int m, int m_pad, int n, int k, hipStream_t st);

hipError_t launch_partial_w8a8(const int8_t *xq, int64_t ldx, const float *sx, const int8_t *wq, int64_t ldw,
                               const float *sw, uint16_t *out, int32_t *acc, int m, int m_pad, int n, int k,
                               hipStream_t st);

hipError_t launch_reduce_rmsnorm(const PartialPtrs &p, int tp, int m_chunk, int n, const uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y, uint16_t *residual_out,
                                 hipStream_t st);

// The single-launch decode path (decode_fused.hip).  Workspace: a FD_WS_HEADER-byte header
// (bytes 8..11 the status word, 12..15 the poll bound, from 256 one 32-bit call count per
// workgroup), then the tagged hand-off slots, 8 bytes for two bf16 products each: [m][tp][n/2].
// The whole workspace is zero before its first use.
constexpr int FD_MAX_GRID = 1024;   // most workgroups of one launch (all resident at once)
constexpr int64_t FD_WS_HEADER = 256 + 4 * FD_MAX_GRID;
constexpr int64_t FD_MAX_N = 8192;  // row width one epilogue workgroup holds in registers
struct FusedDecodeArgs {
    const uint16_t *x[MAX_TP];  // per shard: [m_valid, k] rows, stride ldx
    const uint16_t *w[MAX_TP];  // per shard: [n, k], stride ldw
    int64_t ldx, ldw;
    int tp, m, m_valid, n, k;
    const uint16_t *residual, *gamma;
    float eps;
    uint16_t *y, *residual_out;
    unsigned *calls;                  // header bytes 256..: one call count per workgroup
    unsigned *status;                 // header bytes 8..11
    const unsigned *poll_limit;       // header bytes 12..15
    unsigned long long *p_slots;      // [m][tp][n / 2]
};
int64_t fused_decode_workspace_bytes(int64_t m, int64_t n, int64_t tp);
// The no-allocation form's hand-off memory: a static device array of this size, and its
// device address on the current device.
constexpr int64_t FD_SCRATCH_BYTES = int64_t(4) << 20;
hipError_t fused_decode_scratch(void **ptr);
hipError_t launch_decode_fused(const FusedDecodeArgs &a, hipStream_t st);

hipError_t launch_sum_partials(const PartialPtrs &p, int tp, int m, int n, int64_t ldp, uint16_t *out,
                               hipStream_t st);
hipError_t launch_shard_rows(const uint16_t *x, int64_t ldx, int m, int n, int tp, int rank, uint16_t *out,
                             hipStream_t st);
hipError_t launch_gather_rows(const PartialPtrs &chunks, int m_chunk, int64_t ld, int m, int n, uint16_t *out,
                              hipStream_t st);
hipError_t launch_slice_sumsq(const PartialPtrs &p, int tp, int m, int ns, int64_t ld, const uint16_t *residual,
                              uint16_t *residual_out, float *h, float *sumsq, hipStream_t st);
hipError_t launch_slice_apply(const float *h, const SumsqPtrs &s, int tp, int m, int ns, int n_total,
                              const uint16_t *gamma, float eps, uint16_t *y, int64_t ld, hipStream_t st);

hipError_t launch_quant_per_token(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq, float *scale, int m,
                                  int k, hipStream_t st);

}  // namespace rpl
