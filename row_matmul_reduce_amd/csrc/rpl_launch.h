// rpl_launch.h -- internal launchers of librpl (host side, not part of the ABI).
// Arguments reaching these functions have already been validated by rpl_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpl {

constexpr int MAX_TP = 16;
constexpr int NUM_CU = 256;  // MI355X compute units

struct PartialPtrs {
    const uint16_t *p[MAX_TP];
};

// Output tile width for the 256-row tile engine: 224 when it divides n and
// packs the grid into fewer/fuller waves of workgroups over the 256 CUs than
// 256 does, else 256.
inline int pick_tile_n(int m_pad, int n) {
    auto fill = [&](int bn) {
        const long tiles = (long)((m_pad + 255) / 256) * ((n + bn - 1) / bn);
        const long waves = (tiles + NUM_CU - 1) / NUM_CU;
        const double useful = (double)m_pad * n;
        return useful / ((double)waves * NUM_CU * 256.0 * bn);  // useful share of the issued tile waves
    };
    if (n % 224 == 0 && fill(224) > fill(256) + 1e-9) return 224;
    return 256;
}

hipError_t launch_partial_bf16(const uint16_t *x, int64_t ldx, const uint16_t *w, int64_t ldw, uint16_t *out,
                               int m, int m_pad, int n, int k, hipStream_t st);

hipError_t launch_partial_w8a8(const int8_t *xq, int64_t ldx, const float *sx, const int8_t *wq, int64_t ldw,
                               const float *sw, uint16_t *out, int32_t *acc, int m, int m_pad, int n, int k,
                               hipStream_t st);

hipError_t launch_reduce_rmsnorm(const PartialPtrs &p, int tp, int m_chunk, int n, const uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y, uint16_t *residual_out,
                                 hipStream_t st);

}  // namespace rpl
