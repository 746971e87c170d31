// read_ceiling.hip -- a plain streaming read, for measurement only: what one
// standalone launch that does nothing but read a buffer achieves on this device.
// The decode-shaped kernels move a few MB per launch, where launch, first-touch
// latency and ramp-up keep any kernel well below the HBM peak; this kernel, timed
// on the same bytes and in the same way, gives the practical ceiling they are
// judged against.  It is not a step of the method.
//
// Each thread reads 16-byte chunks in a grid-stride loop, four loads in flight
// per iteration, and folds them into one word; the word is stored only if it
// equals a value the caller passes (never, in practice), so the loads cannot be
// dropped and nothing is written.
#include "../../include/rpl_measure.h"
#include "rpl_device.h"

namespace rpl {

__global__ void __launch_bounds__(256) read_ceiling_kernel(const u32x4 *__restrict__ p, int64_t chunks,
                                                           uint32_t never, uint32_t *sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (a[0] ^ b[1]) ^ (c[2] ^ d[3]);
    }
    for (; i < chunks; i += stride) acc ^= p[i][0];
    if (acc == never) sink[0] = acc;
}

}  // namespace rpl

extern "C" rpl_status rpl_read_ceiling(const void *p, int64_t bytes, int32_t grid, uint32_t *sink, void *stream) {
    if (!p || !sink) return RPL_ERR_NULL;
    if (bytes < 16 || bytes % 16 || grid < 1 || grid > 65536) return RPL_ERR_INVALID;
    if (reinterpret_cast<uintptr_t>(p) % 16 || reinterpret_cast<uintptr_t>(sink) % 4) return RPL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(rpl::read_ceiling_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const rpl::u32x4 *>(p), bytes / 16, 0x9E3779B9u, sink);
    return hipGetLastError() == hipSuccess ? RPL_OK : RPL_ERR_LAUNCH;
}
