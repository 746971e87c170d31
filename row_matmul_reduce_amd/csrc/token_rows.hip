// token_rows.hip -- the token-row movement around the exchange in the
// FlashComm1 layout, on gfx950.  Both are HBM-bound copies of bf16 rows.
//
// xLLM pull request #1890, "feat: add FlashComm1 and MMRS fusion support for
// Qwen3.5 NPU", review thread (sequence pad/shard helpers): the M token rows
// are padded at the end to tp * M_c rows (M_c = ceil(M / tp)); rank r keeps the
// block of padded rows that starts at r * M_c; after the layer the blocks of
// all ranks are gathered in rank order and cut back to the first M rows.
//   shard:   out[i, :] = x[r * M_c + i, :] if r * M_c + i < M, else 0
//   gather:  out[i, :] = block[i / M_c][i mod M_c, :]            for i < M
// The shard writes the rank's block in one pass, so the padded copy that the
// helper makes first (a review comment asks whether it can be avoided) never
// exists.  On one GPU the gather is given every rank's block directly, as the
// reduce is given every rank's partial.
//
// One workgroup per output row (rows grid-strided); a thread moves up to 4
// 16-byte chunks of the row per pass, all loads issued before the stores.  The
// gather, which moves every token row, loads with streaming loads (see ld16_nt);
// the shard, one rank's block, with ordinary ones.
#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

constexpr int TR_U = 4;

template <bool NTL>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
token_rows_kernel(PartialPtrs src, int64_t ld, int rows_out, int n, int gather, int64_t row0, int m_src,
                  int m_chunk, uint16_t *__restrict__ out) {
    const int nch = n >> 3;
    for (int i = blockIdx.x; i < rows_out; i += gridDim.x) {
        const uint16_t *sp = nullptr;  // source row; null: a pad row (zeros)
        if (gather) {
            const int c = i / m_chunk;
            sp = src.p[c] + (int64_t)(i - c * m_chunk) * ld;
        } else if (row0 + i < m_src) {
            sp = src.p[0] + (row0 + i) * ld;
        }
        uint16_t *op = out + (int64_t)i * n;
        for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * TR_U) {
            u32x4 v[TR_U];
#pragma unroll
            for (int u = 0; u < TR_U; ++u) {
                const int c = c0 + u * 256;
                v[u] = (sp && c < nch) ? (NTL ? ld16_nt(sp + c * 8) : ld16(sp + c * 8)) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < TR_U; ++u) {
                const int c = c0 + u * 256;
                if (c < nch) st16_nt(op + c * 8, v[u]);
            }
        }
    }
}

static hipError_t launch_rows(const PartialPtrs &p, int64_t ld, int rows_out, int n, int gather, int64_t row0,
                              int m_src, int m_chunk, uint16_t *out, hipStream_t st) {
    const int grid = rows_out < 16384 ? rows_out : 16384;
    if (gather)
        hipLaunchKernelGGL(token_rows_kernel<true>, dim3(grid), dim3(256), 0, st, p, ld, rows_out, n, gather, row0,
                           m_src, m_chunk, out);
    else
        hipLaunchKernelGGL(token_rows_kernel<false>, dim3(grid), dim3(256), 0, st, p, ld, rows_out, n, gather, row0,
                           m_src, m_chunk, out);
    return hipGetLastError();
}

hipError_t launch_shard_rows(const uint16_t *x, int64_t ldx, int m, int n, int tp, int rank, uint16_t *out,
                             hipStream_t st) {
    const int mc = (m + tp - 1) / tp;
    PartialPtrs p{};
    p.p[0] = x;
    return launch_rows(p, ldx, mc, n, 0, (int64_t)rank * mc, m, mc, out, st);
}

hipError_t launch_gather_rows(const PartialPtrs &chunks, int m_chunk, int64_t ld, int m, int n, uint16_t *out,
                              hipStream_t st) {
    return launch_rows(chunks, ld, m, n, 1, 0, m, m_chunk, out, st);
}

}  // namespace rpl
