// quant_per_token.hip -- per-token dynamic int8 quantisation of a bf16
// activation on gfx950, the first step of the w8a8_dynamic row-parallel matmul.
//
// What it computes (xLLM pull request #1890, "feat: add FlashComm1 and MMRS
// fusion support for Qwen3.5 NPU", review thread: the RowParallelLinear forward
// quantises its scattered activation before the w8a8_dynamic int8 matmul, whose
// weight carries a per-channel weight_scale; the page names the step, not its
// arithmetic, and the reading taken is the symmetric per-row form):
//   amax[r]  = max_k |x[r, k]|
//   scale[r] = amax[r] / 127                          fp32 division, nearest-even
//   xq[r, k] = clamp(rint(x[r, k] / scale[r]), -127, 127)   fp32 division,
//              round half to even; an all-zero row gets scale 0 and codes 0.
// Codes are integers decided in fp32 and every code equals the one from the
// correctly rounded quotient (the quotient itself may differ from RN(x / scale)
// where |x / scale| < 1/4, whose code is 0 either way), so the codes are exact
// functions of the inputs.
//
// HBM-bound (2 bytes read, 1 byte written per element).  A row is owned by a
// team of RW wavefronts; lane t of the team keeps 16-byte chunks t, t + 64*RW,
// ... of the row (CPL of them) in registers, so the row is read once: absmax by
// a wavefront butterfly (plus an LDS exchange between the team's waves), then
// each chunk's 8 codes leave as one 8-byte store.  Rows longer than 2048 chunks
// take a two-pass kernel that reads the row again (from L2) to quantise it.
#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float chunk_absmax(u32x4 v, float a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) a = fmaxf(a, fmaxf(fabsf(bf16_lo(v[e])), fabsf(bf16_hi(v[e]))));
    return a;
}

// The row's divisor and how to divide by it.  The quotient x / scale must be
// the correctly rounded one.  A full IEEE division per element costs about ten
// VALU operations, so rows whose scale is comfortably normal use Markstein's
// correction step instead (P. Markstein, "Computation of elementary functions
// on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990): with
// y = RN(1/scale) (one IEEE division per row) and q0 = RN(x * y), which is
// within one ulp of x / scale, the remainder r = x - q0 * scale is exact in one
// FMA and RN(q0 + r * y) is exactly RN(x / scale), as long as nothing
// underflows.  With scale >= 2^-67 every quotient whose rounding can matter
// (|x / scale| >= 1/4) has x, q0, r well inside the normal range; smaller
// quotients round to code 0 either way.  A host replay of this arithmetic over
// every bf16 absmax >= 2^-60 and every bf16 |x| <= absmax (both signs, about
// 1e9 pairs) finds no code that differs from rint(RN(x / scale)).  Rows with a
// smaller scale (absmax below 2^-60) divide element by element.
struct RowDiv {
    float scale, recip;
    bool fast, zero;
};

__device__ __forceinline__ RowDiv row_div(float amax) {
    RowDiv d;
    d.scale = amax / 127.f;
    d.zero = !(amax > 0.f);
    d.fast = amax >= 0x1p-60f;
    d.recip = d.fast ? 1.f / d.scale : 0.f;
    return d;
}

template <bool FAST>
__device__ __forceinline__ uint32_t code_byte(float x, const RowDiv &d) {
    float t;
    if (FAST) {
        const float q0 = x * d.recip;
        const float r = __builtin_fmaf(-q0, d.scale, x);
        t = __builtin_fmaf(r, d.recip, q0);
    } else {
        t = x / d.scale;
    }
    const float q = fminf(fmaxf(__builtin_rintf(t), -127.f), 127.f);
    return (uint32_t)((int32_t)q) & 0xFFu;
}

// 8 bf16 values -> 8 int8 codes (byte e of the result = element e).
template <bool FAST>
__device__ __forceinline__ u32x2 quant_chunk(u32x4 v, const RowDiv &d) {
    u32x2 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t b0 = code_byte<FAST>(bf16_lo(v[2 * h]), d), b1 = code_byte<FAST>(bf16_hi(v[2 * h]), d);
        const uint32_t b2 = code_byte<FAST>(bf16_lo(v[2 * h + 1]), d);
        const uint32_t b3 = code_byte<FAST>(bf16_hi(v[2 * h + 1]), d);
        r[h] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    return r;
}

// Codes of CPL chunks held in registers; `d` is uniform over the row's team, so
// exactly one of the three branches runs.
template <int CPL>
__device__ __forceinline__ void quant_chunks(const u32x4 *v, const RowDiv &d, u32x2 *out) {
    if (d.zero) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) out[j] = u32x2{0u, 0u};
    } else if (d.fast) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) out[j] = quant_chunk<true>(v[j], d);
    } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) out[j] = quant_chunk<false>(v[j], d);
    }
}

template <int CPL, int RW, int ROWS>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * RW * ROWS, 64 * RW * ROWS)))
quant_rows_kernel(const uint16_t *__restrict__ x, int64_t ldx, int8_t *__restrict__ xq, int64_t ldq,
                  float *__restrict__ scale, int m, int k) {
    __shared__ float team_max[RW * ROWS];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * ROWS + wave / RW;
    const int t = (wave % RW) * 64 + lane;
    const int nch = k >> 3;
    const bool row_ok = row < m;  // RW > 1: the whole workgroup shares one row
    const uint16_t *xr = x + (int64_t)row * ldx;

    u32x4 v[CPL];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        v[j] = (row_ok && c < nch) ? ld16(xr + c * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) amax = chunk_absmax(v[j], amax);
    amax = wave_max(amax);
    if (RW > 1) {
        if (lane == 0) team_max[wave] = amax;
        __syncthreads();
        const int tb = (wave / RW) * RW;
        amax = team_max[tb];
#pragma unroll
        for (int q = 1; q < RW; ++q) amax = fmaxf(amax, team_max[tb + q]);
    }
    if (!row_ok) return;
    const RowDiv d = row_div(amax);
    int8_t *qr = xq + (int64_t)row * ldq;
    u32x2 codes[CPL];
    quant_chunks<CPL>(v, d, codes);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = t + j * 64 * RW;
        if (c < nch) st8(qr + c * 8, codes[j]);
    }
    if (t == 0) scale[row] = d.scale;
}

// Rows of more than 2048 chunks: one 256-thread workgroup per row, absmax pass,
// then a second pass over the (L2-resident) row that quantises and stores.
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256)))
quant_rows_long_kernel(const uint16_t *__restrict__ x, int64_t ldx, int8_t *__restrict__ xq, int64_t ldq,
                       float *__restrict__ scale, int m, int k) {
    constexpr int U = 4;  // chunks in flight per lane
    __shared__ float wmax[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x;
    const int nch = k >> 3;
    const uint16_t *xr = x + (int64_t)row * ldx;
    float amax = 0.f;
    for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 256;
            v[u] = c < nch ? ld16(xr + c * 8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) amax = chunk_absmax(v[u], amax);
    }
    amax = wave_max(amax);
    if (lane == 0) wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const RowDiv d = row_div(amax);
    int8_t *qr = xq + (int64_t)row * ldq;
    for (int c0 = threadIdx.x; c0 < nch; c0 += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 256;
            v[u] = c < nch ? ld16(xr + c * 8) : u32x4{0, 0, 0, 0};
        }
        u32x2 codes[U];
        quant_chunks<U>(v, d, codes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 256;
            if (c < nch) st8(qr + c * 8, codes[u]);
        }
    }
    if (threadIdx.x == 0) scale[row] = d.scale;
}

template <int CPL, int RW, int ROWS = 4 / RW>
static hipError_t launch_q(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq, float *scale, int m, int k,
                           hipStream_t st) {
    hipLaunchKernelGGL((quant_rows_kernel<CPL, RW, ROWS>), dim3((m + ROWS - 1) / ROWS), dim3(64 * RW * ROWS), 0, st,
                       x, ldx, xq, ldq, scale, m, k);
    return hipGetLastError();
}

hipError_t launch_quant_per_token(const uint16_t *x, int64_t ldx, int8_t *xq, int64_t ldq, float *scale, int m,
                                  int k, hipStream_t st) {
    // Few rows (decode steps): each row over 4 wavefronts, one row per workgroup, so the
    // rows spread over the CUs (8 rows of 1792: 2.6 -> 2.3 us).  Many rows: the fewest
    // wavefronts per row that keep each lane at <= 4 chunks, or 4 wavefronts with up to
    // 8 chunks; longer rows take the two-pass kernel.
    const int nch = k / 8;
#define QQ(C, W) \
    case C: return launch_q<C, W>(x, ldx, xq, ldq, scale, m, k, st);
#define QL(C) \
    case C: return launch_q<C, 4, 1>(x, ldx, xq, ldq, scale, m, k, st);
    if (m < 512 && nch <= 256 * 8) {
        switch ((nch + 255) / 256) { QL(1) QL(2) QL(3) QL(4) QL(5) QL(6) QL(7) QL(8) }
    } else if (nch <= 64 * 4) {
        switch ((nch + 63) / 64) { QQ(1, 1) QQ(2, 1) QQ(3, 1) QQ(4, 1) }
    } else if (nch <= 128 * 4) {
        switch ((nch + 127) / 128) { QQ(3, 2) QQ(4, 2) }
    } else if (nch <= 256 * 8) {
        switch ((nch + 255) / 256) { QQ(3, 4) QQ(4, 4) QQ(5, 4) QQ(6, 4) QQ(7, 4) QQ(8, 4) }
    } else {
        hipLaunchKernelGGL(quant_rows_long_kernel, dim3(m), dim3(256), 0, st, x, ldx, xq, ldq, scale, m, k);
        return hipGetLastError();
    }
#undef QQ
#undef QL
    return hipErrorInvalidValue;
}

}  // namespace rpl
