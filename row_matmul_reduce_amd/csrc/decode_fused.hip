// decode_fused.hip -- the whole path for a decode-sized block of token rows in
// one launch on gfx950: every tensor-parallel shard's product, the sum of the
// shards, residual add and RMSNorm.
//
// What it computes (Dewu tech blog "国产算力·昇腾 910C 大模型推理优化（下）：源码修改与
// 算子优化", communication-fusion section: one operator holds o_proj matmul +
// AllReduce + residual add + RMSNorm for up to 40 rows, reducing across ranks as
// matmul tiles finish and normalising with a cross-rank sum of squares; its
// fallback is the unfused composition matmul + all_reduce + add_rms_norm):
//   P_s[i, j]       = bf16( sum_k x_s[i, k] * w_s[j, k] )     (pad rows i >= m_valid: 0)
//   h[i, j]         = sum_s P_s[i, j] + residual[i, j]         (fp32)
//   residual_out    = bf16(h)
//   y[i, j]         = bf16( gamma[j] * h[i, j] * rsqrt(mean_j h[i, :]^2 + eps) )
// Each shard's product is rounded to bf16 before the sum, exactly as a partial
// crosses the wire in the unfused path, so both paths have one definition.
//
// One workgroup per 16 output columns, 16 waves (8 above 16 token rows): the shards'
// products are computed concurrently by groups of waves/tp waves, each group
// splitting its shard's K range; every wave issues up to 8 or 16 K steps of loads
// before its MFMAs.  The waves' MFMA partials meet in LDS, where wave 0 sums each
// shard's group, rounds the shard's product to bf16 and adds it to a running fp32
// sum.  After
// the residual add, wave 0 writes residual_out, the fp32 h of its columns and
// each row's partial sum of squares over its 16 columns to the workspace.  The
// row norm needs every column: the workgroup that finishes last (a device-scope
// counter in the workspace, incremented once per workgroup after a release
// fence; the last one then takes an acquire fence) sums the partial sums, then
// writes y for all columns from the fp32 h, and resets the counter.  No
// workgroup waits for another, so nothing spins.
#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

// Waves per workgroup: 16 for up to 16 token rows (more waves in flight per column block
// shortened the products from 11.5 to 10.3 us on the decode chunk), 8 for more rows, where
// each wave holds up to four row blocks of activation fragments.
template <int RB>
constexpr int fd_waves() { return RB == 1 ? 16 : 8; }

// Waves per shard: the workgroup's waves split into tp groups (up to one shard per wave);
// a group splits its shard's K range.  More shards than waves are taken in passes.
__device__ __forceinline__ int fd_waves_per_shard(int tp, int waves) { return tp >= waves ? 1 : waves / tp; }

template <int RB, int FD_WAVES = fd_waves<RB>()>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * FD_WAVES, 64 * FD_WAVES)))
decode_fused_kernel(FusedDecodeArgs a) {
    // K steps (32 values each) whose loads are issued together, sized to the registers a wave has
    constexpr int BATCH = FD_WAVES == 16 ? 8 : RB <= 2 ? 16 : 8;
    __shared__ f32x4 red[FD_WAVES][RB][64];
    __shared__ float inv_rms[16 * RB];
    __shared__ int last_flag;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = gridDim.x;
    const int n0 = blockIdx.x * 16;
    const int steps = (a.k + 31) / 32;
    const int wps = fd_waves_per_shard(a.tp, FD_WAVES);
    const int group = wave / wps, sub = wave % wps;         // shard group, position in it
    const int per = (steps + wps - 1) / wps;
    const int s_begin = sub * per, s_end = min(steps, s_begin + per);
    const int r16 = lane & 15, g = lane >> 4;
    const int wrow = n0 + r16;
    const bool wrow_ok = wrow < a.n;
    const int groups = FD_WAVES / wps;                       // shards handled per pass

    f32x4 hsum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) hsum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s0 = 0; s0 < a.tp; s0 += groups) {
        const int s = s0 + group;
        const bool shard_ok = group < groups && s < a.tp;
        f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (shard_ok) {
            const uint16_t *wp = a.w[s] + (int64_t)(wrow_ok ? wrow : 0) * a.ldw + g * 8;
            for (int t0 = s_begin; t0 < s_end; t0 += BATCH) {
                u32x4 wf[BATCH], xf[BATCH][RB];
#pragma unroll
                for (int j = 0; j < BATCH; ++j) {
                    const int t = t0 + j;
                    const int kel = t * 32 + g * 8;
                    const bool live = t < s_end && kel < a.k;
                    wf[j] = (live && wrow_ok) ? ld16(wp + t * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const int xrow = rb * 16 + r16;
                        xf[j][rb] = (live && xrow < a.m_valid) ? ld16(a.x[s] + (int64_t)xrow * a.ldx + kel)
                                                               : u32x4{0, 0, 0, 0};
                    }
                }
#pragma unroll
                for (int j = 0; j < BATCH; ++j)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j]),
                                                                          __builtin_bit_cast(bf16x8, xf[j][rb]),
                                                                          acc[rb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) red[wave][rb][lane] = acc[rb];
        __syncthreads();
        if (wave == 0) {
            // shards in order: each shard's waves summed in order, rounded to bf16 (the
            // product as it would cross the wire), added to the running fp32 sum
            for (int q = 0; q < groups && s0 + q < a.tp; ++q) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    f32x4 p = red[q * wps][rb][lane];
                    for (int v = 1; v < wps; ++v) p += red[q * wps + v][rb][lane];
                    const uint32_t lo = pack_bf16x2(p[0], p[1]), hi = pack_bf16x2(p[2], p[3]);
                    hsum[rb] += f32x4{bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
                }
            }
        }
        __syncthreads();  // red is reused by the next pass
    }

    // Lane (wave 0) holds h for token row rb*16 + r16, columns n0 + 4g .. n0 + 4g + 3.
    if (wave == 0) {
        const int col = n0 + g * 4;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int row = rb * 16 + r16;
            float ss = 0.f;
            if (row < a.m && col < a.n) {
                const int64_t off = (int64_t)row * a.n + col;
                const u32x2 rv = *reinterpret_cast<const u32x2 *>(a.residual + off);
                const f32x4 h = hsum[rb] + f32x4{bf16_lo(rv[0]), bf16_hi(rv[0]), bf16_lo(rv[1]), bf16_hi(rv[1])};
                st8(a.residual_out + off, u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])});
                *reinterpret_cast<f32x4 *>(a.h_ws + off) = h;
                ss = h[0] * h[0] + h[1] * h[1] + h[2] * h[2] + h[3] * h[3];
            }
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            if (g == 0 && row < a.m) a.ss_ws[(int64_t)row * nblk + blockIdx.x] = ss;
        }
        // Release this workgroup's h and partial sums at device (agent) scope -- an L2
        // write-back on this multi-XCD part, so only the one wave that wrote them pays it --
        // then count in.  A release fence, not a full one: nothing is read after it.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) last_flag = (atomicAdd(a.counter, 1u) == (unsigned)nblk - 1) ? 1 : 0;
    }
    __syncthreads();
    if (!last_flag) return;

    // Last workgroup: every other workgroup's results are visible after an acquire fence
    // (the counter's read-modify-write read the increments that followed their release
    // fences).  The first batch of h and gamma loads is issued before the partial sums are
    // reduced, so the two round trips overlap.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    constexpr int U = 4;
    const int nch = a.n / 8;  // 8 outputs per chunk
    const int total = a.m * nch;
    f32x4 hv[U][2];
    u32x4 gv[U];
    auto load_batch = [&](int c0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 64 * FD_WAVES;
            if (c < total) {
                const int row = c / nch, cc = c - row * nch;
                const float *hp = a.h_ws + (int64_t)row * a.n + cc * 8;
                hv[u][0] = *reinterpret_cast<const f32x4 *>(hp);
                hv[u][1] = *reinterpret_cast<const f32x4 *>(hp + 4);
                gv[u] = ld16(a.gamma + cc * 8);
            }
        }
    };
    load_batch(threadIdx.x);
    for (int row = wave; row < a.m; row += FD_WAVES) {
        float ss = 0.f;
        for (int b = lane; b < nblk; b += 64) ss += a.ss_ws[(int64_t)row * nblk + b];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if (lane == 0) inv_rms[row] = rsqrtf(ss / (float)a.n + a.eps);
    }
    __syncthreads();
    for (int c0 = threadIdx.x; c0 < total; c0 += 64 * FD_WAVES * U) {
        if (c0 != (int)threadIdx.x) load_batch(c0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * 64 * FD_WAVES;
            if (c < total) {
                const int row = c / nch, cc = c - row * nch;
                const float inv = inv_rms[row];
                u32x4 yo;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float h0 = hv[u][q >> 1][(q & 1) * 2], h1 = hv[u][q >> 1][(q & 1) * 2 + 1];
                    yo[q] = pack_bf16x2(bf16_lo(gv[u][q]) * (h0 * inv), bf16_hi(gv[u][q]) * (h1 * inv));
                }
                st16(a.y + (int64_t)row * a.n + cc * 8, yo);
            }
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int64_t fused_decode_ss_bytes(int64_t m, int64_t n) {
    const int64_t nblk = (n + 15) / 16;
    return (4 * m * nblk + 255) / 256 * 256;
}

int64_t fused_decode_workspace_bytes(int64_t m, int64_t n) {
    return FD_WS_HEADER + fused_decode_ss_bytes(m, n) + 4 * m * n;
}

hipError_t launch_decode_fused(const FusedDecodeArgs &a, hipStream_t st) {
    const dim3 grid((a.n + 15) / 16);
    switch ((a.m + 15) / 16) {
        case 1: hipLaunchKernelGGL(decode_fused_kernel<1>, grid, dim3(64 * fd_waves<1>()), 0, st, a); break;
        case 2: hipLaunchKernelGGL(decode_fused_kernel<2>, grid, dim3(64 * fd_waves<2>()), 0, st, a); break;
        case 3: hipLaunchKernelGGL(decode_fused_kernel<3>, grid, dim3(64 * fd_waves<3>()), 0, st, a); break;
        case 4: hipLaunchKernelGGL(decode_fused_kernel<4>, grid, dim3(64 * fd_waves<4>()), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rpl
