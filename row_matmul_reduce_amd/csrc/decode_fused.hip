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
//   h[i, j]         = sum_s P_s[i, j] + residual[i, j]         (fp32, shards in order)
//   residual_out    = bf16(h)
//   y[i, j]         = bf16( gamma[j] * h[i, j] * rsqrt(mean_j h[i, :]^2 + eps) )
// Each shard's product is rounded to bf16 before the sum, exactly as a partial
// crosses the wire in the unfused path, so both paths have one definition.
//
// Work items are (16-column block cb, shard s) pairs, the decode partial's
// layout: eight waves split the shard's K range, every wave issues a batch of
// weight loads before its MFMAs, and the waves' sums meet in LDS.  With one item
// per workgroup (the decode shapes: tp * n/16 product workgroups) every CU
// streams weight rows.  Each product workgroup rounds its block to bf16 (the
// value that would cross the wire) and hands it on.  The last m workgroups of
// the grid are the rows' epilogues: the workgroup of row r prefetches the row's
// residual and gamma, collects the row's products of every shard as they are
// handed on, sums them in shard order, adds the residual, writes residual_out,
// takes the row's sum of squares with a block reduction and writes y.  The
// product hand-off is the only wait on the critical path (one round trip after
// the last product), and the row norm needs no second exchange.
//
// Hand-offs go through tagged slots in the workspace: a slot is one 64-bit word
// holding two bf16 products and the call's 32-bit tag, written and read with
// agent-scope atomic stores and loads (coherent across the XCDs' L2 caches
// without fences), so a value and its "ready" mark travel together and an
// epilogue polls the slots themselves.  The tag is the number of earlier calls
// on the workspace (plus one, so never a zeroed slot's 0): workgroup w keeps
// that count in its own word of the workspace, reads it at its start and stores
// it plus one, and workgroup 0 also advances the words of workgroups this launch
// does not have, so every word holds the same count when a call starts.  No two
// workgroups touch one word (one shared counter, bumped by every workgroup of a
// call, cost 25 us of serialised atomics), slots never need resetting, and a
// call whose wait gives up leaves no state behind.  Every wait polls a bounded
// number of times; past the bound the row's epilogue raises the workspace's
// status word and writes NaN to the row's y.  Waiting needs the epilogues
// resident with every product workgroup: the grid is capped at what the device
// holds at once (two workgroups of eight waves per CU), larger problems loop
// over their items, and products never wait.  (A cooperative launch gives the same
// guarantee but measured about 20 us more per launch here.)
#include <algorithm>
#include <atomic>
#include <mutex>

#include "rpl_device.h"
#include "rpl_launch.h"

namespace rpl {

constexpr int FD_WAVES = 8;  // waves per workgroup (8 took the decode chunk from 12.7 to 11.2 us)
constexpr unsigned FD_DEFAULT_POLLS = 1u << 22;  // re-reads of a slot group before a wait gives up

// K steps (32 values each) whose loads a wave issues together: 10-18 16-byte loads (up to
// 72 registers), within the 128 registers of four waves per SIMD.  8 steps cover a wave's
// eighth of K = 1792 (hidden 3584, TP = 2) in one batch.
template <int RB, int XP>
constexpr int fd_batch() { return RB == 1 ? 8 : RB == 2 ? 6 : RB == 3 ? 4 : 2; }

__device__ __forceinline__ void slot_put(unsigned long long *p, unsigned tag, uint32_t v) {
    __hip_atomic_store(p, ((unsigned long long)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long slot_get(const unsigned long long *p) {
    return __hip_atomic_load(const_cast<unsigned long long *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool slot_ready(unsigned long long v, unsigned tag) { return (unsigned)(v >> 32) == tag; }
__device__ __forceinline__ uint32_t slot_value(unsigned long long v) { return (uint32_t)v; }

__device__ __forceinline__ float fd_wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;  // xor butterfly: every lane ends with the same bits
}

// One work item's product: the 16 x (16 * RB) block P_s[rows, cb's columns] in fp32, summed
// over the waves' K ranges into wave 0's registers (lane: token row rb * 16 + (lane & 15),
// columns n0 + 4 * (lane >> 4) .. + 3).  XP K steps share one activation load (m <= 16 / XP):
// lane row r loads token row r % (16 / XP) of step t + r / (16 / XP), moved into place by row
// shifts; output rows past 16 / XP then hold other steps' products and are never used.
template <int RB, int XP>
__device__ __forceinline__ void fd_product(const FusedDecodeArgs &a, int s, int n0, f32x4 (&acc)[RB],
                                           f32x4 (*red)[RB][64]) {
    constexpr int BATCH = fd_batch<RB, XP>();
    constexpr int XR = 16 / XP;
    static_assert(XP == 1 || RB == 1, "activation packing only with one row block");
    static_assert(BATCH % XP == 0, "whole activation loads per batch");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int steps = (a.k + 31) / 32;
    const int per = (steps + FD_WAVES - 1) / FD_WAVES;
    const int s_begin = wave * per, s_end = min(steps, s_begin + per);
    const int r16 = lane & 15, g = lane >> 4;
    const int wrow = n0 + r16;
    const bool wrow_ok = wrow < a.n;
    const uint16_t *wp = a.w[s] + (int64_t)(wrow_ok ? wrow : 0) * a.ldw + g * 8;
    const int xrow0 = r16 % XR, xsub = r16 / XR;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = s_begin; t0 < s_end; t0 += BATCH) {
        // activation loads first (every MFMA needs one), then the weight loads in MFMA order
        u32x4 xf[BATCH / XP][RB], wf[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH / XP; ++j) {
            const int t = t0 + j * XP + xsub;
            const bool live = t < s_end && t * 32 + g * 8 < a.k;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int xrow = rb * 16 + xrow0;
                xf[j][rb] = (live && xrow < a.m_valid) ? ld16(a.x[s] + (int64_t)xrow * a.ldx + t * 32 + g * 8)
                                                       : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            const int t = t0 + j;
            const bool live = t < s_end && t * 32 + g * 8 < a.k;
            wf[j] = (live && wrow_ok) ? ld16(wp + t * 32) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                u32x4 xv = xf[j / XP][rb];
                if constexpr (XP == 2) {
                    if (j % 2) xv = lanes_down<8>(xv);
                } else if constexpr (XP == 4) {
                    if (j % 4 == 1) xv = lanes_down<4>(xv);
                    if (j % 4 == 2) xv = lanes_down<8>(xv);
                    if (j % 4 == 3) xv = lanes_down<12>(xv);
                }
                acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j]),
                                                                  __builtin_bit_cast(bf16x8, xv), acc[rb], 0, 0, 0);
            }
    }
    if (wave > 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) red[wave - 1][rb][lane] = acc[rb];
    __syncthreads();
    if (wave == 0)
#pragma unroll
        for (int v = 0; v < FD_WAVES - 1; ++v)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) acc[rb] += red[v][rb][lane];
    __syncthreads();  // red is free for the next item
}

// An epilogue thread owns EQ quads (4 columns) of its row, rows up to 8192 wide; a poll
// covers SG shards' slots of them (16 slots, 32 registers in flight).
constexpr int FD_EQ = 4, FD_SG = 2;

template <int RB, int XP>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * FD_WAVES, 64 * FD_WAVES)))
__attribute__((amdgpu_waves_per_eu(4)))
decode_fused_kernel(FusedDecodeArgs a) {
    __shared__ f32x4 red[FD_WAVES - 1][RB][64];
    __shared__ float part[FD_WAVES];
    __shared__ unsigned tag_sh;
    __shared__ int late_sh;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nblk = (a.n + 15) >> 4;
    const int items = a.tp * nblk;
    const int prod = gridDim.x - a.m;  // product workgroups; the last m are the rows' epilogues
    const int64_t half = a.n >> 1;     // slots per (row, shard)

    // The call count (see the header comment): read at the start and first needed after the
    // product (product workgroups) or before the first poll (epilogues); the next call's count
    // is stored at once (no other workgroup touches this word).
    unsigned calls = 0;
    if (wave == 0) {
        if (lane == 0) {
            calls = a.calls[blockIdx.x];
            a.calls[blockIdx.x] = calls + 1u;
        }
        if (blockIdx.x == 0) {  // the words of workgroups this launch does not have
            const unsigned c0 = __builtin_amdgcn_readfirstlane(calls);
            for (int j = gridDim.x + lane; j < FD_MAX_GRID; j += 64) a.calls[j] = c0 + 1u;
        }
    }

    if ((int)blockIdx.x < prod) {
        // ---- products: items blockIdx.x, blockIdx.x + prod, ...; item i is shard i / nblk,
        // column block i % nblk.  Wave 0 hands each block on: lane (r16, g) holds token row
        // rb * 16 + r16, columns n0 + 4g .. + 3, i.e. two slots of the row's shard plane.
        const int r16 = lane & 15, g = lane >> 4;
        for (int i = blockIdx.x; i < items; i += prod) {
            const int s = i / nblk, cb = i - s * nblk, n0 = cb * 16, col = n0 + 4 * g;
            f32x4 acc[RB];
            fd_product<RB, XP>(a, s, n0, acc, red);
            if (wave != 0) continue;
            const unsigned tag = __builtin_amdgcn_readfirstlane(calls) % 0xFFFFFFFFu + 1u;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row = rb * 16 + r16;
                if (row < a.m && col < a.n) {
                    unsigned long long *sl = a.p_slots + ((int64_t)row * a.tp + s) * half + (col >> 1);
                    slot_put(sl, tag, pack_bf16x2(acc[rb][0], acc[rb][1]));
                    slot_put(sl + 1, tag, pack_bf16x2(acc[rb][2], acc[rb][3]));
                }
            }
        }
        return;
    }

    // ---- the epilogue of token row r: thread t owns quads t, t + NT, ... (EQ of them); the
    // residual and gamma are loaded before the first poll
    constexpr int NT = 64 * FD_WAVES, EQ = FD_EQ, SG = FD_SG, QC = FD_EQ;
    constexpr bool EARLY = true;
    const int r = blockIdx.x - prod;
    const int nq = a.n >> 2;
    const int64_t rbase = (int64_t)r * a.n;
    auto quad_ok = [&](int j) { return (int)threadIdx.x + NT * j < nq; };
    auto col_of = [&](int j) { return 4 * ((int)threadIdx.x + NT * j); };
    u32x2 rv[EQ], gv[EQ];
    f32x4 h[EQ];
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
        h[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (EARLY) {
            rv[j] = quad_ok(j) ? *reinterpret_cast<const u32x2 *>(a.residual + rbase + col_of(j)) : u32x2{0u, 0u};
            gv[j] = quad_ok(j) ? *reinterpret_cast<const u32x2 *>(a.gamma + col_of(j)) : u32x2{0u, 0u};
        }
    }
    if (threadIdx.x == 0) {
        tag_sh = calls % 0xFFFFFFFFu + 1u;
        late_sh = 0;
    }
    __syncthreads();
    const unsigned tag = tag_sh;
    const unsigned polls = a.poll_limit[0] ? a.poll_limit[0] : FD_DEFAULT_POLLS;
    bool late = false;
    const unsigned long long *rs = a.p_slots + (int64_t)r * a.tp * half;
    for (int s0 = 0; s0 < a.tp; s0 += SG) {  // shards in order: every quad's sum has a fixed order
#pragma unroll
        for (int c = 0; c < EQ; c += QC) {
            unsigned long long v[SG][QC][2];
            for (unsigned it = 0;; ++it) {
                bool ok = true;
#pragma unroll
                for (int q = 0; q < SG; ++q)
#pragma unroll
                    for (int j = 0; j < QC; ++j) {
                        if (s0 + q < a.tp && quad_ok(c + j)) {
                            const unsigned long long *sl = rs + (int64_t)(s0 + q) * half + (col_of(c + j) >> 1);
                            v[q][j][0] = slot_get(sl);
                            v[q][j][1] = slot_get(sl + 1);
                            ok = ok && slot_ready(v[q][j][0], tag) && slot_ready(v[q][j][1], tag);
                        } else {
                            v[q][j][0] = v[q][j][1] = 0;
                        }
                    }
                if (ok) break;
                if (it >= polls) {
                    late = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
#pragma unroll
            for (int q = 0; q < SG; ++q)
#pragma unroll
                for (int j = 0; j < QC; ++j) {
                    const uint32_t lo = slot_value(v[q][j][0]), hi = slot_value(v[q][j][1]);
                    h[c + j] += f32x4{bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi)};
                }
        }
    }
    // residual add, residual_out, the row's sum of squares
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
        if (!EARLY) rv[j] = quad_ok(j) ? *reinterpret_cast<const u32x2 *>(a.residual + rbase + col_of(j)) : u32x2{0u, 0u};
        h[j] += f32x4{bf16_lo(rv[j][0]), bf16_hi(rv[j][0]), bf16_lo(rv[j][1]), bf16_hi(rv[j][1])};
        if (quad_ok(j)) {
            st8(a.residual_out + rbase + col_of(j),
                u32x2{pack_bf16x2(h[j][0], h[j][1]), pack_bf16x2(h[j][2], h[j][3])});
            ss += h[j][0] * h[j][0] + h[j][1] * h[j][1] + h[j][2] * h[j][2] + h[j][3] * h[j][3];
        }
    }
    ss = fd_wave_sum(ss);
    if (lane == 0) part[wave] = ss;
    if (late) late_sh = 1;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < FD_WAVES; ++w) tot += part[w];
    const float inv = rsqrtf(tot / (float)a.n + a.eps);
    const bool bad = late_sh != 0;
#pragma unroll
    for (int j = 0; j < EQ; ++j) {
        if (!quad_ok(j)) continue;
        if (!EARLY) gv[j] = *reinterpret_cast<const u32x2 *>(a.gamma + col_of(j));
        u32x2 yo = {pack_bf16x2(bf16_lo(gv[j][0]) * (h[j][0] * inv), bf16_hi(gv[j][0]) * (h[j][1] * inv)),
                    pack_bf16x2(bf16_lo(gv[j][1]) * (h[j][2] * inv), bf16_hi(gv[j][1]) * (h[j][3] * inv))};
        if (bad) yo = u32x2{0x7FC07FC0u, 0x7FC07FC0u};  // NaN: the result is not valid
        st8(a.y + rbase + col_of(j), yo);
    }
    if (bad && threadIdx.x == 0) __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace layout (bytes): [8, 12) the status word (nonzero after a wait gave up), [12, 16)
// the poll bound (0 = default), [256, 256 + 4 * FD_MAX_GRID) the workgroups' call counts; from
// FD_WS_HEADER the product slots [m][tp][n / 2], 8 bytes each.
int64_t fused_decode_workspace_bytes(int64_t m, int64_t n, int64_t tp) { return FD_WS_HEADER + 4 * m * tp * n; }

// Hand-off memory of rpl_matmul_reduce_rmsnorm_noalloc, for callers that cannot allocate: the
// same layout as a caller's workspace, in a file-scope device array that each GPU holds until the
// process ends.  Static storage starts zero-filled, which is all the hand-off protocol needs:
// calls leave it ready for the next one, so nothing is cleared between calls.
static __device__ __align__(256) uint8_t scratch[FD_SCRATCH_BYTES];

// The device address of `scratch` on the current device.  In host code the array's name is a
// host-side stand-in, not a device address: the address is looked up once per device (with that
// device current) and kept; kernels only ever receive the looked-up pointer.
hipError_t fused_decode_scratch(void **ptr) {
    constexpr int MAX_DEV = 64;
    static std::mutex mu;
    static void *addr[MAX_DEV];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// Workgroups of one kernel variant the current device holds at once, at most FD_MAX_GRID
// (looked up once per device and variant).
static int fd_resident(const void *kernel, int variant) {
    constexpr int MAX_DEV = 64, VARIANTS = 6;
    static std::atomic<int> cache[MAX_DEV][VARIANTS];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEV) return 0;
    int v = cache[dev][variant].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * FD_WAVES, 0) != hipSuccess)
            return 0;
        v = (int)std::min<long>((long)cus * per_cu, FD_MAX_GRID);
        cache[dev][variant].store(v, std::memory_order_relaxed);
    }
    return v;
}

template <int RB, int XP>
static hipError_t fd_launch(const FusedDecodeArgs &a, int variant, hipStream_t st) {
    const void *kernel = reinterpret_cast<const void *>(&decode_fused_kernel<RB, XP>);
    const int64_t items = (int64_t)a.tp * ((a.n + 15) / 16);
    const int resident = fd_resident(kernel, variant);
    if (resident < a.m + 1) return hipErrorCooperativeLaunchTooLarge;  // not all resident at once
    const int prod = (int)std::min<int64_t>(items, resident - a.m);
    hipLaunchKernelGGL((decode_fused_kernel<RB, XP>), dim3(prod + a.m), dim3(64 * FD_WAVES), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_decode_fused(const FusedDecodeArgs &a, hipStream_t st) {
    if (a.n > 4 * 64 * FD_WAVES * FD_EQ) return hipErrorInvalidValue;
    if (a.m <= 4) return fd_launch<1, 4>(a, 0, st);
    if (a.m <= 8) return fd_launch<1, 2>(a, 1, st);
    switch ((a.m + 15) / 16) {
        case 1: return fd_launch<1, 1>(a, 2, st);
        case 2: return fd_launch<2, 1>(a, 3, st);
        case 3: return fd_launch<3, 1>(a, 4, st);
        case 4: return fd_launch<4, 1>(a, 5, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rpl
