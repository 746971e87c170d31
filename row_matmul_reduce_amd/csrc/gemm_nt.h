// gemm_nt.h -- the MFMA tile engine behind the rank partial (bf16) and the
// w8a8 partial (int8) on gfx950.
//
// Both products are "NT": the activation shard X [m, K] and the weight shard
// W [n, K] are row-major with K contiguous, which is exactly the operand layout
// the MFMA instructions want, so no transposed weight copy is ever made (a
// copy that the xLLM pull request #1890 "feat: add FlashComm1 and MMRS fusion
// support for Qwen3.5 NPU" caches in its review thread; here it is not needed).
//
// One workgroup computes a BM x BN output tile with WM x WN wavefronts.  A K
// step stages 128 bytes of every operand row (64 bf16 or 128 int8 values)
// through LDS, double-buffered: the global loads of step t+1 are issued before
// the MFMAs of step t and written to the other LDS buffer afterwards, so one
// barrier per step suffices.  LDS rows are 128 bytes; the 16-byte chunk c of
// tile row r lives at chunk (c ^ (r & 7)), which spreads the 16 rows that an
// MFMA fragment read touches over distinct banks.
//
// MFMA operand roles are swapped (A <- weight rows, B <- activation rows) so
// that each lane's 4 accumulators are 4 consecutive output columns of one
// token row: the epilogue stores 4 values per lane as one 8-byte write.
//
// Tile order is XCD-aware: the hardware deals workgroups round-robin to the 8
// XCDs, so consecutive tile ids are remapped onto one XCD, and tiles are
// walked in bands of GROUP_M tile rows so that the tiles an XCD runs at the
// same time share activation rows and weight rows in that XCD's L2.
#pragma once

#include "rpl_device.h"

namespace rpl {

constexpr int KT_BYTES = 128;  // bytes of K staged per step, per operand row
constexpr int NUM_XCD = 8;

struct GemmShape {
    const uint8_t *x;    // activation shard, byte pointer, row stride ldx bytes
    const uint8_t *w;    // weight shard, byte pointer, row stride ldw bytes
    int64_t ldx, ldw;    // bytes
    int m;               // valid activation rows
    int m_pad;           // output rows (rows m..m_pad-1 are the zero padding)
    int n;               // output columns
    int kbytes;          // K in bytes (multiple of 16)
    int group_m;         // tile-row band height of the XCD-aware order
};

// Map the hardware block id to an output tile (tm, tn).
__device__ __forceinline__ void tile_of_block(int bid, int nt_m, int nt_n, int group_m, int &tm, int &tn) {
    const int total = nt_m * nt_n;
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    const int xcd = bid % NUM_XCD, local = bid / NUM_XCD;
    const int tile = (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
    const int band = group_m * nt_n;
    const int first_m = (tile / band) * group_m;
    const int gsz = min(nt_m - first_m, group_m);
    const int in_band = tile % band;
    tm = first_m + in_band % gsz;
    tn = in_band / gsz;
}

__device__ __forceinline__ int swz_off(int row, int chunk) { return row * KT_BYTES + ((chunk ^ (row & 7)) << 4); }

// Op supplies: Frag (16-byte operand), Acc (4-lane accumulator), mfma(), zero(),
// and the epilogue store(acc, m_row, n_col, valid_m) for 4 consecutive columns.
template <int BM, int BN, int WM, int WN, bool CHECK, class Op>
__device__ __forceinline__ void gemm_nt_tile(const GemmShape &g, const Op &op, uint8_t *smem) {
    constexpr int T = 64 * WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    constexpr int A_CH = BM * 8, B_CH = BN * 8;  // 16-byte chunks per K step
    constexpr int A_PER = (A_CH + T - 1) / T, B_PER = (B_CH + T - 1) / T;
    constexpr int STAGE = (BM + BN) * KT_BYTES;
    using Frag = typename Op::Frag;
    using Acc = typename Op::Acc;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;

    int tm, tn;
    const int nt_m = (g.m_pad + BM - 1) / BM, nt_n = (g.n + BN - 1) / BN;
    tile_of_block(blockIdx.x, nt_m, nt_n, g.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int ksteps = (g.kbytes + KT_BYTES - 1) / KT_BYTES;

    u32x4 ra[A_PER], rb[B_PER];

    auto gload = [&](int kt) {
        const int kb = kt * KT_BYTES;
#pragma unroll
        for (int j = 0; j < A_PER; ++j) {
            const int i = tid + j * T;
            if (A_CH % T == 0 || i < A_CH) {
                const int row = i >> 3, c = i & 7;
                const int grow = m0 + row, kbyte = kb + c * 16;
                const bool ok = !CHECK || (grow < g.m && kbyte < g.kbytes);
                ra[j] = ok ? ld16(g.x + (int64_t)grow * g.ldx + kbyte) : u32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int j = 0; j < B_PER; ++j) {
            const int i = tid + j * T;
            if (B_CH % T == 0 || i < B_CH) {
                const int row = i >> 3, c = i & 7;
                const int grow = n0 + row, kbyte = kb + c * 16;
                const bool ok = !CHECK || (grow < g.n && kbyte < g.kbytes);
                rb[j] = ok ? ld16(g.w + (int64_t)grow * g.ldw + kbyte) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto sstore = [&](int buf) {
        uint8_t *base = smem + buf * STAGE;
#pragma unroll
        for (int j = 0; j < A_PER; ++j) {
            const int i = tid + j * T;
            if (A_CH % T == 0 || i < A_CH) st16(base + swz_off(i >> 3, i & 7), ra[j]);
        }
#pragma unroll
        for (int j = 0; j < B_PER; ++j) {
            const int i = tid + j * T;
            if (B_CH % T == 0 || i < B_CH) st16(base + BM * KT_BYTES + swz_off(i >> 3, i & 7), rb[j]);
        }
    };

    Acc acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b) acc[a][b] = Op::zero();

    gload(0);
    sstore(0);
    __syncthreads();

    const int frow = lane & 15, fchunk = lane >> 4;
    for (int kt = 0; kt < ksteps; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < ksteps) gload(kt + 1);
        const uint8_t *sa = smem + cur * STAGE;
        const uint8_t *sb = sa + BM * KT_BYTES;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            Frag xf[FM], wf[FN];
#pragma unroll
            for (int a = 0; a < FM; ++a)
                xf[a] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4 *>(
                                                     sa + swz_off(wm0 + a * 16 + frow, kk * 4 + fchunk)));
#pragma unroll
            for (int b = 0; b < FN; ++b)
                wf[b] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4 *>(
                                                     sb + swz_off(wn0 + b * 16 + frow, kk * 4 + fchunk)));
#pragma unroll
            for (int a = 0; a < FM; ++a)
#pragma unroll
                for (int b = 0; b < FN; ++b) acc[a][b] = Op::mfma(wf[b], xf[a], acc[a][b]);
        }
        if (kt + 1 < ksteps) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: lane holds out[m0+wm0+a*16+(lane&15)][n0+wn0+b*16+4*(lane>>4) + 0..3].
#pragma unroll
    for (int a = 0; a < FM; ++a) {
        const int mrow = m0 + wm0 + a * 16 + frow;
#pragma unroll
        for (int b = 0; b < FN; ++b) {
            const int ncol = n0 + wn0 + b * 16 + fchunk * 4;
            if (!CHECK || (mrow < g.m_pad && ncol < g.n)) op.store(acc[a][b], mrow, ncol);
        }
    }
}

}  // namespace rpl
