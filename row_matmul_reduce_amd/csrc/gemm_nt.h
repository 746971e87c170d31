// gemm_nt.h -- the MFMA tile engine behind the rank partial (bf16) and the
// w8a8 partial (int8) on gfx950.
//
// Both products are "NT": the activation shard X [m, K] and the weight shard
// W [n, K] are row-major with K contiguous, which is exactly the operand layout
// the MFMA instructions want, so no transposed weight copy is ever made (a
// copy that the xLLM pull request #1890 "feat: add FlashComm1 and MMRS fusion
// support for Qwen3.5 NPU" caches in its review thread; here it is not needed).
//
// One workgroup computes a 256 x 224 (or 256 x 256) output tile with 2 x 2 wavefronts,
// 128 x 112 (128 x 128) outputs per wave, the accumulators held in the accumulation registers.
//
// Staging.  A K step stages 128 bytes of every operand row (64 bf16 or 128
// int8 values) in LDS: the activation double-buffered, the weight in a ring of
// three steps where the LDS holds it (two otherwise).  Rows reach LDS straight from memory
// with buffer_load_dwordx4 ... lds (no VGPR round trip): one wave instruction
// fills 8 rows x 128 bytes.  The buffer descriptor of each operand starts at
// the tile's first row and its record count ends at the operand's last valid
// byte, so rows past m (or n) read as zero in hardware; K-tail chunks get an
// out-of-range offset and read as zero too.  Ragged shapes therefore need no
// separate bounds-checked kernel.  In LDS the 16-byte chunk c of tile row r
// sits at chunk (c ^ (r & 7)), so the 16 rows one MFMA fragment read touches
// fall on distinct banks (zero bank conflicts measured with rocprofv3).
//
// L2 prefetch.  Two buffers of LDS give the DMA of step k+2 one step of lead,
// less than the latency of HBM under load.  The weight ring's third buffer gives
// the weight DMA (step k+3) two; for the activation each step also touches the
// lines of step k+PF (PF = 3) -- one 4-byte DMA per 128-byte line into a
// 256-byte LDS sink that is never read -- so that the real DMA finds them in
// L2.  The workgroups of an XCD that share activation rows split their
// prefetch between them, so each line is touched about once per XCD rather
// than once per sharer (half the L2 requests of a per-workgroup prefetch).
// Only the activation is prefetched: the four workgroups of an XCD that share
// a weight tile request its lines together anyway, and prefetching it as well
// measured 2% slower.  The barrier waits for every load but the newest prefetch
// (and, with the weight ring, the weight DMAs of the step after next).
//
// MFMA operand roles are swapped (A <- weight rows, B <- activation rows) so
// that each lane's 4 accumulators are 4 consecutive output columns of one
// token row: the epilogue stores 4 values per lane as one 8-byte write.
//
// Tile order is XCD-aware: the hardware deals workgroups round-robin to the 8
// XCDs, so consecutive tile ids are remapped onto one XCD, and tiles are
// walked in bands of GROUP_M tile rows so that the tiles an XCD runs at the
// same time share activation rows and weight rows in that XCD's L2.  At most
// 256 workgroups run (one per CU); each loops over its tiles.
#pragma once

#include "rpl_device.h"

namespace rpl {

constexpr int KT_BYTES = 128;  // bytes of K staged per step, per operand row
constexpr int NUM_CU = 256;  // MI355X compute units
constexpr int NUM_XCD = 8;
constexpr int PF_BYTES = 256;  // LDS sink of the prefetch loads (64 lanes x 4 bytes)
constexpr int PF_SHARE_X = 8;  // workgroups of one XCD that share an activation row at a time
// Largest operand row stride (bytes) the 32-bit buffer offsets of a 256-row tile can address.
constexpr int64_t MAX_LD_BYTES = int64_t(1) << 23;

struct GemmShape {
    const uint8_t *x;    // activation shard, byte pointer, row stride ldx bytes
    const uint8_t *w;    // weight shard, byte pointer, row stride ldw bytes
    int64_t ldx, ldw;    // bytes (< MAX_LD_BYTES)
    int m;               // valid activation rows
    int m_pad;           // output rows (rows m..m_pad-1 are the zero padding)
    int n;               // output columns
    int kbytes;          // K in bytes (multiple of 16)
    int group_m;         // tile-row band height of the XCD-aware order
};

typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int32_t RSRC_DWORD3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t OOB_OFFSET = 0x80000000u; // beyond every record count: reads as zero

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

// Buffer descriptor over rows [r0, rows) of a row-major operand with row stride ld bytes
// and kbytes valid bytes per row; rows at or past `rows` read as zero.
// The same as a base and a record count, for descriptors rebuilt per K step.
struct TileSpan {
    const uint8_t *base;
    uint32_t nrec;
};
__device__ __forceinline__ TileSpan tile_span(const uint8_t *base, int r0, int rows, int64_t ld, int kbytes) {
    const bool live = r0 < rows;
    const int64_t start = (int64_t)r0 * ld;
    const int64_t span = (int64_t)(rows - 1) * ld + kbytes;  // bytes from row 0 to the last valid byte
    const uint32_t nrec = __builtin_amdgcn_readfirstlane(live ? (uint32_t)min<int64_t>(span - start, 0x7FFFFFFF) : 0u);
    return TileSpan{base + (live ? start : 0), nrec};
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const TileSpan &t, bool live) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(t.base), (short)0, live ? (int)t.nrec : 0,
                                             RSRC_DWORD3);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t *base, int r0, int rows, int64_t ld,
                                                            int kbytes) {
    return span_rsrc(tile_span(base, r0, rows, ld, kbytes), true);
}

constexpr int WIDE_STAGE_BYTES = 2 * (256 + 256) * 4;
constexpr int LDS_BYTES = 160 * 1024;  // per workgroup on gfx950

// Weight steps in the engine's LDS ring: three where they fit next to the activation's two, the
// prefetch sink and (staged Ops) the staging area, else two.
__host__ __device__ constexpr int wide_w_stages(int bn, bool staged) {
    return (2 * 256 + 3 * bn) * KT_BYTES + PF_BYTES + (staged ? WIDE_STAGE_BYTES : 0) <= LDS_BYTES ? 3 : 2;
}
// LDS bytes of the engine's operand rings (two activation steps and wide_w_stages weight steps of a
// 256 x BN tile) or, when larger, of the row-major copy a finished tile is stored through (rows
// padded by 16 bytes); the prefetch sink and any staging area follow it.
__host__ __device__ constexpr int wide_main_bytes(int bn, bool staged) {
    return (2 * 256 + wide_w_stages(bn, staged) * bn) * KT_BYTES > 256 * (bn * 2 + 16)
               ? (2 * 256 + wide_w_stages(bn, staged) * bn) * KT_BYTES
               : 256 * (bn * 2 + 16);
}

// The engine: a 256 x BN tile (BN = 224 or 256) on 2 x 2 waves, 128 x BN/2
// outputs per wave.  Per MFMA it reads a third fewer fragments from LDS than an
// 8-wave layout (16 fragment reads feed 64 MFMAs instead of 8 feeding 16), and
// with one wave per SIMD each wave owns the whole register file: the
// 128 x 112 (or 128 x 128) fp32 accumulators live in the 256 accumulation
// registers, pinned there by Op::mfma_acc (an MFMA written as inline assembly on
// an "a"-constrained operand), which leaves the 256 vector registers to the two
// fragment sets and the addressing.
//
// Per step: 128 bytes of K per row, DMA of the activation's step k+2 (and of the weight's
// step k+3 with a three-step ring, else k+2) into the buffers released by step k's barrier,
// L2 prefetch of the activation's step k+PF.  (The third weight buffer: prefill share
// 195.1 -> 192.3, 199.2 -> 195.7 and 195.2 -> 191.1 us on three boxes, bit-identical.)  The interleave
// is explicit rather than requested from the scheduler: each half-step is cut
// into FM+FN groups of MFMAs, each followed by fragment reads of the other
// half (two per group in the first half, one in the second) and, in the second
// half, one DMA instruction, with a sched_barrier after every group, so the
// issue order is exactly that.  (Against one read per group, activation
// fragments first and a wait for all of them at the end of each half: prefill
// share 199.8 -> 197.3 us, long-prefill share 396.2 -> 390.8 us on one box; in
// cycles a little more, as the card then runs a slightly lower clock.)  Each wave issues 8 + FN DMA instructions per step (activation
// groups wave, wave+4, ...; weight groups likewise), as many as it reads
// fragments.  The K loop is unrolled by two (six with a three-step weight ring) so
// that the buffer addresses are constants.
//
// Hazards the compiler cannot see through inline assembly: zeroed accumulators
// are written before the first MFMA reads them (a tie to each, then s_nop), and
// the results of the last MFMAs of a tile are read only after enough wait
// states (an s_nop tied to the accumulators of the last group; every earlier
// group sits behind a sched_barrier and has long completed).
//
// Op supplies: Frag (16-byte operand) and Acc (4-lane accumulator) types, zero(),
// mfma_acc(acc, weight_frag, activation_frag), and either store(acc, row, col) of 4
// consecutive columns and pack(acc) of them as 8 output bytes (STAGED = false) or, with
// STAGED = true, stage(rows, cols, m0, n0, wave, lane), which DMAs a value per tile row
// and per tile column into LDS, store_staged(acc, row, col, row_value, column_values) and
// pack_staged(acc, row_value, column_values); and store16(row, col, v) of 8 consecutive
// output columns and coalesced_final(), whether the last tile may take the path below.
//
// Finished tiles are stored through LDS: each lane writes its 4-column pieces into a
// row-major copy of the tile, then the workgroup stores whole rows with 16 bytes per lane,
// so every store instruction covers full 128-byte lines instead of 32-byte pieces of 16
// rows.  The last tile of a workgroup (the only one on shares with one tile per CU) is
// stored after the K loop (bf16 prefill share: 202.7 -> 199.5 us in a probe of the same
// engine, the store itself being about 10 us of the kernel); a tile with a successor is
// stored before the successor's first DMAs, since its copy needs the operand buffers
// (long-prefill share: 429.1 -> 417.9 us against the direct store overlapped with those
// DMAs).  Staged Ops take this path only for the last tile and only when coalesced_final()
// (a second copy of it pushes the int8 kernel's registers into spills).
// smem: wide_main_bytes(BN, Op::STAGED) + PF_BYTES bytes of LDS, plus WIDE_STAGE_BYTES
// for a staged Op.  KTAIL: K is not a whole number of steps (kbytes % KT_BYTES != 0), so the
// last step's chunks past K are cut lane by lane; without a tail only whole steps past
// the end are cut, by one uniform test per step, and the DMA addressing needs no
// vector instruction at all (the prefill share 188.5-189.2 us against 196.6-197.4 us in the
// per-lane form, one box).
template <int BN, int PF, bool KTAIL, class Op, bool CO_LOOP = true>
__device__ __forceinline__ void gemm_nt_wide(const GemmShape &g, const Op &op, uint8_t *smem) {
    constexpr int BM = 256, NW = 4, WN = 2;
    constexpr int TM = BM / 2, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int GA = BM / 8, GB = BN / 8;            // 8-row (1 KB) groups per operand per step
    constexpr int NA = GA / NW, NB = GB / NW;          // DMA instructions per wave per step
    constexpr int NR = FM + FN, NM = FM * FN;          // fragment reads and MFMAs per half-step
    static_assert(GA % NW == 0 && GB % NW == 0 && NA + NB == NR, "one DMA per fragment read");
    static_assert(BM / PF_SHARE_X <= 64, "activation prefetch slice fits one wave");
    constexpr int WS = wide_w_stages(BN, Op::STAGED);  // weight steps in the ring
    constexpr int XB = BM * KT_BYTES, WB = BN * KT_BYTES;
    constexpr int STAGE_FLOATS = BM + 256;  // one staging area: a value per tile row and per column
    using Frag = typename Op::Frag;
    using Acc = typename Op::Acc;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;
    const int nt_m = (g.m_pad + BM - 1) / BM, nt_n = (g.n + BN - 1) / BN;
    const int total = nt_m * nt_n;
    const int ksteps = (g.kbytes + KT_BYTES - 1) / KT_BYTES;
    constexpr int MAIN = wide_main_bytes(BN, Op::STAGED);
    static_assert(MAIN + PF_BYTES + (Op::STAGED ? WIDE_STAGE_BYTES : 0) <= LDS_BYTES, "LDS budget");
    uint8_t *const X0 = smem, *const X1 = smem + XB;                       // activation steps
    uint8_t *const W0 = smem + 2 * XB, *const W1 = W0 + WB, *const W2 = W1 + WB;  // weight steps
    uint8_t *const sink = smem + MAIN;
    const int lr = lane >> 3;
    const int pc = (lane & 7) ^ lr;
    const int frow = lane & 15, fchunk = lane >> 4;

    __amdgpu_buffer_rsrc_t rx, rw;
    TileSpan sx{}, sw{};  // the same tiles as base and record count (per-step descriptors)
    int pfx0 = 0;  // first row of this workgroup's activation prefetch slice
    // DMA instruction j: activation group j*NW + wave of step ktx into xbuf (j < NA), else
    // weight group (j-NA)*NW + wave of step ktw into wbuf.  j is a compile-time constant at
    // every call.
    // With a K tail each lane's offset is cut to OOB_OFFSET past K.  Without one the
    // per-lane offset is the same at every step (the compiler keeps it in a register)
    // and the step's byte offset goes in the scalar offset; a step past the end gets a
    // descriptor with no records, so its loads read nothing.  Either way a lane's byte
    // is row * ld + k, inside the row's K bytes or out of range.
    auto dma = [&](int ktx, uint8_t *xbuf, int ktw, uint8_t *wbuf, int j) {
        const int kt = j < NA ? ktx : ktw;
        if constexpr (KTAIL) {
            const int kb = kt * KT_BYTES + pc * 16;
            const bool kin = kb < g.kbytes;
            if (j < NA) {
                const int gi = j * NW + wave;
                const uint32_t v = kin ? (uint32_t)((gi * 8 + lr) * g.ldx + kb) : OOB_OFFSET;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)(xbuf + gi * 1024), 16, v, 0, 0, 0);
            } else {
                const int gj = (j - NA) * NW + wave;
                const uint32_t v = kin ? (uint32_t)((gj * 8 + lr) * g.ldw + kb) : OOB_OFFSET;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void_t *)(wbuf + gj * 1024), 16, v, 0, 0, 0);
            }
        } else {
            const bool live = kt * KT_BYTES < g.kbytes;
            const int kstep = live ? kt * KT_BYTES : 0;
            if (j < NA) {
                const int gi = j * NW + wave;
                const uint32_t v = (uint32_t)((gi * 8 + lr) * g.ldx + pc * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(span_rsrc(sx, live), (lds_void_t *)(xbuf + gi * 1024), 16, v,
                                                         kstep, 0, 0);
            } else {
                const int gj = (j - NA) * NW + wave;
                const uint32_t v = (uint32_t)((gj * 8 + lr) * g.ldw + pc * 16);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(span_rsrc(sw, live), (lds_void_t *)(wbuf + gj * 1024), 16, v,
                                                         kstep, 0, 0);
            }
        }
    };
    // Shared L2 prefetch of the activation slice on wave 0, an out-of-range load on
    // the others (the barrier's vmcnt counts on one).
    auto prefetch = [&](int kt) {
        const int kb = kt * KT_BYTES;
        uint32_t v = OOB_OFFSET;
        if (wave == 0 && lane < BM / PF_SHARE_X && kb < g.kbytes) v = (uint32_t)((pfx0 + lane) * g.ldx + kb);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void_t *)sink, 4, v, 0, 0, 0);
    };

    Acc acc[FM][FN];
    Frag xa[FM], wa[FN], xb[FM], wb[FN];
    // Fragment i of a half is 16 rows below fragment 0 and, as wm0, wn0 and 16 are multiples
    // of 8, has the same swizzle: one lane offset per operand and half, plus a constant.
    static_assert(TM % 8 == 0 && TN % 8 == 0, "fragment rows keep the swizzle of the first");
    const uint32_t fx0 = swz_off(wm0 + frow, fchunk), fx1 = swz_off(wm0 + frow, 4 + fchunk);
    const uint32_t fw0 = swz_off(wn0 + frow, fchunk), fw1 = swz_off(wn0 + frow, 4 + fchunk);
    auto frag = [&](const uint8_t *xbuf, const uint8_t *wbuf, bool isw, int i, int half) -> Frag {
        const uint32_t off = isw ? (half ? fw1 : fw0) : (half ? fx1 : fx0);
        return __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4 *>((isw ? wbuf : xbuf) + off + i * 16 * KT_BYTES));
    };
    // One half-step: the MFMAs on (x, w) in NR groups; after each group the next RP fragments
    // of the other set are read from (rxb, rwb), weight fragments first (the next half's first
    // MFMAs take all of them and the first activation fragment), and in the second half DMA
    // instruction q of the activation's step dkt into dxb and of the weight's step dkt + WS - 2
    // into dwb.  The first half reads two fragments per group
    // (RP = 2), so its reads are done by mid-half and the wait for them before the barrier
    // finds them landed; the second half, whose DMAs share the groups, reads one per group.
    auto half = [&](const Frag *x, const Frag *w, Frag *lx, Frag *lw, const uint8_t *rxb, const uint8_t *rwb,
                    int rhalf, bool with_dma, int dkt, uint8_t *dxb, uint8_t *dwb) {
        const int RP = with_dma ? 1 : 2;  // a constant at each (inlined) call
#pragma unroll
        for (int q = 0; q < NR; ++q) {
#pragma unroll
            for (int i = q * NM / NR; i < (q + 1) * NM / NR; ++i) Op::mfma_acc(acc[i / FN][i % FN], w[i % FN], x[i / FN]);
#pragma unroll
            for (int r = q * RP; r < (q + 1) * RP && r < NR; ++r) {
                if (r < FN) lw[r] = frag(rxb, rwb, true, r, rhalf);
                else lx[r - FN] = frag(rxb, rwb, false, r - FN, rhalf);
            }
            if (with_dma) dma(dkt, dxb, dkt + WS - 2, dwb, q);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto landed = [&](const Frag *xf, const Frag *wf) {
#pragma unroll
        for (int a = 0; a < FM; ++a) asm volatile("" ::"v"(xf[a]));
#pragma unroll
        for (int b = 0; b < FN; ++b) asm volatile("" ::"v"(wf[b]));
    };
    // Waits for step kt+1: what may stay in flight is the newest prefetch and, with a three-step
    // weight ring, the weight DMAs of step kt+2 (the last NB DMAs of the previous step).
    constexpr int INFLIGHT = (PF > 0 ? 1 : 0) + (WS == 3 ? NB : 0);
    auto barrier = [&]() {
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(INFLIGHT) : "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // Step kt reads (xc, wc); step kt+1 lands in (xn, wn); the activation's step kt+2 goes into xc
    // and the weight's step kt+WS into wc once every wave has passed this step's barrier.
    auto kstep = [&](int kt, uint8_t *xc, uint8_t *wc, uint8_t *xn, uint8_t *wn) {
        if (PF > 0) prefetch(kt + PF);  // past the end: out of range, reads nothing
        __builtin_amdgcn_sched_barrier(0);
        half(xa, wa, xb, wb, xc, wc, 1, false, 0, nullptr, nullptr);
        landed(xb, wb);
        barrier();
        // Unconditional (one basic block): after the last step the reads fetch a buffer
        // nobody uses and the DMA offsets are out of range (zero fill of this wave's own
        // groups, ahead of its next tile's DMA into them).
        // No wait here: each MFMA of the next half waits (in the compiler's counts) only for
        // the fragments it takes, and the reads land in the order the MFMAs take them.
        half(xb, wb, xa, wa, xn, wn, 0, true, kt + 2, xc, wc);
    };
    // Epilogue: lane holds out[m0+wm0+a*16+(lane&15)][n0+wn0+b*16+4*(lane>>4) + 0..3].
    // Ops with per-row and per-column epilogue operands (Op::STAGED) have them DMA'd into
    // LDS at the start of each tile (Op::stage), so the epilogue reads LDS instead of
    // waiting on global loads behind the next tile's DMA.  Two areas alternate by tile:
    // a tile's staging never lands where the previous tile's epilogue still reads.
    float *const stage_area = reinterpret_cast<float *>(smem + MAIN + PF_BYTES);
    auto store_tile = [&](int m0, int n0, int par) {
        constexpr int LAST = (NR - 1) * NM / NR;  // first MFMA of the last group
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[LAST / FN][LAST % FN]));
#pragma unroll
        for (int i = LAST + 1; i < NM; ++i) asm volatile("" : "+a"(acc[i / FN][i % FN]));
        const float *srow = stage_area + par * STAGE_FLOATS, *scol = srow + BM;
#pragma unroll
        for (int a = 0; a < FM; ++a) {
            const int mrow = m0 + wm0 + a * 16 + frow;
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int ncol = n0 + wn0 + b * 16 + fchunk * 4;
                if (mrow < g.m_pad && ncol < g.n) {
                    if constexpr (Op::STAGED)
                        op.store_staged(acc[a][b], mrow, ncol, srow[mrow - m0],
                                        *reinterpret_cast<const f32x4 *>(scol + (ncol - n0)));
                    else
                        op.store(acc[a][b], mrow, ncol);
                }
            }
        }
    };

    // A finished tile through LDS (no K step may be in flight): each lane writes its 4-column
    // pieces into a row-major copy of the tile, then the workgroup stores whole rows, 16 bytes
    // per lane.  Ends with the LDS free again.
    auto store_tile_lds = [&](int m0, int n0, int p) {
        constexpr int ROWB = BN * 2 + 16;  // tile row in LDS, padded so that 16 rows fall on distinct banks
        constexpr int CPR = BN / 8;        // 16-byte chunks per tile row
        static_assert(BM * ROWB <= MAIN, "the tile copy fits the engine's LDS");
        constexpr int LAST = (NR - 1) * NM / NR;
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[LAST / FN][LAST % FN]));
#pragma unroll
        for (int i = LAST + 1; i < NM; ++i) asm volatile("" : "+a"(acc[i / FN][i % FN]));
        const float *srow = stage_area + p * STAGE_FLOATS, *scol = srow + BM;  // staged Ops only
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the last steps' out-of-range DMAs into LDS
        __syncthreads();  // every wave's DMAs have landed and its fragment reads are done
        // The lane's first byte in the copy, formed here from a lane index the compiler cannot see
        // through: hoisted to the kernel's start, the per-row addresses outlive the K loop in
        // scratch memory, and each reload here is a memory round trip.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t cbase = (uint32_t)((wm0 + (ln & 15)) * ROWB + (wn0 + (ln >> 4) * 4) * 2);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                const int r = wm0 + a * 16 + frow, c = wn0 + b * 16 + fchunk * 4;
                u32x2 v;
                if constexpr (Op::STAGED)
                    v = op.pack_staged(acc[a][b], srow[r], *reinterpret_cast<const f32x4 *>(scol + c));
                else
                    v = Op::pack(acc[a][b]);
                *reinterpret_cast<u32x2 *>(smem + cbase + (a * 16 * ROWB + b * 16 * 2)) = v;
            }
        __syncthreads();
        // Each thread stores PER chunks, in batches of SB whose LDS reads are all issued before
        // the batch's stores, so a store never waits alone for its read.
        constexpr int PER = BM * CPR / (NW * 64), SB = PER / 4;
        static_assert(PER * NW * 64 == BM * CPR && SB * 4 == PER, "whole batches of chunks per thread");
#pragma unroll 1
        for (int b0 = 0; b0 < PER; b0 += SB) {
            u32x4 v[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int i = tid + (b0 + u) * NW * 64, r = i / CPR, c = i - r * CPR;
                v[u] = *reinterpret_cast<const u32x4 *>(smem + r * ROWB + c * 16);
            }
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int i = tid + (b0 + u) * NW * 64, r = i / CPR, c = i - r * CPR;
                if (m0 + r < g.m_pad && n0 + c * 8 < g.n) op.store16(m0 + r, n0 + c * 8, v[u]);
            }
        }
        __syncthreads();  // every wave's reads of the copy have returned before LDS is reused
    };
    const bool co = op.coalesced_final();  // uniform: a kernel argument

    int pm0 = 0, pn0 = 0, par = 0;
    bool have_prev = false;
    for (int t = blockIdx.x; t < total; t += gridDim.x) {
        int tm, tn;
        tile_of_block(t, nt_m, nt_n, g.group_m, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        sx = tile_span(g.x, m0, g.m, g.ldx, g.kbytes);
        sw = tile_span(g.w, n0, g.n, g.ldw, g.kbytes);
        rx = span_rsrc(sx, true);
        rw = span_rsrc(sw, true);
        pfx0 = (tn % PF_SHARE_X) * (BM / PF_SHARE_X);
        // (staged Ops keep the direct store between tiles: the second copy of the LDS path
        // pushes the int8 kernel's registers into spills)
        const bool lds_store = CO_LOOP && !Op::STAGED && co && have_prev;  // uniform
        if (lds_store) {  // the previous tile goes out first, through LDS
            store_tile_lds(pm0, pn0, par);
            par = 1 - par;
        }
        if constexpr (Op::STAGED) {
            float *srow = stage_area + (have_prev && !lds_store ? 1 - par : par) * STAGE_FLOATS;
            op.stage(srow, srow + BM, m0, n0, wave, lane);  // lands before this prologue's barrier
        }
        for (int d = 2; d < PF; ++d) prefetch(d);
#pragma unroll
        for (int j = 0; j < NR; ++j) dma(0, X0, 0, W0, j);  // the previous tile's reads all ended at its barriers
        if (have_prev && !lds_store) {
            store_tile(pm0, pn0, par);
            par = 1 - par;
        }
#pragma unroll
        for (int j = 0; j < NR; ++j) dma(1, X1, 1, W1, j);  // out of range (zeros) past the last step
        if constexpr (WS == 3) {
#pragma unroll
            for (int j = NA; j < NR; ++j) dma(0, X0, 2, W2, j);  // weight groups only
        }
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b) {
                acc[a][b] = Op::zero();
                asm volatile("" : "+a"(acc[a][b]));
            }
        // step 0 and the stores have landed (step 1's NR DMAs and the weight's step 2 may still
        // be in flight); the s_nop separates the accumulator writes from the first MFMA
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier\n\ts_nop 4" ::"n"(NR + (WS == 3 ? NB : 0)) : "memory");
#pragma unroll
        for (int a = 0; a < FM; ++a) xa[a] = frag(X0, W0, false, a, 0);
#pragma unroll
        for (int b = 0; b < FN; ++b) wa[b] = frag(X0, W0, true, b, 0);
        landed(xa, wa);
        if constexpr (WS == 3) {
            for (int kt = 0; kt < ksteps; kt += 6) {
                kstep(kt, X0, W0, X1, W1);
                if (kt + 1 < ksteps) kstep(kt + 1, X1, W1, X0, W2);
                if (kt + 2 < ksteps) kstep(kt + 2, X0, W2, X1, W0);
                if (kt + 3 < ksteps) kstep(kt + 3, X1, W0, X0, W1);
                if (kt + 4 < ksteps) kstep(kt + 4, X0, W1, X1, W2);
                if (kt + 5 < ksteps) kstep(kt + 5, X1, W2, X0, W0);
            }
        } else {
            for (int kt = 0; kt < ksteps; kt += 2) {
                kstep(kt, X0, W0, X1, W1);
                if (kt + 1 < ksteps) kstep(kt + 1, X1, W1, X0, W0);
            }
        }
        pm0 = m0;
        pn0 = n0;
        have_prev = true;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS write in flight when the workgroup retires
    if (have_prev) {  // uniform over the workgroup
        if (co) store_tile_lds(pm0, pn0, par);
        else store_tile(pm0, pn0, par);
    }
}

// Grid of the persistent tile loop.
__host__ __device__ inline int persistent_grid(int tiles) { return tiles < NUM_CU ? tiles : NUM_CU; }

}  // namespace rpl
