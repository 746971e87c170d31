// rpl_device.h -- device-side helpers shared by the gfx950 kernels of librpl.
//
// Vector types for 16-byte global/LDS traffic and for the MFMA operands, and
// bfloat16 <-> fp32 conversions.  fp32 -> bf16 uses the compiler's __bf16
// conversion, which gfx950 lowers to v_cvt_pk_bf16_f32 (round to nearest,
// ties to even); bf16 -> fp32 is exact (a shift).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rpl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (low half = a), nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 h = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// Packed bf16 pair -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// 16-byte global load / store (the address must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ void st8(void *p, u32x2 v) { *reinterpret_cast<u32x2 *>(p) = v; }
// Streaming (non-temporal) stores, for large outputs: their lines leave for HBM while the
// producer runs instead of staying dirty in the 256 MB memory-side cache, where the next
// kernel's reads would pay for their write-back.  Measured on MI355X: after a partial product
// that wrote 168 MB with ordinary stores, the next 230 MB chunk reduce took 58 us, against
// 43 us after one that wrote the same bytes with these stores.
__device__ __forceinline__ void st16_nt(void *p, u32x4 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p)); }
__device__ __forceinline__ void st8_nt(void *p, u32x2 v) { __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p)); }
// Streaming (non-temporal) load, for inputs read once in volumes beyond what the memory-side
// cache could keep for a later reader.  Measured on MI355X (bench steps, inputs rotated beyond
// twice that cache): the 230 MB long-prefill chunk reduce 43.8 -> 41.0 us, the 73 MB prefill chunk
// reduce 14.7 -> 14.2 us, the 335 MB token-row gather 57.3 -> 54.2 us; not used where it measured
// slower (the quantiser +3%, the all-reduce sum and the hidden-split step 1 +1-2%).
__device__ __forceinline__ u32x4 ld16_nt(const void *p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)); }

// Lane i of the result takes lane i + SH of v within each row of 16 lanes (zero past the
// row): a DPP row shift, which moves an MFMA operand fragment between token-row lanes.
template <int SH>
__device__ __forceinline__ u32x4 lanes_down(u32x4 v) {
    static_assert(SH > 0 && SH < 16, "a row shift");
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_update_dpp(0u, v[q], 0x100 + SH, 0xF, 0xF, true);
    return r;
}

}  // namespace rpl
