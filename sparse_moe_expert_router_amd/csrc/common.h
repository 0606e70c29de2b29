// Internal helpers shared by the HIP kernels of libmoe (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// True when either bf16 of a packed pair is denormal (exponent field 0,
// mantissa not 0).
__device__ __forceinline__ bool bf16x2_has_denormal(uint32_t w) {
    const bool lo = (w & 0x7F80u) == 0 && (w & 0x007Fu) != 0;
    const bool hi = (w & 0x7F800000u) == 0 && (w & 0x007F0000u) != 0;
    return lo || hi;
}

// Round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// A 16-byte load of data that is read once per call (expert weights streamed
// at decode), with the non-temporal hint: the lines do not displace data that
// is reused (the staged activations, the scales, the outputs).  Measured on
// the 16-token decode layers, routed call: bf16 243 -> 221 us, FP8 140 ->
// 127 us, output-major AWQ 104 -> 96 us; NVFP4 unchanged.
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// A 16-byte store with the non-temporal hint, for outputs that are written
// once and read once by a later kernel (the prefill GEMMs' h and rows: the
// pruned 32768-token layer 4.51 -> 4.44 ms a step).
__device__ __forceinline__ void st_stream(void* p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// Two floats to a packed bf16 pair with one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// v_dot2_f32_bf16: a.lo*b.lo + a.hi*b.hi + c
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (a & m) | c as one v_and_or_b32.  A VOP3 instruction on gfx9 takes no
// literal operand, so with both constants written as literals the compiler
// falls back to a separate AND and OR; here the mask travels in a VGPR and
// the constant in an SGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "s"(c));
    return r;
}

// silu(a) = a / (1 + e^-a) with the hardware base-2 exponential and
// reciprocal (v_exp_f32, v_rcp_f32, each within about one ulp): a few ulp of
// fp32 in all, far below the bf16 rounding that every caller applies to
// silu(gate) * up.  Large negative a gives e^-a = inf and a * 0 = -0.
__device__ __forceinline__ float silu(float a) {
    const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);  // log2(e)
    return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// Which group of a segmented list (offsets[0..n], non-decreasing) holds item `i`:
// the largest g with offsets[g] <= i, restricted to non-empty groups.
__device__ __forceinline__ int find_group(const int32_t* offsets, int n, int i) {
    int lo = 0, hi = n;  // offsets[lo] <= i < offsets[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (offsets[mid] <= i) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) { return __shfl_xor(v, m, kWave); }

// Maximum of v over the 64 lanes of a wave whose lanes are all active; the
// result is uniform.  Four DPP steps inside each row of 16 lanes (swap
// neighbours, swap pairs, mirror the half-row, mirror the row) leave the row
// maximum in every lane of the row; the four rows are then read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// One DPP move of an fp64 value (both 32-bit halves).
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, kCtrl, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), kCtrl, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum of v over the 64 lanes of a wave whose lanes are all active (fp64,
// one fixed order); the result is uniform.  The same four DPP steps as
// wave_max_u32, then the four row sums.
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<0xB1>(v);   // quad_perm 1,0,3,2
    v += dpp_f64<0x4E>(v);   // quad_perm 2,3,0,1
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

}  // namespace moe
