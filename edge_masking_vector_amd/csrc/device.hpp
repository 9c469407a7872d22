// device.hpp -- gfx950 device helpers shared by the tilemap kernels: 16-byte vector access,
// masked loads, and wavefront reductions built from DPP, ds_swizzle and readlane.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tmk {

constexpr int kBlock = 256;      // threads per workgroup of the reductions: four wave64s
constexpr int kMaxBlock = 1024;  // largest workgroup (the maps: up to one 1024-chunk tile block)
constexpr float kMaxFill = -1.0e30f;  // masked-max fill, f32 bits 0xF149F2CA

typedef float f4 __attribute__((ext_vector_type(4)));

// 16-byte load / store (global_load_dwordx4 / global_store_dwordx4); p must be 16-byte aligned.
__device__ __forceinline__ f4 ld16(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st16(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }

// Streaming variants with the non-temporal hint (the `nt` bit): data touched once is not kept in
// the caches.  Same values, same ordering; only the cache policy differs.
__device__ __forceinline__ f4 ld16_nt(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
}
__device__ __forceinline__ void st16_nt(float *p, f4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f4 *>(p));
}
__device__ __forceinline__ float ld4_nt(const float *p) { return __builtin_nontemporal_load(p); }

// 16-byte load from a 4-byte aligned address (one global_load_dwordx4: the HSA ABI runs the GPU in
// its unaligned access mode, so a vector access need only be aligned to its element).
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ f4 ld16u_nt(const float *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f4u *>(p));
}
__device__ __forceinline__ f4 ld16u(const float *p) { return *reinterpret_cast<const f4u *>(p); }
__device__ __forceinline__ void st4_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }

// One contiguous block of `bytes` bytes addressed through a buffer resource (raw buffer: stride 0,
// 32-bit data format in the fourth descriptor word); a store at or past `bytes` is dropped by the
// hardware's range check.  Stores carry the device-scope (sc1) and non-temporal (nt) cache-policy
// bits: the same values and ordering as plain stores.
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kPolicyDeviceStream = 16 | 2;  // sc1 | nt
constexpr int kPolicyStream = 2;              // nt
__device__ __forceinline__ __amdgpu_buffer_rsrc_t segment_rsrc(const float *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, bytes, kRawBufferWord3);
}
__device__ __forceinline__ void st16_seg(__amdgpu_buffer_rsrc_t r, int byte_off, f4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, byte_off, 0, kPolicyDeviceStream);
}
__device__ __forceinline__ void st4_seg(__amdgpu_buffer_rsrc_t r, int byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, byte_off, 0, kPolicyDeviceStream);
}

// a / d and a % d for a 32-bit a and a fixed divisor d, given c = ceil(2^64 / d) (0 when d = 1):
// the multiply-high method of Lemire, Kaser and Kurz ("Faster remainder by direct computation",
// 2019), exact for every 32-bit a.  A handful of scalar instructions where a run-time division
// takes dozens.
__device__ __forceinline__ uint32_t fast_div(uint32_t a, uint64_t c, uint32_t d) {
    return d == 1 ? a : static_cast<uint32_t>(__umul64hi(c, a));
}
__device__ __forceinline__ uint32_t fast_mod(uint32_t a, uint64_t c, uint32_t d) {
    return d == 1 ? 0u : static_cast<uint32_t>(__umul64hi(c * a, d));
}

// e^x in f32 for the softmax statistics, by the change of base e^x = 2^(x * log2 e) and the
// hardware base-2 exponential (V_EXP_F32 of the CDNA ISA, about 1 ulp): two instructions where
// the math library's expf takes a dozen, which made the statistics ALU-bound.  The callers pass
// x = s - b with b the running maximum, so x <= 0; the product x * log2(e) is within about 2^-23
// of its exact value (relative), so the result is within about |x| * 1.2e-7 (relative) of e^x.
// A term's weight in the normaliser is e^x, so terms far below the maximum, where this grows,
// barely count: the sum stays within about ln(n) * 1.2e-7 for n terms.  Results below 2^-126 may
// flush to 0; such a term is under 1.2e-38 of the row's largest term (which is 1).
__device__ __forceinline__ float exp_f32(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// ---- reduction operators ------------------------------------------------------------------
struct SumOp {
    static constexpr float kFill = 0.0f;  // masked elements read as 0
    __device__ __forceinline__ static float f(float a, float b) { return a + b; }
};
struct MaxOp {
    static constexpr float kFill = kMaxFill;  // a value no real score reaches
    __device__ __forceinline__ static float f(float a, float b) { return __builtin_fmaxf(a, b); }
};

// ---- cross-lane moves ---------------------------------------------------------------------
// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] swaps lane pairs, [2,3,0,1] swaps pairs of
// pairs, row_half_mirror reverses each 8-lane half-row, row_mirror reverses each 16-lane row.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
// ds_swizzle bit-mask mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 -> lane ^ 16 within 32 lanes.
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float swizzle_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), kSwizzleXor16));
}

// Combine `v` over aligned groups of LPR consecutive lanes (LPR a power of two <= 64).  Every lane
// of a group ends with the same bits: each step combines two equal-sized halves whose values are
// uniform, and the operators are commutative.  All 64 lanes of the wave must be active.
template <class Op, int LPR>
__device__ __forceinline__ float group_reduce(float v) {
    if constexpr (LPR >= 2) v = Op::f(v, dpp<kDppXor1>(v));
    if constexpr (LPR >= 4) v = Op::f(v, dpp<kDppXor2>(v));
    if constexpr (LPR >= 8) v = Op::f(v, dpp<kDppHalfMirror>(v));
    if constexpr (LPR >= 16) v = Op::f(v, dpp<kDppMirror>(v));
    if constexpr (LPR >= 32) v = Op::f(v, swizzle_xor16(v));
    if constexpr (LPR >= 64) {
        const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
        const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
        v = Op::f(lo, hi);
    }
    return v;
}

}  // namespace tmk
