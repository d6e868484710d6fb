// Device helpers shared by the gfx950 kernels of libconvrot_amd: bf16 conversion, the fixed fp32
// exponential, wave reductions and the XCD-aware tile mapping.
//
// Built with -ffp-contract=off: every fp32 expression below is evaluated as separate IEEE operations in
// the order written (fused multiply-adds only where written explicitly), which is what makes the kernels
// reproducible bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace crk {

constexpr int kWave = 64;  // CDNA wavefront width

__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t float_to_bf16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 values -> packed bf16 (lo in bits 0-15), same rounding, one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// The library's fixed fp32 exponential E(x): Cody-Waite reduction x = n ln2 + r with ln2 split into a
// 16-significant-bit head (n * head exact for |n| < 256) and an fp32 tail (one fused multiply-add each), e^r
// from the Taylor series through r^7 (coefficients 1/k! rounded to fp32) by Horner's rule in fused
// multiply-adds, and p * 2^n rounded once: exact scaling for a normal result; for a subnormal one (n < -126)
// an exact scale by 2^(n+100) and one IEEE multiply by 2^-100, so the single rounding does not depend on how
// the scaling instruction treats subnormal results.  E therefore underflows through the subnormals to 0 below
// about -103.97 and overflows to +inf above about 88.72, as the fp32 rounding of e^x does.  The argument is
// clamped to [-150, 100] first, which keeps |n| < 256 and changes no result.
__device__ __forceinline__ float exp_fixed(float x) {
    const float kLog2e = 0x1.715476p+0f;
    const float kLn2Hi = 0x1.62e4p-1f;
    const float kLn2Lo = 0x1.7f7d1cp-20f;
    x = __builtin_amdgcn_fmed3f(x, -150.0f, 100.0f);
    const float n = rintf(x * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, x);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = 1.0f / 5040.0f;
    p = __builtin_fmaf(p, r, 1.0f / 720.0f);
    p = __builtin_fmaf(p, r, 1.0f / 120.0f);
    p = __builtin_fmaf(p, r, 1.0f / 24.0f);
    p = __builtin_fmaf(p, r, 1.0f / 6.0f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    const int ni = (int)n;
    const bool sub = ni < -126;
    return __builtin_amdgcn_ldexpf(p, sub ? ni + 100 : ni) * (sub ? 0x1p-100f : 1.0f);
}

// silu(g) = g / (1 + E(-g)); below g = -64, where 1 + E(g) is exactly 1 in fp32, the same value is g * E(g),
// which does not overflow.
__device__ __forceinline__ float silu_fixed(float g) {
    if (g < -64.0f) return g * exp_fixed(g);
    float e = exp_fixed(-g);
    float den = 1.0f + e;
    return g / den;
}

// Maximum over the wavefront (all lanes active), wave-uniform result: DPP quad permutations and row rotations
// leave every lane with its 16-lane row's maximum, then four lane reads combine the rows.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));   // 1,0,3,2
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));   // 2,3,0,1
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));  // row_ror:4
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));  // row_ror:8
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m);
    return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD i % 8).  Remap the
// hardware workgroup id so that each XCD receives a contiguous range of logical tiles: consecutive tiles
// (the N-tiles of one expert) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
    constexpr int kXcd = 8;
    int xcd = hw_id % kXcd;
    int local = hw_id / kXcd;
    int base = total / kXcd, extra = total % kXcd;
    int start = xcd * base + (xcd < extra ? xcd : extra);
    return start + local;
}

}  // namespace crk
