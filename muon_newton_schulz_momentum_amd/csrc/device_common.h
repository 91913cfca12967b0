// Device helpers shared by the libmuon kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace muon {
namespace dev {

// float32 -> bfloat16 bits, round to nearest, ties to even.  Adding 0x7FFF plus the
// lowest kept bit to the 32-bit pattern carries into the kept half exactly when the
// dropped half is above the midpoint, or at it with an odd kept half.  NaNs stay NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float64 -> bfloat16 bits with one rounding (to nearest, ties to even), so that a value
// computed in float64 is not rounded twice on its way to bf16.
//  * In bf16's normal range (|x| >= 2^-126) the 52-bit fraction is rounded to 7 bits on
//    the integer pattern (the carry may step the exponent up); the result has at most
//    8 significant bits and converts to float32 exactly, or to infinity past 2^128.
//  * Below 2^-126 the step is a fixed 2^-133: scale, round half-even, scale back.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t bexp = (uint32_t)(u >> 52) & 0x7ffu;
    if (bexp == 0x7ffu) {
        const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
        return (u & 0x000fffffffffffffull) ? (uint16_t)(sign | 0x7fc0u) : (uint16_t)(sign | 0x7f80u);
    }
    if (bexp >= 1023u - 126u) {
        u += 0x00000fffffffffffull + ((u >> 45) & 1ull);
        u &= ~0x00001fffffffffffull;
        const float f = (float)__longlong_as_double((long long)u);
        return (uint16_t)(__float_as_uint(f) >> 16);
    }
    const double r = ldexp(rint(ldexp(x, 133)), -133);
    return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// The epilogue combine of the Newton–Schulz products, alpha * E + gamma * P, as one
// pinned sequence: gamma * P rounded to float32, then one fused multiply-add.  Written out
// so that every kernel (tiled or fused) rounds it the same way, whatever the compiler
// would contract on its own.
__device__ __forceinline__ float ns_combine(float alpha, float e, float gamma, float prod) {
    return __builtin_fmaf(alpha, e, gamma * prod);
}

// Sum over the 64 lanes of a wavefront by butterfly.  The order of additions is fixed,
// so the result is the same on every run (no atomics anywhere in the reductions).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace dev
}  // namespace muon
