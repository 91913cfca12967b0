// Device helpers shared by the libmuon kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace muon {
namespace dev {

// float32 -> bfloat16 bits, round to nearest, ties to even, by gfx950's packed
// conversion instruction (v_cvt_pk_bf16_f32).  It was checked on the device over all 2^32
// float32 patterns against the integer formulation -- add 0x7FFF plus the lowest kept bit
// to the 32-bit pattern (a carry into the kept half exactly when the dropped half is above
// the midpoint, or at it with an odd kept half); a NaN becomes the quiet NaN with the same
// sign and top payload bits -- with no difference, denormals and NaNs included.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two values in one instruction: lo in bits 0..15, hi in bits 16..31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.0f); }

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
