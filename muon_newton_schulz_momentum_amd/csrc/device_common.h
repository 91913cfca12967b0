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

// A positive float64 value rounded to float32 "to odd": the float32 value nearest d when d
// is one, otherwise whichever of its two float32 neighbours has an odd significand.  With
// 24 significant bits against bfloat16's 8, rounding that value to bf16 (to nearest even)
// is the one rounding of d to bf16.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
    const float f = (float)d;
    const double back = (double)f;
    if (back == d || (__float_as_uint(f) & 1u)) return f;
    return __uint_as_float(__float_as_uint(f) + (back < d ? 1u : 0xffffffffu));
}

// The float32 scale s of a matrix's normalisation X = bf16(X0 * s) (normalize8): the float32
// value nearest inv for which bf16(f32(m * s)) = bf16(m * inv), with m * inv rounded once
// from its float64 product, for each of the 128 bf16 significands m in [1, 2).  Scaling by a
// power of two changes neither rounding while the values stay normal, so with that s the
// float32 products give every normal-range element of X as X0 * inv rounded once.  One whole
// wave calls this with the same inv (each lane checks two significands) and gets the same s;
// candidates are f32(inv) moved by 0, +1, -1, ..., +8, -8 units of its last place (a move of
// more than 2 was never needed over 2 million random normalisers); if none fits, or inv is
// not a positive float32-range number, the result is f32(inv).
__device__ __forceinline__ float exact_scale(double inv) {
    const float s0 = (float)inv;
    if (!(inv > 0.0) || !(inv <= 3.4028234663852886e38)) return s0;
    const int lane = threadIdx.x & 63;
    const float m0 = 1.0f + (float)lane * 0.0078125f, m1 = m0 + 0.5f;
    const uint16_t t0 = f32_to_bf16(f64_to_f32_odd((double)m0 * inv));
    const uint16_t t1 = f32_to_bf16(f64_to_f32_odd((double)m1 * inv));
    for (int k = 0; k <= 16; ++k) {
        const int d = (k & 1) ? (k + 1) / 2 : -(k / 2);
        const float s = __uint_as_float(__float_as_uint(s0) + (uint32_t)d);
        const bool ok = f32_to_bf16(m0 * s) == t0 && f32_to_bf16(m1 * s) == t1;
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) return s;
    }
    return s0;
}

// The normalisation of one 16-byte unit of 8 bf16 values: X = bf16(X0 * s) for the matrix's
// scale s (exact_scale), each product in float32 and rounded to bf16 by the packed
// conversion; elements from `valid` on (the padding past the matrix's last column) are zero.
// Every kernel that normalises (one stream, side stream, grouped, fused small matrices, the
// first product iteration's loads) uses this arithmetic, so their results agree bitwise.
__device__ __forceinline__ uint4 normalize8(uint4 in, int32_t valid, float s) {
    const uint32_t w[4] = {in.x, in.y, in.z, in.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t y = f32x2_to_bf16x2(__uint_as_float(w[j] << 16) * s, __uint_as_float(w[j] & 0xffff0000u) * s);
        if (2 * j + 1 >= valid) y &= (2 * j < valid) ? 0x0000ffffu : 0u;
        o[j] = y;
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// The same normalisation for 4 values (8 bytes): per element exactly what normalize8 does,
// so a fused path that normalises the values it loads agrees bitwise with the separate pass.
__device__ __forceinline__ uint2 normalize4(uint2 in, int32_t valid, float s) {
    const uint32_t w[2] = {in.x, in.y};
    uint32_t o[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        uint32_t y = f32x2_to_bf16x2(__uint_as_float(w[j] << 16) * s, __uint_as_float(w[j] & 0xffff0000u) * s);
        if (2 * j + 1 >= valid) y &= (2 * j < valid) ? 0x0000ffffu : 0u;
        o[j] = y;
    }
    return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

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
