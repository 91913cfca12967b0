// The whole Newton–Schulz orthogonalisation of small matrices, one workgroup per matrix,
// everything in LDS (bf16 MFMA, float32 accumulate).
//
// The pages treat small, frequently replicated matrices such as MoE router weights apart
// from the bulk of the experts ("Frontier Pre-training at Microsoft AI", method details
// section 5, the router-weight note of "Scaling Muon to 16K GPUs").  On one GPU such a
// matrix is too small to fill the chip with tiles: the tiled path spends two launches on
// the normaliser and three per iteration on a handful of workgroups each.  Here a
// workgroup takes one canonical m x n matrix with m <= 64 and n (padded) <= 1024, keeps X
// (64 x n bf16), A and B (64 x 64 bf16 each) in 144 KB of LDS and runs
//     inv = 1 / (||X0||_F + eps),  X = bf16(inv * X0),
//     for t = 1..k:  A = X X^T,  B = b_t A + c_t A A,  X = a_t X + B X,
// writing only the result.  All matrices of every small chunk of a plan go in one launch.
//
// Every product accumulates its 16-wide K slices in the same order as the tiled kernels
// with 64 x 64 tiles, the epilogues apply the same float32 expressions, and the norm is
// summed in the same order as the tiled path's finalize kernel, so the result is bitwise
// the one of the tiled path.
//
// X is updated in place: X' = a X + B X needs, for an output column, only that column of
// X, and each wave owns whole 32-column blocks (it reads the block for both row halves
// before writing any of it).
#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int SM_ROWS = 64;
constexpr int X_BYTES = SM_ROWS * SMALL_NS_MAX_N * 2;   // 128 KB
constexpr int M_BYTES = SM_ROWS * SM_ROWS * 2;          // 8 KB

// ds_read_b64_tr_b16: lane 4a+b of each group of 16 receives element b of the 8-byte rows
// addressed by lanes a, a+4, a+8, a+12.
__device__ __forceinline__ bf16x4 tr16(const char* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(const __attribute__((address_space(3))) char*)p);
    return __builtin_bit_cast(bf16x4, v);
}

__global__ __launch_bounds__(256) void ns_small_kernel(SmallNsArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[X_BYTES + 2 * M_BYTES];
    __shared__ double red[4];
    __shared__ double inv_s;
    char* const X = smem;
    char* const Am = smem + X_BYTES;
    char* const Bm = Am + M_BYTES;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int jc = 0;
    while (jc + 1 < a.n_jobs && (int)blockIdx.x >= a.job[jc + 1].first) ++jc;
    const SmallJob J = a.job[jc];
    const int64_t mat = (int64_t)blockIdx.x - J.first;
    const int np = J.np, m = J.m, n = J.n;
    const int RB = np * 2;                                // bytes per X row
    const int CPR = np >> 3;                              // 16-byte chunks per X row
    // chunk swizzle mask: c ^ (r & SW) must stay inside the row, so SW + 1 divides CPR
    // (np is a multiple of 64, so CPR is a multiple of 8)
    const int SW = (CPR & 15) == 0 ? 15 : 7;
    // X element (r, c): row r, 16-byte chunk (c / 8) stored at chunk (c / 8) ^ (r & SW)
    auto xb = [&](int r, int c) { return r * RB + ((((c >> 3) ^ (r & SW))) << 4) + (c & 7) * 2; };
    // A, B element (r, c): 128-byte rows, chunk (c / 8) stored at (c / 8) ^ (r & 7)
    auto mb = [](int r, int c) { return r * 128 + ((((c >> 3) ^ (r & 7))) << 4) + (c & 7) * 2; };

    // ---- the normalisation scale, summed and searched as the finalize kernel does ------
    {
        double s = 0.0;
        for (int64_t i = tid; i < J.ew_tiles; i += 256) s += J.partials[mat * J.ew_tiles + i];
        s = dev::wave_sum(s);
        if (lane == 0) red[wave] = s;
        __syncthreads();
        if (wave == 0) {
            const double tot = (red[0] + red[1]) + (red[2] + red[3]);
            const float scale = dev::exact_scale(1.0 / (sqrt(tot) + a.eps));
            if (lane == 0) inv_s = (double)scale;
        }
        __syncthreads();
    }
    const double inv = inv_s;

    // ---- X = bf16(inv * X0) into LDS (zero outside the m x n region) -------------------
    const uint16_t* x0 = J.xq + mat * SM_ROWS * np;
    for (int u = tid; u < SM_ROWS * CPR; u += 256) {
        const int r = u / CPR, c = (u - r * CPR) * 8;
        uint4 o4 = make_uint4(0, 0, 0, 0);
        if (r < m && c < n)
            o4 = dev::normalize8(*reinterpret_cast<const uint4*>(x0 + (int64_t)r * np + c), n - c, (float)inv);
        *reinterpret_cast<uint4*>(X + xb(r, c)) = o4;
    }
    __syncthreads();

    // MFMA lane layout (v_mfma_f32_32x32x16_bf16): operand lanes supply row (lane & 31),
    // K elements 8 * (lane >> 5) + 0..7; result lane holds rows 8q + 4 * (lane >> 5) + w
    // (v = 4q + w) of column (lane & 31).
    const int lr = lane & 31, kh = lane >> 5;
    const int wi = wave >> 1, wj = wave & 1;              // this wave's 32 x 32 block of A, B
    const int tg = lane >> 4, tx = lane & 15;             // transposing-read groups

    for (int it = 0; it < a.steps; ++it) {
        // ---- A = X X^T ----------------------------------------------------------------
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
        for (int kk = 0; kk < np / 16; ++kk) {
            const int c = 16 * kk + 8 * kh;
            const bf16x8 fa = *reinterpret_cast<const bf16x8*>(X + xb(32 * wi + lr, c));
            const bf16x8 fb = *reinterpret_cast<const bf16x8*>(X + xb(32 * wj + lr, c));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 32 * wi + 8 * (v >> 2) + 4 * kh + (v & 3);
            *reinterpret_cast<uint16_t*>(Am + mb(r, 32 * wj + lr)) = dev::f32_to_bf16(acc[v]);
        }
        __syncthreads();

        // ---- B = b A + c A A^T (= b A + c A A: A is symmetric) ---------------------------
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int kk = 0; kk < SM_ROWS / 16; ++kk) {
            const int c = 16 * kk + 8 * kh;
            const bf16x8 fa = *reinterpret_cast<const bf16x8*>(Am + mb(32 * wi + lr, c));
            const bf16x8 fb = *reinterpret_cast<const bf16x8*>(Am + mb(32 * wj + lr, c));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int r = 32 * wi + 8 * (v >> 2) + 4 * kh + (v & 3);
            const float e = dev::bf16_to_f32(*reinterpret_cast<const uint16_t*>(Am + mb(r, 32 * wj + lr)));
            const float val = dev::ns_combine(a.abc[it][1], e, a.abc[it][2], acc[v]);
            *reinterpret_cast<uint16_t*>(Bm + mb(r, 32 * wj + lr)) = dev::f32_to_bf16(val);
        }
        __syncthreads();

        // ---- X = a X + B X, in place, one 32-column block per wave at a time ----------
        for (int cb = wave; cb < np / 32; cb += 4) {
            const int n0 = 32 * cb;
            f32x16 acc2[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc2[h2][v] = 0.f;
#pragma unroll
            for (int kk = 0; kk < SM_ROWS / 16; ++kk) {
                // right operand X[k][n0 + (lane & 31)], k = 16 kk + 8 (lane >> 5) + 0..7,
                // from two transposing reads of 4 K rows each
                bf16x4 t[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 16 * kk + 4 * h + 8 * (tg >> 1) + (tx >> 2);
                    const int nn = n0 + 16 * (tg & 1) + 4 * (tx & 3);
                    t[h] = tr16(X + xb(k, nn));
                }
                const bf16x8 fb = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const bf16x8 fa = *reinterpret_cast<const bf16x8*>(Bm + mb(32 * h2 + lr, 16 * kk + 8 * kh));
                    acc2[h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc2[h2], 0, 0, 0);
                }
            }
            float e[2][16];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 32 * h2 + 8 * (v >> 2) + 4 * kh + (v & 3);
                    e[h2][v] = dev::bf16_to_f32(*reinterpret_cast<const uint16_t*>(X + xb(r, n0 + lr)));
                }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 32 * h2 + 8 * (v >> 2) + 4 * kh + (v & 3);
                    const float val = dev::ns_combine(a.abc[it][0], e[h2][v], 1.f, acc2[h2][v]);
                    *reinterpret_cast<uint16_t*>(X + xb(r, n0 + lr)) = dev::f32_to_bf16(val);
                }
        }
        __syncthreads();
    }

    // ---- O = X to the chunk's output buffer ------------------------------------------------
    uint16_t* xo = J.xp + mat * SM_ROWS * np;
    for (int u = tid; u < SM_ROWS * CPR; u += 256) {
        const int r = u / CPR, c = (u - r * CPR) * 8;
        *reinterpret_cast<uint4*>(xo + (int64_t)r * np + c) = *reinterpret_cast<const uint4*>(X + xb(r, c));
    }
}

}  // namespace

hipError_t launch_ns_small(const SmallNsArgs& a, int64_t total, hipStream_t s) {
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(ns_small_kernel, dim3((unsigned)total), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
