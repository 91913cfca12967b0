// Batched Newton–Schulz products on gfx950 matrix cores (bf16 MFMA, float32 accumulate).
//
// One quintic Newton–Schulz step on a canonical m x n matrix X (m <= n) is
//     A = X X^T,   B = b A + c A A,   X' = a X + B X.
// The pages run this on whole momentum matrices with an operator built for the
// symmetric intermediates ("Frontier Pre-training at Microsoft AI", method details
// section 5, resharding step 3; "symmetry-aware Newton–Schulz kernels" in the recipe
// page's section "How to Make Parameter Updates Faster and More Stable?").  Here:
//   * NS_SYRK  A = X X^T: only tiles (i, j) with i <= j are computed; each off-diagonal
//              tile is stored twice (as itself and mirrored), so A is exactly symmetric.
//   * NS_POLY  B = b A + c A A^T: A is symmetric, so A A = A A^T and the same
//              upper-triangle scheme applies; b A is added in the epilogue.
//   * NS_AXPY  X' = a X + B X: a full GEMM with the axpy fused into its epilogue.
//
// All three share one main loop: a TILE x TILE output tile per workgroup, K in steps of
// 64, operands staged through LDS in two buffers (the next step's global loads are in
// flight while the current step's MFMAs run), v_mfma_f32_32x32x16_bf16 on 32 x 32
// sub-tiles.  Both operands are stored in LDS with K contiguous (row stride 72 bf16 =
// 144 B, which spreads the 16-byte MFMA operand reads of 8 consecutive rows over all
// banks).  In NS_AXPY the right operand X is K x N with N contiguous in memory: each
// thread loads an 8 x 8 bf16 block and transposes it in registers before the LDS store.
//
// Matrices are padded to multiples of TILE with zero rows and columns, so no kernel
// needs a bounds check: zero padding stays zero through all three products.
//
// Workgroups are remapped so that the tiles of one matrix run on the same XCD (the
// hardware hands consecutive workgroup ids to the 8 XCDs in turn), keeping a matrix's
// panels in that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int NUM_XCD = 8;

__device__ __forceinline__ int xcd_remap(int b, int g) {
    const int xcd = b % NUM_XCD, local = b / NUM_XCD;
    const int q = g / NUM_XCD, r = g % NUM_XCD;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Upper-triangle tile t of a T x T tile grid, row-major: row i holds tiles (i, i..T-1).
__device__ __forceinline__ void tri_decode(int t, int T, int& ti, int& tj) {
    int i = 0;
    while (t >= T - i) { t -= T - i; ++i; }
    ti = i;
    tj = i + t;
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

template <int MODE, int TILE, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void ns_gemm_kernel(NsArgs p) {
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = TILE / WM, WTN = TILE / WN;  // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;      // 32 x 32 MFMA blocks per wave
    constexpr int CH = TILE * (BK / 8) / NT;         // 16-byte chunks per thread per operand
    constexpr int NBLK = (BK / 8) * (TILE / 8);      // 8 x 8 blocks of the K x N operand
    static_assert(FM >= 1 && FN >= 1 && CH >= 1, "tile configuration");
    static_assert(NBLK <= NT, "one transpose block per thread at most");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][TILE * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    const int b = xcd_remap(blockIdx.x, gridDim.x);
    const int mat = b / p.tiles_per_mat;
    const int t = b - mat * p.tiles_per_mat;
    int ti, tj;
    if (MODE == NS_AXPY) {
        ti = t / p.tiles_n;
        tj = t - ti * p.tiles_n;
    } else {
        tri_decode(t, p.tiles_m, ti, tj);
    }

    const uint16_t* Ag = p.opa + (int64_t)mat * p.stride_a + (int64_t)ti * TILE * p.lda;
    const uint16_t* Bg = (MODE == NS_AXPY)
                             ? p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE
                             : p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE * p.ldb;

    uint4 ra[CH], rb[CH];
    uint4 rt[8];
    const int kg = tid & 7, ng = tid >> 3;   // transpose block of this thread (NS_AXPY)

    auto gload = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * NT, row = idx >> 3, ch = idx & 7;
            ra[i] = *reinterpret_cast<const uint4*>(Ag + (int64_t)row * p.lda + k0 + ch * 8);
        }
        if (MODE != NS_AXPY) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int idx = tid + i * NT, row = idx >> 3, ch = idx & 7;
                rb[i] = *reinterpret_cast<const uint4*>(Bg + (int64_t)row * p.ldb + k0 + ch * 8);
            }
        } else if (tid < NBLK) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                rt[r] = *reinterpret_cast<const uint4*>(Bg + (int64_t)(k0 + kg * 8 + r) * p.ldb + ng * 8);
        }
    };

    auto lstore = [&](int s) {
        uint16_t* As = smem[s][0];
        uint16_t* Bs = smem[s][1];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int idx = tid + i * NT, row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<uint4*>(As + row * LDK + ch * 8) = ra[i];
        }
        if (MODE != NS_AXPY) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int idx = tid + i * NT, row = idx >> 3, ch = idx & 7;
                *reinterpret_cast<uint4*>(Bs + row * LDK + ch * 8) = rb[i];
            }
        } else if (tid < NBLK) {
            // rt[r] holds row k0+kg*8+r, columns ng*8..ng*8+7 (two bf16 per dword).
            // Column j of the block becomes LDS row ng*8+j, K positions kg*8..kg*8+7.
            const uint32_t* v = reinterpret_cast<const uint32_t*>(rt);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int dw = j >> 1;
                uint4 w;
                if ((j & 1) == 0) {
                    w.x = lo_pair(v[0 * 4 + dw], v[1 * 4 + dw]);
                    w.y = lo_pair(v[2 * 4 + dw], v[3 * 4 + dw]);
                    w.z = lo_pair(v[4 * 4 + dw], v[5 * 4 + dw]);
                    w.w = lo_pair(v[6 * 4 + dw], v[7 * 4 + dw]);
                } else {
                    w.x = hi_pair(v[0 * 4 + dw], v[1 * 4 + dw]);
                    w.y = hi_pair(v[2 * 4 + dw], v[3 * 4 + dw]);
                    w.z = hi_pair(v[4 * 4 + dw], v[5 * 4 + dw]);
                    w.w = hi_pair(v[6 * 4 + dw], v[7 * 4 + dw]);
                }
                *reinterpret_cast<uint4*>(Bs + (ng * 8 + j) * LDK + kg * 8) = w;
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int nk = p.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();

    const int arow = lane & 31, akoff = (lane >> 5) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint16_t* As = smem[s][0];
        const uint16_t* Bs = smem[s][1];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(As + (wm0 + i * 32 + arow) * LDK + kk * 16 + akoff);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn0 + j * 32 + arow) * LDK + kk * 16 + akoff);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(s ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds rows 8q + 4*(lane/32) + (0..3) of column lane%32 ----------
    uint16_t* out = p.out + (int64_t)mat * p.stride_o;
    const uint16_t* ep = p.ep + (int64_t)mat * p.stride_o;
    const int col_in = lane & 31, rsub = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gc = tj * TILE + wn0 + j * 32 + col_in;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gr0 = ti * TILE + wm0 + i * 32 + q * 8 + rsub;
                uint16_t h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int gr = gr0 + v;
                    float val = acc[i][j][q * 4 + v];
                    if (MODE == NS_POLY || MODE == NS_AXPY)
                        val = p.alpha * dev::bf16_to_f32(ep[(int64_t)gr * p.ldo + gc]) + p.gamma * val;
                    h[v] = dev::f32_to_bf16(val);
                    out[(int64_t)gr * p.ldo + gc] = h[v];
                }
                if (MODE != NS_AXPY && ti != tj) {
                    uint2 m2;
                    m2.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                    m2.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                    *reinterpret_cast<uint2*>(out + (int64_t)gc * p.ldo + gr0) = m2;
                }
            }
        }
    }
}

template <int MODE, int TILE, int WM, int WN>
hipError_t launch_cfg(const NsArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ns_gemm_kernel<MODE, TILE, WM, WN>), dim3((unsigned)a.total_tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int32_t tile, const NsArgs& a, hipStream_t s) {
    switch (tile) {
        case TILE_256: return launch_cfg<MODE, 256, 2, 4>(a, s);
        case TILE_128: return launch_cfg<MODE, 128, 2, 2>(a, s);
        case TILE_64: return launch_cfg<MODE, 64, 2, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_ns(NsMode mode, int32_t tile, const NsArgs& a, hipStream_t s) {
    switch (mode) {
        case NS_SYRK: return launch_mode<NS_SYRK>(tile, a, s);
        case NS_POLY: return launch_mode<NS_POLY>(tile, a, s);
        case NS_AXPY: return launch_mode<NS_AXPY>(tile, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace muon
