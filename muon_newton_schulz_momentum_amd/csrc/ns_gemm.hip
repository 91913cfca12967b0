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
// Main loop (all three modes): one TILE x TILE output tile per workgroup, K in steps of
// 64, two LDS stages.  Operand tiles go from global memory straight into LDS with
// global_load_lds_dwordx4 (no VGPR staging): each lane's 16 bytes land at the
// instruction's LDS base + 16 * lane, and the lane picks which global 16 bytes to fetch,
// so the LDS image can be XOR-swizzled for conflict-free reads.  The next K step's loads
// are in flight while the current step's v_mfma_f32_32x32x16_bf16 run.
//   * Row-panel operands (K contiguous: X in SYRK, A in POLY, B in AXPY) are stored as
//     rows of 64 bf16 (128 B) whose eight 16-byte chunks are permuted by chunk ^ (row % 8);
//     an MFMA operand is one ds_read_b128 per lane.
//   * The K x N operand of NS_AXPY (X, N contiguous) is stored as rows of TILE bf16 in its
//     own orientation, with 64-byte granules permuted per row, and read with
//     ds_read_b64_tr_b16, which transposes 4 x 4 blocks of 16-bit values across each group
//     of 16 lanes into exactly the K-packed layout the MFMA wants.
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
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

constexpr int BK = 64;          // K step (bf16 elements)
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

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// vmcnt(0) and lgkmcnt(0): this wave's direct-to-LDS loads have landed and its LDS reads
// have returned, so after the barrier other waves may overwrite the stage it read.
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0x0070); }

// 16 bytes from global memory into LDS at base + 16 * lane (base wave-uniform).
__device__ __forceinline__ void load_to_lds(const uint16_t* src, uint16_t* lds_base) {
    __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)lds_base, 16, 0, 0);
}

// ds_read_b64_tr_b16 issued as inline assembly.  Through the compiler intrinsic, every
// such read would first wait for all outstanding direct-to-LDS loads (the compiler cannot
// tell that they target the other stage), which would expose the global-load latency
// once per K step.  Issued this way the compiler does not track the read; its result is
// released by lds_wait_tied() below, whose register operands carry the dependency to
// the MFMAs that consume it.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    const uint32_t addr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
    uint2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// Row of the 64-byte granule swizzle for the K x N operand: the 8 rows one transposing
// read touches (k0..k0+3 and k0+8..k0+11) get 8 different granules.
__device__ __forceinline__ int kn_swz(int k) { return (k & 3) | ((k >> 1) & 4); }

// Granule swizzle of the epilogue input tile: a transposing read there touches 8
// consecutive rows, which get 8 different granules.
__device__ __forceinline__ int ep_swz(int r) { return r & 7; }

template <int MODE, int TILE, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void ns_gemm_kernel(NsArgs p) {
    constexpr int NW = WM * WN;
    constexpr int WTM = TILE / WM, WTN = TILE / WN;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;       // 32 x 32 MFMA blocks per wave
    constexpr int PANEL = TILE * BK;                  // elements of one operand tile
    constexpr int RP_INSTR = TILE / 8;                // 1 KB load instructions per row-panel tile
    constexpr int RP_PER_WAVE = RP_INSTR / NW;
    constexpr int KN_ROWS_PER_INSTR = 512 / TILE;     // K x N tile rows per 1 KB instruction
    constexpr int KN_INSTR = BK / KN_ROWS_PER_INSTR;
    constexpr int KN_PER_WAVE = KN_INSTR / NW;
    constexpr int KN_CHUNKS = TILE / 8;               // 16-byte chunks per K x N row
    constexpr int KN_NG = TILE / 32;                  // 64-byte granules per K x N row
    static_assert(FM >= 1 && FN >= 1, "tile configuration");
    static_assert(RP_PER_WAVE >= 1 && RP_INSTR % NW == 0, "row-panel load split");
    static_assert(MODE != NS_AXPY || (KN_PER_WAVE >= 1 && KN_INSTR % NW == 0), "K x N load split");

    __shared__ __attribute__((aligned(1024))) uint16_t smem[2][2][PANEL];

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
    const bool diag = MODE != NS_AXPY && ti == tj;    // one panel serves both operands

    const uint16_t* Ag = p.opa + (int64_t)mat * p.stride_a + (int64_t)ti * TILE * p.lda;
    const uint16_t* Bg = (MODE == NS_AXPY)
                             ? p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE
                             : p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE * p.ldb;

    // ---- per-lane source offsets of the direct-to-LDS loads (fixed across K steps) ----
    // Row panel: instruction q covers rows 8q..8q+7; lane -> row 8q + lane/8, physical
    // chunk lane%8 holding logical chunk (lane%8) ^ (lane/8).
    int64_t ra_off[RP_PER_WAVE], rb_off[RP_PER_WAVE];
#pragma unroll
    for (int i = 0; i < RP_PER_WAVE; ++i) {
        const int q = wave + NW * i;
        const int row = 8 * q + (lane >> 3);
        const int chunk = (lane & 7) ^ (lane >> 3);
        ra_off[i] = (int64_t)row * p.lda + chunk * 8;
        rb_off[i] = (int64_t)row * p.ldb + chunk * 8;
    }
    // K x N panel (NS_AXPY): instruction q covers rows q*KN_ROWS_PER_INSTR..; lane ->
    // row within the instruction lane / KN_CHUNKS, physical chunk lane % KN_CHUNKS.
    int64_t kn_off[MODE == NS_AXPY ? KN_PER_WAVE : 1];
    if (MODE == NS_AXPY) {
#pragma unroll
        for (int i = 0; i < KN_PER_WAVE; ++i) {
            const int q = wave + NW * i;
            const int k = q * KN_ROWS_PER_INSTR + lane / KN_CHUNKS;
            const int pc = lane % KN_CHUNKS;
            const int g = (pc >> 2) ^ (kn_swz(k) % KN_NG);
            kn_off[i] = (int64_t)k * p.ldb + (g * 4 + (pc & 3)) * 8;
        }
    }

    auto issue_loads = [&](int kt, int s) {
        const int k0 = kt * BK;
        uint16_t* As = smem[s][0];
        uint16_t* Bs = smem[s][1];
#pragma unroll
        for (int i = 0; i < RP_PER_WAVE; ++i)
            load_to_lds(Ag + ra_off[i] + k0, As + (wave + NW * i) * 512);
        if (MODE == NS_AXPY) {
#pragma unroll
            for (int i = 0; i < KN_PER_WAVE; ++i)
                load_to_lds(Bg + kn_off[i] + (int64_t)k0 * p.ldb, Bs + (wave + NW * i) * 512);
        } else if (!diag) {
#pragma unroll
            for (int i = 0; i < RP_PER_WAVE; ++i)
                load_to_lds(Bg + rb_off[i] + k0, Bs + (wave + NW * i) * 512);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // per-lane LDS read offsets (elements)
    const int arow = lane & 31, khalf = lane >> 5;
    int a_rd[FM], b_rd[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a_rd[i] = (wm0 + i * 32 + arow) * BK;
#pragma unroll
    for (int j = 0; j < FN; ++j) b_rd[j] = (wn0 + j * 32 + arow) * BK;
    // transposing reads: lane -> (group g, index i) = (lane/16, lane%16)
    const int tg = lane >> 4, tix = lane & 15;
    const int tr_k = 8 * (tg >> 1) + (tix >> 2);          // + kk*16 + 4*h
    const int tr_n = 16 * (tg & 1) + 4 * (tix & 3);       // + wn0 + j*32

    // Fragment loads of one 16-wide K sub-step from an LDS stage into registers.  The
    // K x N operand's fragments come back as raw 64-bit halves (tr[j][h]) and are only
    // usable after lds_wait_tied().
    auto load_frags = [&](const uint16_t* As, const uint16_t* Bs, int kk, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN],
                          uint2 (&tr)[FN][2]) {
        const int c = kk * 2 + khalf;                     // logical 16-byte chunk
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(As + a_rd[i] + ((c ^ (arow & 7)) << 3));
        if (MODE == NS_AXPY) {
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = wn0 + j * 32 + tr_n;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = kk * 16 + 4 * h + tr_k;
                    const int g = (n >> 5) ^ (kn_swz(k) % KN_NG);
                    tr[j][h] = lds_read_tr16(Bs + k * TILE + g * 32 + (n & 31));
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + b_rd[j] + ((c ^ (arow & 7)) << 3));
        }
    };
    // Wait for every LDS read of this wave, with the transposed halves as in/out operands
    // so that no MFMA using them can be scheduled before the wait; then assemble them.
    auto lds_wait_tied = [&](uint2 (&tr)[FN][2], bf16x8 (&bfr)[FN]) {
        if (MODE == NS_AXPY) {
            if constexpr (FN == 4) {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(tr[0][0]), "+v"(tr[0][1]), "+v"(tr[1][0]), "+v"(tr[1][1]),
                               "+v"(tr[2][0]), "+v"(tr[2][1]), "+v"(tr[3][0]), "+v"(tr[3][1]));
            } else if constexpr (FN == 2) {
                asm volatile("s_waitcnt lgkmcnt(0)"
                             : "+v"(tr[0][0]), "+v"(tr[0][1]), "+v"(tr[1][0]), "+v"(tr[1][1]));
            } else {
                static_assert(FN == 1, "FN");
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(tr[0][0]), "+v"(tr[0][1]));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const uint4 w = make_uint4(tr[j][0].x, tr[j][0].y, tr[j][1].x, tr[j][1].y);
                bfr[j] = __builtin_bit_cast(bf16x8, w);
            }
        }
    };
    // MFMAs of one sub-step, in two halves (flat index over the FM x FN blocks).
    constexpr int NMF = FM * FN, HALF = (NMF + 1) / 2;
    auto mfmas = [&](const bf16x8 (&af)[FM], const bf16x8 (&bfr)[FN], int lo, int hi) {
#pragma unroll
        for (int f = 0; f < NMF; ++f) {
            if (f < lo || f >= hi) continue;
            const int i = f / FN, j = f % FN;
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    };
    auto stage_a = [&](int s) -> const uint16_t* { return smem[s][0]; };
    auto stage_b = [&](int s) -> const uint16_t* {
        return (MODE != NS_AXPY && diag) ? smem[s][0] : smem[s][1];
    };

    const int nk = p.K / BK;
    issue_loads(0, 0);
    wait_vmem();
    __syncthreads();

    // Two register sets of fragments.  Each sub-step issues its first half of MFMAs, then
    // the LDS reads of the next sub-step, then its second half, so that the reads overlap
    // MFMA execution and at most one sub-step of reads is outstanding when a wait is due.
    // The barrier that publishes the next LDS stage sits inside the last sub-step, so the
    // next stage's first fragments are read while that sub-step's second half executes.
    bf16x8 fa[2][FM], fb[2][FN];
    uint2 ftr[2][FN][2];
    load_frags(stage_a(0), stage_b(0), 0, fa[0], fb[0], ftr[0]);
    lds_wait_tied(ftr[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) issue_loads(kt + 1, s ^ 1);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa[cur], fb[cur], 0, HALF);
            __builtin_amdgcn_sched_barrier(0);
            if (kk + 1 < BK / 16) {
                load_frags(stage_a(s), stage_b(s), kk + 1, fa[nxt], fb[nxt], ftr[nxt]);
            } else if (more) {
                wait_all_mem();
                __syncthreads();
                load_frags(stage_a(s ^ 1), stage_b(s ^ 1), 0, fa[nxt], fb[nxt], ftr[nxt]);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa[cur], fb[cur], HALF, NMF);
            __builtin_amdgcn_sched_barrier(0);
            if (kk + 1 < BK / 16 || more) lds_wait_tied(ftr[nxt], fb[nxt]);
        }
    }

    // ---- epilogue ---------------------------------------------------------------------
    // Lane holds, for each 32 x 32 block (i, j) and q = 0..3, rows 8q + 4*(lane/32) + v
    // (v = 0..3) of column lane%32.
    //
    // NS_POLY and NS_AXPY combine the product with the tile of A (or X) at the same place.
    // That tile is brought into LDS with direct-to-LDS loads (coalesced, 1 KB per
    // instruction) and read back with ds_read_b64_tr_b16, which hands every lane exactly
    // its 4 rows x 1 column in one instruction.
    uint16_t* out = p.out + (int64_t)mat * p.stride_o;
    constexpr int EP_CHUNKS = TILE / 8;                   // 16-byte chunks per tile row
    constexpr int EP_ROWS_PER_INSTR = 512 / TILE;
    constexpr int EP_INSTR = TILE / EP_ROWS_PER_INSTR;
    constexpr int EP_PER_WAVE = EP_INSTR / NW;
    uint16_t* Es = &smem[0][0][0];                        // TILE x TILE bf16 fits in the two stages
    if (MODE == NS_POLY || MODE == NS_AXPY) {
        const uint16_t* Eg = p.ep + (int64_t)mat * p.stride_o + (int64_t)ti * TILE * p.ldo + (int64_t)tj * TILE;
        // every wave must be done reading the K stages before they are overwritten
        wait_all_mem();
        __syncthreads();
#pragma unroll 4
        for (int i = 0; i < EP_PER_WAVE; ++i) {
            const int q = wave + NW * i;
            const int r = q * EP_ROWS_PER_INSTR + lane / EP_CHUNKS;
            const int pc = lane % EP_CHUNKS;
            const int g = (pc >> 2) ^ (ep_swz(r) % KN_NG);
            load_to_lds(Eg + (int64_t)r * p.ldo + (g * 4 + (pc & 3)) * 8, Es + q * 512);
        }
        wait_vmem();
        __syncthreads();
    }
    const int col_in = lane & 31, rsub = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gc = tj * TILE + wn0 + j * 32 + col_in;
            uint2 e[4];
            if (MODE == NS_POLY || MODE == NS_AXPY) {
                const int c = wn0 + j * 32 + tr_n;        // supplying-lane column block
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wm0 + i * 32 + q * 8 + 4 * (tg >> 1) + (tix >> 2);
                    const int g = (c >> 5) ^ (ep_swz(r) % KN_NG);
                    e[q] = lds_read_tr16(Es + r * TILE + g * 32 + (c & 31));
                }
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gr0 = ti * TILE + wm0 + i * 32 + q * 8 + rsub;
                uint16_t h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float val = acc[i][j][q * 4 + v];
                    if (MODE == NS_POLY || MODE == NS_AXPY) {
                        const uint32_t w = (v < 2) ? e[q].x : e[q].y;
                        const uint32_t hv = (v & 1) ? (w >> 16) : (w & 0xffffu);
                        val = p.alpha * dev::bf16_to_f32(hv) + p.gamma * val;
                    }
                    h[v] = dev::f32_to_bf16(val);
                    out[(int64_t)(gr0 + v) * p.ldo + gc] = h[v];
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
        case TILE_256: return launch_cfg<MODE, 256, 2, 2>(a, s);
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
