// Batched Newton–Schulz products on gfx950 matrix cores (bf16 MFMA, float32 accumulate).
//
// One quintic Newton–Schulz step on a canonical m x n matrix X (m <= n) is
//     A = X X^T,   B = b A + c A A,   X' = a X + B X.
// The pages run this on whole momentum matrices with an operator that exploits the
// symmetry of the intermediates ("Frontier Pre-training at Microsoft AI", method details
// section 5, resharding step 3; the recipe page, section "How to Make Parameter Updates
// Faster and More Stable?").  Here:
//   * NS_SYRK  A = X X^T: only tiles (i, j) with i <= j are computed; each off-diagonal
//              tile is stored twice (as itself and mirrored), so A is exactly symmetric.
//   * NS_POLY  B = b A + c A A^T: A is symmetric, so A A = A A^T and the same
//              upper-triangle scheme applies; b A is added in the epilogue.
//   * NS_AXPY  X' = a X + B X: a full GEMM with the axpy fused into its epilogue.
//
// Two kernels share the tile order, the fragment layouts and the epilogue:
//   * ns_vs_kernel (256 x 256 tiles, the large buckets): 8 waves of 128 x 64, two waves
//     per SIMD.  Operand tiles go global -> VGPR (buffer loads) -> LDS, one K step ahead
//     of the LDS stage being multiplied; on gfx950 this path keeps more requests in
//     flight than the direct-to-LDS loads when operands miss in L2 (measured 20-30 % more
//     bytes per CU from the Infinity Cache).  The result tile is staged in LDS and leaves
//     in 16-byte stores.
//   * ns_gemm_kernel (128 and 64 tiles, the small buckets): operand tiles go from global
//     memory straight into LDS with global_load_lds_dwordx4 (no VGPR staging): each
//     lane's 16 bytes land at the instruction's LDS base + 16 * lane, and the lane picks
//     which global 16 bytes to fetch, so the LDS image can be XOR-swizzled.  Loads run
//     STAGES - 1 K steps ahead of the v_mfma_f32_32x32x16_bf16 that consume them.
// Common to both:
//   * Row-panel operands (K contiguous: X in SYRK, A in POLY, B in AXPY) are stored so
//     that the 16 lanes the LDS serves together (64 banks, one ds_read_b128 each) never
//     share a bank.  An MFMA operand is one ds_read_b128 per lane.
//   * The K x N operand of NS_AXPY (X, N contiguous) is stored as rows of TILE bf16 in its
//     own orientation, with 64-byte granules permuted per row, and read with
//     ds_read_b64_tr_b16, which transposes 4 x 4 blocks of 16-bit values across each group
//     of 16 lanes into exactly the K-packed layout the MFMA wants.
//   * Each MFMA is followed by at most a few LDS reads, LDS writes or loads (the issue
//     order is pinned with scheduling barriers), so those issue while the matrix pipe is
//     busy.
//
// Matrices are padded to multiples of TILE with zero rows and columns, so no kernel
// needs a bounds check: zero padding stays zero through all three products.
//
// Workgroups are remapped so that the tiles of one matrix run on the same XCD (the
// hardware hands consecutive workgroup ids to the 8 XCDs in turn), keeping a matrix's
// panels in that XCD's L2, and tiles are ordered in groups that share operand panels.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace muon {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int NUM_XCD = 8;

__device__ __forceinline__ int xcd_remap(int b, int g) {
    const int xcd = b % NUM_XCD, local = b / NUM_XCD;
    const int q = g / NUM_XCD, r = g % NUM_XCD;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Persistent launches (one workgroup per CU, NUM_XCD | gridDim.x): workgroup w runs on XCD
// w % NUM_XCD (the hardware deals consecutive workgroup ids to the XCDs in turn).  The tile
// order is cut into the contiguous XCD shares of xcd_remap, and each XCD's workgroups take
// the tiles of its share one by one from a counter (so that the tiles one XCD runs at the
// same time are neighbours in that order, as in the one-tile-per-workgroup launch, and a
// slower CU simply takes fewer tiles); a workgroup whose share is used up takes tiles
// from the other XCDs' shares.  Only atomic increments, no waiting: every workgroup stops
// once all eight counters are past their shares.  -1 when done.
__device__ __forceinline__ int grab_tile(uint32_t* sched, int xcd, int total) {
    const int q = total / NUM_XCD, r = total % NUM_XCD;
    for (int k = 0; k < NUM_XCD; ++k) {
        const int x = (xcd + k) % NUM_XCD;
        const int start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
        const int size = q + (x < r ? 1 : 0);
        const uint32_t loc = atomicAdd(&sched[x], 1u);
        if ((int)loc < size) return start + (int)loc;
    }
    return -1;
}

// Tile order.  The 32 tiles an XCD runs at once should share as few operand panels as
// possible (each panel K-slice is then fetched into that XCD's L2 once and reused).
constexpr int GROUP = 8;

// Full tm x tn grid (NS_AXPY): bands of GROUP tile rows, each band walked column by
// column, so concurrent tiles form a GROUP-tall block (GROUP + 32/GROUP panels).
__device__ __forceinline__ void grid_decode(int t, int tm, int tn, int& ti, int& tj) {
    const int band = t / (GROUP * tn);
    const int r0 = band * GROUP;
    const int gm = min(GROUP, tm - r0);
    const int w = t - band * GROUP * tn;
    tj = w / gm;
    ti = r0 + (w - tj * gm);
}

// Upper triangle of a T x T tile grid (NS_SYRK, NS_POLY): GROUP x GROUP super-blocks
// (I <= J) in row-major order; inside a block, its tiles with i <= j row by row.
__device__ __forceinline__ void tri_decode(int t, int T, int& ti, int& tj) {
    const int NB = (T + GROUP - 1) / GROUP;
    for (int I = 0; I < NB; ++I) {
        const int rows = min(GROUP, T - I * GROUP);
        for (int J = I; J < NB; ++J) {
            const int cols = min(GROUP, T - J * GROUP);
            const int cnt = (I == J) ? rows * (rows + 1) / 2 : rows * cols;
            if (t < cnt) {
                if (I == J) {
                    int i = 0;
                    while (t >= rows - i) { t -= rows - i; ++i; }
                    ti = I * GROUP + i;
                    tj = I * GROUP + i + t;
                } else {
                    ti = I * GROUP + t / cols;
                    tj = J * GROUP + t % cols;
                }
                return;
            }
            t -= cnt;
        }
    }
    ti = tj = 0;   // not reached for t < T(T+1)/2
}

// s_waitcnt with vmcnt(N) (gfx9 encoding: low 4 bits, high 2 bits at 15:14), expcnt
// left open and lgkmcnt(0) or left open.
template <int N, bool LGKM0>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int imm = (N & 15) | (((N >> 4) & 3) << 14) | (7 << 4) | (LGKM0 ? 0 : (15 << 8));
    __builtin_amdgcn_s_waitcnt(imm);
}

// 16 bytes from global memory into LDS at base + 16 * lane (base wave-uniform), issued
// as inline assembly so that the compiler does not track it: through the compiler
// intrinsic, every later LDS read would first wait for all outstanding direct-to-LDS
// loads (the compiler cannot tell that they target other stages), exposing the
// global-load latency at every read.  Completion is therefore waited for explicitly
// (wait_vm) before the barrier that publishes a stage.  The LDS base goes through M0,
// which the statement declares clobbered, so the compiler keeps nothing of its own there.
__device__ __forceinline__ void load_to_lds(const uint16_t* src, const uint16_t* lds_base) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)lds_base);
    // one wait state between writing M0 and the LDS-DMA instruction that reads it
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(base) : "memory", "m0");
}

// ds_read_b64_tr_b16: 4 x 4 blocks of 16-bit values transposed across each group of 16
// lanes (lane 4a+b receives element b of the 8-byte rows addressed by lanes a, a+4,
// a+8, a+12).
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(const __attribute__((address_space(3))) uint16_t*)p);
    return __builtin_bit_cast(bf16x4, v);
}

// Granule swizzle of the K x N operand: the 8 rows one transposing read touches
// (k0..k0+3 and k0+8..k0+11) get 8 different 64-byte granules.
__device__ __forceinline__ int kn_swz(int k) { return (k & 3) | ((k >> 1) & 4); }

// Granule swizzle of the epilogue input tile: a transposing read there touches 8
// consecutive rows, which get 8 different granules.
__device__ __forceinline__ int ep_swz(int r) { return r & 7; }

// One TILE x TILE output tile (index b of the launch's tile order) of the products on the
// smaller tiles, with the LDS stages at `smem`; run by all 64 * WM * WN threads.
template <int MODE, int TILE, int WM, int WN, int BK, int STAGES>
__device__ __forceinline__ void gemm_tile(const NsArgs& p, const int b, uint16_t (*smem)[2][TILE * BK]) {
    constexpr int NW = WM * WN;
    constexpr int WTM = TILE / WM, WTN = TILE / WN;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;       // 32 x 32 MFMA blocks per wave
    constexpr int PANEL = TILE * BK;                  // elements of one operand tile
    // row panels: rows of BK bf16
    constexpr int CPR = BK / 8;                       // 16-byte chunks per row
    constexpr int RPI = 512 / BK;                     // rows per 1 KB load instruction
    constexpr int RP_INSTR = TILE / RPI;
    constexpr int RP_PER_WAVE = RP_INSTR / NW;
    constexpr int ROWS_PER_BANKLINE = 256 / (2 * BK); // rows sharing one 64-bank line
    // K x N panel: rows of TILE bf16
    constexpr int KN_ROWS_PER_INSTR = 512 / TILE;
    constexpr int KN_INSTR = BK / KN_ROWS_PER_INSTR;
    constexpr int KN_PER_WAVE = KN_INSTR / NW;
    constexpr int KN_CHUNKS = TILE / 8;
    constexpr int KN_NG = TILE / 32;                  // 64-byte granules per K x N row
    constexpr int KSUB = BK / 16;                     // MFMA K sub-steps per K step
    static_assert(FM >= 1 && FN >= 1, "tile configuration");
    static_assert(RP_PER_WAVE >= 1 && RP_INSTR % NW == 0, "row-panel load split");
    static_assert(MODE != NS_AXPY || (KN_PER_WAVE >= 1 && KN_INSTR % NW == 0), "K x N load split");
    static_assert(STAGES >= 2 && KSUB >= 1, "pipeline");
    static_assert(TILE * TILE <= STAGES * 2 * PANEL, "epilogue tile fits in the stages");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    const int mat = b / p.tiles_per_mat;
    const int t = b - mat * p.tiles_per_mat;
    int ti, tj;
    if (MODE == NS_AXPY) {
        grid_decode(t, p.tiles_m, p.tiles_n, ti, tj);
    } else {
        tri_decode(t, p.tiles_m, ti, tj);
    }
    const bool diag = MODE != NS_AXPY && ti == tj;    // one panel serves both operands

    const uint16_t* Ag = p.opa + (int64_t)mat * p.stride_a + (int64_t)ti * TILE * p.lda;
    const uint16_t* Bg = (MODE == NS_AXPY)
                             ? p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE
                             : p.opb + (int64_t)mat * p.stride_b + (int64_t)tj * TILE * p.ldb;

    // Chunk permutation of a row-panel row: 16 consecutive rows at one logical chunk
    // land in 16 different 16-byte bank groups.
    auto rp_swz = [](int row) { return (row / ROWS_PER_BANKLINE) % CPR; };

    // ---- per-lane source offsets of the direct-to-LDS loads (fixed across K steps) ----
    int64_t ra_off[RP_PER_WAVE], rb_off[RP_PER_WAVE];
#pragma unroll
    for (int i = 0; i < RP_PER_WAVE; ++i) {
        const int q = wave + NW * i;
        const int row = RPI * q + lane / CPR;
        const int chunk = (lane % CPR) ^ rp_swz(row);
        ra_off[i] = (int64_t)row * p.lda + chunk * 8;
        rb_off[i] = (int64_t)row * p.ldb + chunk * 8;
    }
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

    // One direct-to-LDS load instruction (index d of this wave's NDMA per K step) of K
    // step kt into stage st.
    constexpr int NDMA = RP_PER_WAVE + ((MODE == NS_AXPY) ? KN_PER_WAVE : RP_PER_WAVE);
    auto dma = [&](int d, int kt, int st) {
        const int k0 = kt * BK;
        if (d < RP_PER_WAVE) {
            load_to_lds(Ag + ra_off[d] + k0, smem[st][0] + (wave + NW * d) * 512);
        } else {
            const int e = d - RP_PER_WAVE;
            if (MODE == NS_AXPY)
                load_to_lds(Bg + kn_off[e] + (int64_t)k0 * p.ldb, smem[st][1] + (wave + NW * e) * 512);
            else if (!diag)
                load_to_lds(Bg + rb_off[e] + k0, smem[st][1] + (wave + NW * e) * 512);
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

    // One LDS fragment read (index r of NRD per sub-step) of sub-step kk from stage st:
    // r < FM are the row-panel fragments af[r]; the rest are the right operand's, either
    // row-panel fragments bfr[j] or, in NS_AXPY, transposed halves tr[j][h].
    constexpr int NRD = FM + ((MODE == NS_AXPY) ? 2 * FN : FN);
    auto rd = [&](int r, int st, int kk, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN], bf16x4 (&tr)[FN][2]) {
        const int c = kk * 2 + khalf;                     // logical 16-byte chunk
        const uint16_t* As = smem[st][0];
        const uint16_t* Bs = (MODE != NS_AXPY && diag) ? smem[st][0] : smem[st][1];
        if (r < FM) {
            af[r] = *reinterpret_cast<const bf16x8*>(As + a_rd[r] + ((c ^ rp_swz(arow)) << 3));
        } else if (MODE == NS_AXPY) {
            const int j = (r - FM) >> 1, h = (r - FM) & 1;
            const int n = wn0 + j * 32 + tr_n;
            const int k = kk * 16 + 4 * h + tr_k;
            const int g = (n >> 5) ^ (kn_swz(k) % KN_NG);
            tr[j][h] = lds_read_tr16(Bs + k * TILE + g * 32 + (n & 31));
        } else {
            const int j = r - FM;
            bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + b_rd[j] + ((c ^ rp_swz(arow)) << 3));
        }
    };
    // Assemble the right operand of NS_AXPY from its two transposed halves.
    auto join_tr = [&](bf16x4 (&tr)[FN][2], bf16x8 (&bfr)[FN]) {
        if (MODE == NS_AXPY) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = __builtin_shufflevector(tr[j][0], tr[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    // Issue schedule of one sub-step (the order is pinned with scheduling barriers): NMF
    // MFMAs, each followed by at most RPS fragment reads of the next sub-step and, in the
    // first sub-step of a K step, DPS direct-to-LDS loads for STAGES - 1 K steps ahead.
    // In the last sub-step of a K step, the wait for the next stage's loads and the
    // barrier that publishes it come first; the next stage's reads then fill the last NRS
    // MFMA slots.
    constexpr int NMF = FM * FN;
    constexpr int RPS = (NRD + NMF - 1) / NMF;
    constexpr int NRS = (NRD + RPS - 1) / RPS;
    constexpr int DPS = (NDMA + NMF - 1) / NMF;
    constexpr int AHEAD = STAGES - 1;                     // K steps of loads in flight
    static_assert(NRS <= NMF, "read slots");

    const int nk = p.K / BK;
    // prologue: fill the first STAGES - 1 stages, wait for stage 0
#pragma unroll
    for (int s0 = 0; s0 < AHEAD; ++s0) {
        if (s0 < nk) {
#pragma unroll
            for (int d = 0; d < NDMA; ++d) dma(d, s0, s0);
        }
    }
    // Diagonal tiles of the symmetric products load one panel, so their batches are
    // RP_PER_WAVE instructions long instead of NDMA.
    auto wait_next_stage = [&](bool younger_in_flight) {
        if (!younger_in_flight) wait_vm<0, true>();
        else if (diag) wait_vm<RP_PER_WAVE * (AHEAD - 1), true>();
        else wait_vm<NDMA * (AHEAD - 1), true>();
    };
    wait_next_stage(nk >= AHEAD);
    __syncthreads();

    bf16x8 fa[2][FM], fb[2][FN];
    bf16x4 ftr[2][FN][2];
#pragma unroll
    for (int r = 0; r < NRD; ++r) rd(r, 0, 0, fa[0], fb[0], ftr[0]);
    join_tr(ftr[0], fb[0]);

    int st = 0;                                           // stage of K step kt
    for (int kt = 0; kt < nk; ++kt) {
        const bool issue = kt + AHEAD < nk;               // loads for K step kt + AHEAD
        const bool more = kt + 1 < nk;
        const int st_next = (st + 1 == STAGES) ? 0 : st + 1;
        const int st_load = (st == 0) ? STAGES - 1 : st - 1;  // (kt + AHEAD) % STAGES
#pragma unroll
        for (int kk = 0; kk < KSUB; ++kk) {
            const int cur = kk & 1, nxt = cur ^ 1;
            const bool last = kk + 1 == KSUB;
            const int rd_lo = last ? NMF - NRS : 0;        // first MFMA slot followed by reads
#pragma unroll
            for (int f = 0; f < NMF; ++f) {
                const int i = f / FN, j = f % FN;
                __builtin_amdgcn_sched_barrier(0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (kk == 0 && issue) {
#pragma unroll
                    for (int q = 0; q < DPS; ++q) {
                        const int d = f * DPS + q;
                        if (d < NDMA) dma(d, kt + AHEAD, st_load);
                    }
                }
                if (last && f == rd_lo && more) {
                    // the next stage's loads were issued AHEAD - 1 K steps ago; let the
                    // younger batches stay in flight
                    wait_next_stage(issue);
                    __syncthreads();
                }
                if (f >= rd_lo && f < rd_lo + NRS && (!last || more)) {
#pragma unroll
                    for (int q = 0; q < RPS; ++q) {
                        const int r = (f - rd_lo) * RPS + q;
                        if (r < NRD) rd(r, last ? st_next : st, last ? 0 : kk + 1, fa[nxt], fb[nxt], ftr[nxt]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (!last || more) join_tr(ftr[nxt], fb[nxt]);
        }
        st = st_next;
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
    uint16_t* Es = &smem[0][0][0];                        // TILE x TILE bf16 fits in the stages
    if (MODE == NS_POLY || MODE == NS_AXPY) {
        const uint16_t* Eg = p.ep + (int64_t)mat * p.stride_o + (int64_t)ti * TILE * p.ldo + (int64_t)tj * TILE;
        // every wave must be done reading the K stages before they are overwritten
        wait_vm<0, true>();
        __syncthreads();
#pragma unroll 4
        for (int i = 0; i < EP_PER_WAVE; ++i) {
            const int q = wave + NW * i;
            const int r = q * EP_ROWS_PER_INSTR + lane / EP_CHUNKS;
            const int pc = lane % EP_CHUNKS;
            const int g = (pc >> 2) ^ (ep_swz(r) % KN_NG);
            load_to_lds(Eg + (int64_t)r * p.ldo + (g * 4 + (pc & 3)) * 8, Es + q * 512);
        }
        wait_vm<0, true>();
        __syncthreads();
    }
    const int col_in = lane & 31, rsub = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int gc = tj * TILE + wn0 + j * 32 + col_in;
            bf16x4 e[4];
            if (MODE == NS_POLY || MODE == NS_AXPY) {
                const int c = wn0 + j * 32 + tr_n;        // supplying-lane column block
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = wm0 + i * 32 + q * 8 + 4 * (tg >> 1) + (tix >> 2);
                    const int g = (c >> 5) ^ (ep_swz(r) % KN_NG);
                    e[q] = lds_read_tr16(Es + r * TILE + g * 32 + (c & 31));
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int gr0 = ti * TILE + wm0 + i * 32 + q * 8 + rsub;
                uint16_t h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float val = acc[i][j][q * 4 + v];
                    if (MODE == NS_POLY || MODE == NS_AXPY)
                        val = dev::ns_combine(p.alpha, (float)e[q][v], p.gamma, val);
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

// One chunk: one tile per workgroup, tiles of a matrix kept on one XCD.
template <int MODE, int TILE, int WM, int WN, int BK, int STAGES>
__global__ __launch_bounds__(64 * WM * WN) void ns_gemm_kernel(NsArgs p) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[STAGES][2][TILE * BK];
    gemm_tile<MODE, TILE, WM, WN, BK, STAGES>(p, xcd_remap(blockIdx.x, gridDim.x), smem);
}

// Every small tiled chunk of a plan in one launch per product: one tile queue over the
// jobs' tiles (job j's tiles are queue entries first_j ..), 128- and 64-row tiles alike.
// Each workgroup takes queue entries blockIdx.x, blockIdx.x + gridDim.x, ..., and runs a
// tile exactly as the one-chunk launch does (same code, same K order), so a matrix's result
// does not depend on which launch computed it.
constexpr int G_BK = 64, G_STAGES = 2;

template <int MODE>
__global__ __launch_bounds__(256) void ns_grouped_kernel(GroupedNsArgs g) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[G_STAGES * 2 * 128 * G_BK];
    for (int t = blockIdx.x; t < g.total_tiles; t += gridDim.x) {
        int j = 0;
        while (j + 1 < g.n_jobs && t >= g.job[j + 1].first) ++j;
        const int b = t - g.job[j].first;
        if (g.job[j].tile == TILE_128)
            gemm_tile<MODE, 128, 2, 2, G_BK, G_STAGES>(g.job[j].a, b, reinterpret_cast<uint16_t (*)[2][128 * G_BK]>(smem));
        else
            gemm_tile<MODE, 64, 2, 2, G_BK, G_STAGES>(g.job[j].a, b, reinterpret_cast<uint16_t (*)[2][64 * G_BK]>(smem));
        __syncthreads();                                  // the tile's LDS reads are done
    }
}

// ---- 256 x 256 tiles, operands staged through VGPRs -------------------------------------
//
// LDS layout (bytes).  Row panels (K contiguous in memory) are stored as 4 K-planes of 16
// elements: row r, K chunk c (16 bytes, c = 0..7) lands at plane c/2, offset r*32 plus
// 16 * ((c & 1) ^ ((r >> 3) & 1)); planes are 8192 + 32 bytes apart.  Every fragment read
// and every staging write is then one per-lane base register plus a compile-time offset
// (plane, fragment, stage).  Bank rules measured on gfx950 (SQ_LDS_BANK_CONFLICT): a
// 128-bit read is served 16 lanes at a time across all 64 banks, a 128-bit write 8 lanes
// at a time across 128 bytes of banks.  A fragment read (16 rows of one plane) covers 16
// distinct 16-byte slots of the 256-byte bank line; a staging write (8 lanes: one row,
// its 8 chunks in 4 planes) covers 8 distinct slots modulo 128 bytes thanks to the 32-byte
// plane rotation.  The K x N panel of the axpy keeps the 512-byte rows with permuted
// 64-byte granules of ns_gemm_kernel, whose writes (8 lanes: two 64-byte granules of
// different parity) are conflict-free under the same rules.
typedef int i32x4 __attribute__((ext_vector_type(4)));

// 8 waves (2 x 4) of 128 x 64: two waves per SIMD, 128 accumulators and 16 staging
// registers each.  Measured on gfx950 against 4 waves of 128 x 128 (one wave per SIMD):
// 4-12 % faster, since a wave waiting on LDS or a barrier leaves the matrix pipe to the
// other wave of its SIMD.
constexpr int VS_WM = 2, VS_WN = 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, int64_t elems) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(elems * 2), 0x00020000);
}

__device__ __forceinline__ void lds_wait_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
using ic = std::integral_constant<int, N>;

// Diagonal tiles of the symmetric products (SYRK, POLY) need only their 32 x 32 blocks on
// or above the diagonal: 36 of 64.  The 8 waves take the tile's eight 128 x 64 regions
// (row half r, column quarter c: region 4r + c) in an order that gives the two waves of
// each SIMD (waves w and w + 4) 8 to 10 needed blocks between them instead of up to 16:
//   wave      0      1      2      3      4      5      6      7
//   region  (0,2)  (0,3)  (0,1)  (1,3)  (1,0)  (1,1)  (1,2)  (0,0)
//   pattern FULL   FULL   B      B      NONE   NONE   A      A
// FULL: all 8 blocks; A: blocks (i, j) with i <= j (3); B: all but (3, 0) (7); NONE: none
// (the wave only stages operands).  The blocks below the diagonal are stored as the
// mirror of those above it.
constexpr uint32_t DIAG_REGION = 0x06547132u;     // nibble w: region of wave w
constexpr uint32_t DIAG_REGION_WAVE = 0x36541027u;  // nibble r: the wave whose region r is
static_assert([] {
    for (int w = 0; w < 8; ++w)
        if (((DIAG_REGION_WAVE >> (4 * ((DIAG_REGION >> (4 * w)) & 15u))) & 15u) != (uint32_t)w) return false;
    return true;
}(), "DIAG_REGION_WAVE inverts DIAG_REGION");
constexpr int PAT_FULL = 0, PAT_A = 1, PAT_B = 2, PAT_NONE = 3;
constexpr uint32_t DIAG_PATTERN = 0x11332200u;    // nibble w: pattern of wave w

__device__ __forceinline__ constexpr bool need_block(int pat, int i, int j) {
    return pat == PAT_FULL || (pat == PAT_A && i <= j) || (pat == PAT_B && !(i == 3 && j == 0));
}
// fragment read r of a sub-step (r < 4: rows 32r of the region; then the columns)
__device__ __forceinline__ constexpr bool need_frag(int pat, int r) {
    return pat == PAT_FULL || pat == PAT_B || (pat == PAT_A && (r < 2 || r >= 4));
}

// NORM (SYRK and AXPY of the first iteration): the X operand is read as X0 and normalised
// in the staging registers on its way to LDS (and the AXPY's E tile as it is combined), with
// the separate normalize pass's arithmetic, so no normalised copy of X is ever written.
template <int MODE, int WM, int WN, bool PERSIST, bool NORM>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WM * WN / 4, WM * WN / 4)))
void ns_vs_kernel(NsArgs p) {
    static_assert(!NORM || MODE != NS_POLY, "only SYRK and AXPY read X");
    constexpr int TILE = 256, BK = 64, NW = WM * WN, NT = 64 * NW;
    constexpr int WTM = TILE / WM, WTN = TILE / WN, FM = WTM / 32, FN = WTN / 32;
    constexpr int RP_ROWS = NT / 8;                   // row-panel rows per staging pass
    constexpr int KN_ROWS = NT / 32;                  // K x N rows per staging pass
    static_assert(RP_ROWS % 16 == 0, "staging rows keep the chunk swizzle");
    constexpr int KSUB = BK / 16;
    constexpr int NCH = TILE * BK / 8 / NT;           // 16-byte chunks per thread and operand
    constexpr int KN_NG = TILE / 32;
    constexpr int PLANE_B = 8192 + 32;
    constexpr int RP_B = 4 * PLANE_B;                 // one row panel (256 x 64 bf16)
    constexpr int KN_B = 64 * TILE * 2;               // one K x N panel (64 x 256 bf16)
    constexpr int OFF_B = 2 * RP_B;                   // second operand's stages
    constexpr int B_STAGE = (MODE == NS_AXPY) ? KN_B : RP_B;
    constexpr int SMEM = OFF_B + 2 * B_STAGE;
    static_assert(SMEM >= TILE * TILE * 2, "epilogue tile fits");
    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  // one tile per workgroup, or (PERSIST) the workgroup's tiles one after another; in the
  // persistent case the next tile's first K step is fetched into the staging registers
  // before the current tile's epilogue (see below)
  i32x4 sa[NCH], sb[NCH];
  __shared__ int next_slot;                             // the next tile, from thread 0's grab
  int b_next = -1;
  if (PERSIST) {
      if (threadIdx.x == 0) next_slot = grab_tile(p.sched, blockIdx.x % NUM_XCD, p.total_tiles);
      __syncthreads();
      b_next = next_slot;
  }
  for (int it = 0;; ++it) {
    int b;
    if (PERSIST) {
        b = b_next;
        if (b < 0) break;
        if (it > 0) __syncthreads();                      // the last tile's LDS reads are done
    } else {
        if (it > 0) break;
        b = xcd_remap(blockIdx.x, gridDim.x);
    }
    // The thread index is made opaque to the compiler in every iteration, so that the
    // offsets derived from it are recomputed per tile instead of being hoisted out of the
    // loop and kept live through the epilogue (which then runs out of registers); the
    // per-wave epilogue needs the same in the one-tile kernel.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    // p.reverse: the chunk's matrices in the opposite order, each one's tiles in the same
    const int mat0 = b / p.tiles_per_mat;
    const int t = b - mat0 * p.tiles_per_mat;
    const int mat = p.reverse ? p.total_tiles / p.tiles_per_mat - 1 - mat0 : mat0;
    int ti, tj;
    if (MODE == NS_AXPY) grid_decode(t, p.tiles_m, p.tiles_n, ti, tj);
    else tri_decode(t, p.tiles_m, ti, tj);
    const bool diag = MODE != NS_AXPY && ti == tj;
    // The wave's 128 x 64 region of the tile: on a diagonal tile of the symmetric products
    // from DIAG_REGION (and only its blocks on or above the diagonal are computed, see
    // DIAG_PATTERN), elsewhere by wave index.
    const int region = diag ? (int)((DIAG_REGION >> (4 * wave)) & 15u) : wave;
    const int wm0 = (region / WN) * WTM, wn0 = (region % WN) * WTN;
    // the matrix's normaliser (NORM), rounded to float32 as the normalize pass rounds it
    const float s_norm = NORM ? (float)p.inv[mat] : 1.f;

    // buffer resources from the first element of each operand panel to the end of its matrix
    const int64_t a0 = (int64_t)ti * TILE * p.lda;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.opa + (int64_t)mat * p.stride_a + a0, p.stride_a - a0);
    const int64_t b0 = (MODE == NS_AXPY) ? (int64_t)tj * TILE : (int64_t)tj * TILE * p.ldb;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.opb + (int64_t)mat * p.stride_b + b0, p.stride_b - b0);

    // staging: row panels -> rows row0 + RP_ROWS i, chunk ch; K x N -> rows klo + KN_ROWS i,
    // chunk nc.  The row swizzle bit (row >> 3) & 1 does not depend on i; the K x N granule
    // swizzle depends at most on the parity of i.
    const int row0 = tid >> 3, ch = tid & 7;
    const int va = row0 * p.lda * 2 + ch * 16;
    const int vb_rp = row0 * p.ldb * 2 + ch * 16;
    const int klo = tid >> 5, nc = tid & 31;
    const int vb_kn = klo * p.ldb * 2 + nc * 16;
    const int w_rp = (ch >> 1) * PLANE_B + row0 * 32 + (((ch & 1) ^ ((row0 >> 3) & 1)) << 4);
    int w_kn[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int swz = kn_swz(klo + KN_ROWS * par);
        w_kn[par] = OFF_B + klo * TILE * 2 + (((((nc >> 2) ^ (swz % KN_NG)) << 2) | (nc & 3)) << 4);
    }

    // K step 0 already in sa / sb (the axpy only: in the symmetric products the extra live
    // registers would cost the side-stream kernels their room on the CU)
    constexpr bool PF = PERSIST && MODE == NS_AXPY;
    const bool prefetched = PF && it > 0;
    auto gload_a = [&](int i, int kt) {
        sa[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, va, kt * BK * 2 + i * RP_ROWS * p.lda * 2, 0);
    };
    auto gload_b = [&](int i, int kt) {
        if (MODE == NS_AXPY)
            sb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, vb_kn, (kt * BK + KN_ROWS * i) * p.ldb * 2, 0);
        else
            sb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, vb_rp, kt * BK * 2 + i * RP_ROWS * p.ldb * 2, 0);
    };
    // NORM: a staged 16-byte piece of X0 becomes bf16(X0 * s).  The padding outside the
    // m x n region needs no mask: the finalize kernel has zeroed it in X0.  The scheduling
    // barriers keep the compiler from spreading the arithmetic over the neighbouring slots
    // (which costs registers the side-stream kernels need).
    auto norm16 = [&](i32x4 v) {
        __builtin_amdgcn_sched_barrier(0);
        const uint4 u = dev::normalize8(__builtin_bit_cast(uint4, v), 8, s_norm);
        __builtin_amdgcn_sched_barrier(0);
        return __builtin_bit_cast(i32x4, u);
    };
    auto swrite_a = [&](int i, int st) {
        i32x4 v = sa[i];
        if (NORM && MODE == NS_SYRK) v = norm16(v);
        *reinterpret_cast<i32x4*>(smem + w_rp + st * RP_B + i * RP_ROWS * 32) = v;
    };
    auto swrite_b = [&](int i, int st) {
        i32x4 v = sb[i];
        if (NORM) v = norm16(v);
        if (MODE == NS_AXPY)
            *reinterpret_cast<i32x4*>(smem + w_kn[i & 1] + st * KN_B + i * KN_ROWS * TILE * 2) = v;
        else
            *reinterpret_cast<i32x4*>(smem + OFF_B + w_rp + st * RP_B + i * RP_ROWS * 32) = v;
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // fragment read bases
    const int arow = lane & 31, khalf = lane >> 5;
    const int rp_lane = arow * 32 + ((khalf ^ ((arow >> 3) & 1)) << 4);
    const int r_a = wm0 * 32 + rp_lane;                               // + st*RP_B + kk*PLANE_B + i*1024
    const int r_b = (diag ? 0 : OFF_B) + wn0 * 32 + rp_lane;          // + st*RP_B + kk*PLANE_B + j*1024
    const int tg = lane >> 4, tix = lane & 15;
    const int tr_k = 8 * (tg >> 1) + (tix >> 2);
    const int tr_n = 16 * (tg & 1) + 4 * (tix & 3);
    int r_tr[FN];                                                     // + st*KN_B + kk*8192 + h*2048
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int g = ((wn0 >> 5) + j) ^ (kn_swz(tr_k) % KN_NG);
        r_tr[j] = OFF_B + tr_k * TILE * 2 + g * 64 + tr_n * 2;
    }

    constexpr int NRD = FM + ((MODE == NS_AXPY) ? 2 * FN : FN);
    auto rd = [&](int r, int st, int kk, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN], bf16x4 (&tr)[FN][2]) {
        if (r < FM) {
            af[r] = *reinterpret_cast<const bf16x8*>(smem + r_a + st * RP_B + kk * PLANE_B + r * 1024);
        } else if (MODE == NS_AXPY) {
            const int j = (r - FM) >> 1, h = (r - FM) & 1;
            tr[j][h] = lds_read_tr16(reinterpret_cast<const uint16_t*>(smem + r_tr[j] + st * KN_B + kk * 8192 + h * 2048));
        } else {
            const int j = r - FM;
            bfr[j] = *reinterpret_cast<const bf16x8*>(smem + r_b + st * RP_B + kk * PLANE_B + j * 1024);
        }
    };
    auto join_tr = [&](bf16x4 (&tr)[FN][2], bf16x8 (&bfr)[FN]) {
        if (MODE == NS_AXPY) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = __builtin_shufflevector(tr[j][0], tr[j][1], 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    constexpr int NMF = FM * FN;                          // MFMAs per sub-step
    static_assert(NRD <= NMF && NCH <= NMF, "issue slots");
    const int nk = p.K / BK;                              // a multiple of 4

    // The epilogue of the axpy and poly tiles works per wave on its own 128 x 64 region, in two halves of 64 rows, each through an
    // 8 KB slot of LDS: half 0 in stage 0 (free once every wave has passed the barrier of
    // the second-to-last K step, so its E rows are fetched during the last K step), half 1
    // in stage 1.  Waves 0-3 use the row-panel stages, waves 4-7 the second operand's.
    // Slot row r (128 bytes) holds 16-byte granule g of the region's row at position
    // g ^ ((r >> 1) & 7): the 8-byte accesses of the combine (32 rows x 8 bytes per
    // half-wave) then touch each bank pair at most twice per 512 bytes.
    constexpr bool HAS_E = MODE != NS_SYRK;
    static_assert(WM == 2 && WN == 4 && 4 * 8192 <= RP_B && 4 * 8192 <= B_STAGE, "epilogue slots");
    auto slot = [&](int h) {
        const int base = (wave < 4) ? (h ? RP_B : 0) : (h ? OFF_B + B_STAGE : OFF_B);
        return base + (wave & 3) * 8192;
    };
    // E rows 64h .. 64h + 63 of the wave's region into its slot h (8 direct-to-LDS loads)
    auto e_issue = [&](int h) {
        const uint16_t* Eg = p.ep + (int64_t)mat * p.stride_o + (int64_t)(ti * TILE + wm0 + 64 * h) * p.ldo +
                             (int64_t)(tj * TILE + wn0);
        const char* sl = smem + slot(h);
        // computed here, not hoisted into the main loop's register peak
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < 8; ++k) {                     // 8 rows (1 KB) per instruction
            const int r = 8 * k + (ln >> 3), pos = ln & 7;
            load_to_lds(Eg + (int64_t)r * p.ldo + (pos ^ ((r >> 1) & 7)) * 8,
                        reinterpret_cast<const uint16_t*>(sl + k * 1024));
        }
    };
    // the next tile (persistent axpy and poly): thread 0's atomic goes out before the last
    // two K steps and its result is published at the barrier that ends the main loop
    int grabbed = -1;

    bf16x8 fa[2][FM], fb[2][FN];
    bf16x4 ftr[2][FN][2];
    // The main loop is straight-line code: every condition below is a compile-time
    // constant (diagonal tile or not, last two K steps or not), so the compiler's wait
    // counts stay exact (a branch would make it wait for every outstanding load).
    auto run = [&](auto diag_c, auto pre_c, auto pat_c) {
        constexpr bool DG = decltype(diag_c)::value, PRE = decltype(pre_c)::value;
        constexpr int PAT = decltype(pat_c)::value;       // DIAG_PATTERN of the wave; PAT_FULL off the diagonal
        static_assert(DG || PAT == PAT_FULL, "patterns are for diagonal tiles");
        // prologue: K step 0 into stage 0 (already in the staging registers when PRE),
        // K step 1 into the staging registers
        if (!PRE) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) { gload_a(i, 0); if (!DG) gload_b(i, 0); }
        }
#pragma unroll
        for (int i = 0; i < NCH; ++i) { swrite_a(i, 0); if (!DG) swrite_b(i, 0); }
#pragma unroll
        for (int i = 0; i < NCH; ++i) { gload_a(i, 1); if (!DG) gload_b(i, 1); }
        lds_wait_barrier();
#pragma unroll
        for (int r = 0; r < NRD; ++r)
            if (need_frag(PAT, r)) rd(r, 0, 0, fa[0], fb[0], ftr[0]);
        join_tr(ftr[0], fb[0]);

        // One K step from stage ST.  Sub-step 1 writes operand A of K step kt + 1 from the
        // staging registers to the other stage and fetches its K step kt + 2; sub-step 2
        // does the same for operand B; sub-step 3 opens with the barrier that publishes
        // the other stage.  Each sub-step's first MFMA slots read the next sub-step's
        // fragments.
        auto kstep = [&](auto st_c, auto stage_c, auto load_c, int kt) {
            constexpr int ST = decltype(st_c)::value, SN = ST ^ 1;
            constexpr bool STAGE = decltype(stage_c)::value, LOAD = decltype(load_c)::value;
#pragma unroll
            for (int kk = 0; kk < KSUB; ++kk) {
                const int cur = kk & 1, nxt = cur ^ 1;
                const bool last = kk + 1 == KSUB;
#pragma unroll
                for (int f = 0; f < NMF; ++f) {
                    const int i = f / FN, j = f % FN;
                    __builtin_amdgcn_sched_barrier(0);
                    if (need_block(PAT, i, j))
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][j], fa[cur][i], acc[i][j], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (STAGE && last && f == 0) lds_wait_barrier();
                    if (f < NRD && (!last || STAGE) && need_frag(PAT, f))
                        rd(f, last ? SN : ST, last ? 0 : kk + 1, fa[nxt], fb[nxt], ftr[nxt]);
                    if (STAGE && kk == 1 && f >= NMF - NCH) {
                        swrite_a(f - (NMF - NCH), SN);
                        if (LOAD) gload_a(f - (NMF - NCH), kt + 2);
                    }
                    if (STAGE && !DG && kk == 2 && f >= NMF - NCH) {
                        swrite_b(f - (NMF - NCH), SN);
                        if (LOAD) gload_b(f - (NMF - NCH), kt + 2);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                if (!last || STAGE) join_tr(ftr[nxt], fb[nxt]);
            }
        };
        const std::true_type yes;
        const std::false_type no;
        for (int kt = 0; kt + 4 <= nk; kt += 2) {     // pairs whose K steps all fetch ahead
            kstep(ic<0>{}, yes, yes, kt);
            kstep(ic<1>{}, yes, yes, kt + 1);
        }
        if (HAS_E && PERSIST && threadIdx.x == 0) grabbed = grab_tile(p.sched, blockIdx.x % NUM_XCD, p.total_tiles);
        kstep(ic<0>{}, yes, no, nk - 2);
        if constexpr (HAS_E) e_issue(0);
        kstep(ic<1>{}, no, no, nk - 1);
    };
    // separate code for prefetched tiles, so that the compiler's wait before the first
    // staging write counts the previous epilogue's stores instead of merging with the
    // fresh-load path
    auto run_diag = [&](auto pre_c) {
        if constexpr (MODE != NS_AXPY) {
            switch ((DIAG_PATTERN >> (4 * wave)) & 15u) {
                case PAT_FULL: run(std::true_type{}, pre_c, ic<PAT_FULL>{}); break;
                case PAT_A: run(std::true_type{}, pre_c, ic<PAT_A>{}); break;
                case PAT_B: run(std::true_type{}, pre_c, ic<PAT_B>{}); break;
                default: run(std::true_type{}, pre_c, ic<PAT_NONE>{}); break;
            }
        }
    };
    if (prefetched) {
        if (diag) run_diag(std::true_type{});
        else run(std::false_type{}, std::true_type{}, ic<PAT_FULL>{});
    } else {
        if (diag) run_diag(std::false_type{});
        else run(std::false_type{}, std::false_type{}, ic<PAT_FULL>{});
    }
    // ---- epilogue ---------------------------------------------------------------------
    // The MFMAs take the right operand first, so each 32 x 32 block is accumulated
    // transposed: acc[i][j][4q + w] = D[wm0 + 32i + (lane & 31)][wn0 + 32j + 8q + 4(lane >> 5) + w],
    // four consecutive columns of one output row per lane and q.
    uint16_t* out = p.out + (int64_t)mat * p.stride_o;
    const int er = lane & 31, ec = 4 * (lane >> 5);
    // The next tile's K step 0 into the staging registers, ahead of the stores still to
    // come: the vector-memory counter retires in issue order and counts stores too, so the
    // next prologue then waits only for these loads, not for the stores to drain.
    auto prefetch_next = [&]() {
        // the staging registers' old contents are dead on every path from here (otherwise
        // they would stay live through the epilogue into the next iteration)
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            sa[i] = __builtin_nondeterministic_value(sa[i]);
            sb[i] = __builtin_nondeterministic_value(sb[i]);
        }
        if (b_next >= 0) {
            const int nmat0 = b_next / p.tiles_per_mat, nt = b_next - nmat0 * p.tiles_per_mat;
            const int nmat = p.reverse ? p.total_tiles / p.tiles_per_mat - 1 - nmat0 : nmat0;
            int nti, ntj;
            if (MODE == NS_AXPY) grid_decode(nt, p.tiles_m, p.tiles_n, nti, ntj);
            else tri_decode(nt, p.tiles_m, nti, ntj);
            const int64_t na0 = (int64_t)nti * TILE * p.lda;
            const __amdgpu_buffer_rsrc_t nra = make_rsrc(p.opa + (int64_t)nmat * p.stride_a + na0, p.stride_a - na0);
            const int64_t nb0 = (MODE == NS_AXPY) ? (int64_t)ntj * TILE : (int64_t)ntj * TILE * p.ldb;
            const __amdgpu_buffer_rsrc_t nrb = make_rsrc(p.opb + (int64_t)nmat * p.stride_b + nb0, p.stride_b - nb0);
            const bool ndiag = MODE != NS_AXPY && nti == ntj;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                sa[i] = __builtin_amdgcn_raw_buffer_load_b128(nra, va, i * RP_ROWS * p.lda * 2, 0);
                if (MODE == NS_AXPY)
                    sb[i] = __builtin_amdgcn_raw_buffer_load_b128(nrb, vb_kn, KN_ROWS * i * p.ldb * 2, 0);
                else if (!ndiag)
                    sb[i] = __builtin_amdgcn_raw_buffer_load_b128(nrb, vb_rp, i * RP_ROWS * p.ldb * 2, 0);
            }
        }
    };
    // Each wave finishes its own region without workgroup barriers: for each half, the E
    // values at its own lanes' positions (axpy: X, poly: A), the combine (the axpy's product
    // has gamma = 1, so its product term is the accumulator itself), the results written
    // over those same 8 bytes, then read back as whole 128-byte row pieces (8 lanes per row)
    // and stored; off the diagonal the poly also stores the half's mirror into tile (tj, ti),
    // read back transposed.  Half 1's E rows go out first, so they arrive while half 0 is
    // combined and stored.  On a diagonal poly tile only the blocks on or above the
    // diagonal are stored from the regions; after a workgroup barrier (every wave's two
    // slots then hold its region) the blocks below it are stored as the transposes of
    // those above, read from the slots of the waves that computed them.
    auto epilogue_per_wave = [&]() {
        if (PERSIST && threadIdx.x == 0) next_slot = grabbed;
        lds_wait_barrier();                               // stage 1 is free; the next tile is published
        if (PERSIST) b_next = next_slot;
        if constexpr (HAS_E) e_issue(1);
        auto soff = [](int r, int c) { return r * 128 + (((c >> 3) ^ ((r >> 1) & 7)) << 4) + (c & 7) * 2; };
        auto half = [&](auto h_c) {
            constexpr int H = decltype(h_c)::value;
            char* sl = smem + slot(H);
            uint2 res[2][FN][4];
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int off = soff(32 * ii + er, 32 * j + 8 * q + ec);
                        float v[4];
#pragma unroll
                        for (int w = 0; w < 4; ++w) v[w] = acc[2 * H + ii][j][4 * q + w];
                        if constexpr (HAS_E) {
                            uint2 e = *reinterpret_cast<const uint2*>(sl + off);
                            if (NORM) e = dev::normalize4(e, 8, s_norm);
                            const uint32_t ew[4] = {e.x << 16, e.x & 0xffff0000u, e.y << 16, e.y & 0xffff0000u};
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                const float ef = __builtin_bit_cast(float, ew[w]);
                                v[w] = (MODE == NS_AXPY) ? __builtin_fmaf(p.alpha, ef, v[w])
                                                         : dev::ns_combine(p.alpha, ef, p.gamma, v[w]);
                            }
                        }
                        res[ii][j][q].x = dev::f32x2_to_bf16x2(v[0], v[1]);
                        res[ii][j][q].y = dev::f32x2_to_bf16x2(v[2], v[3]);
                    }
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < FN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(sl + soff(32 * ii + er, 32 * j + 8 * q + ec)) = res[ii][j][q];
            // the other lanes' results written before they are read back
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_waitcnt(0xc07f);           // lgkmcnt(0)
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            uint16_t* orow = out + (int64_t)(ti * TILE + wm0 + 64 * H) * p.ldo + (int64_t)(tj * TILE + wn0);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = 8 * k + (lane >> 3), pos = lane & 7, g = pos ^ ((r >> 1) & 7);
                const uint4 v = *reinterpret_cast<const uint4*>(sl + r * 128 + pos * 16);
                // a diagonal tile's blocks below the diagonal were not computed
                if (MODE == NS_POLY && diag && ((wm0 + 64 * H + r) >> 5) > ((wn0 + 8 * g) >> 5)) continue;
                *reinterpret_cast<uint4*>(orow + (int64_t)r * p.ldo + g * 8) = v;
            }
            if (MODE == NS_POLY && !diag) {
                // the mirror: row c of it is column c of the half; a transposing read over 16
                // lanes turns 4 slot rows x 16 columns into 16 mirrored rows x 4 elements, two
                // of them give each lane 16 bytes of one mirrored row (8 units of 16 mirrored
                // rows x 32 slot rows)
                uint16_t* omir = out + (int64_t)(tj * TILE + wn0) * p.ldo + (int64_t)(ti * TILE + wm0 + 64 * H);
                const int x = lane & 15, grp = lane >> 4;
                const int ax = x & 3, mx = x >> 2;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c0 = (u & 3) * 16, r0 = (u >> 2) * 32 + 8 * grp;
                    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(sl + soff(r0 + mx, c0 + 4 * ax)));
                    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(sl + soff(r0 + 4 + mx, c0 + 4 * ax)));
                    const bf16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    *reinterpret_cast<bf16x8*>(omir + (int64_t)(c0 + x) * p.ldo + r0) = v8;
                }
            }
        };
        if constexpr (HAS_E) wait_vm<8, true>();          // half 0's E rows (half 1's 8 loads may be out)
        half(ic<0>{});
        if (PF) prefetch_next();
        // half 1's E rows: younger than them are half 0's stores (8 rows, and 8 mirrored off
        // the diagonal of the poly; on the diagonal some row stores may be skipped, so
        // everything is waited for) and the axpy's 8 prefetch loads
        if constexpr (MODE == NS_POLY) {
            if (diag) wait_vm<0, true>();
            else wait_vm<16, true>();
        } else {
            if (PF && b_next >= 0) wait_vm<16, true>();
            else wait_vm<8, true>();
        }
        half(ic<1>{});
        if constexpr (MODE == NS_POLY) {
            if (diag) {
                __syncthreads();                          // every wave's slots hold its region
                // the 28 blocks (bi, bj) below the diagonal, each as two units of 16 rows x 32
                // columns, 7 units per wave: rows bi*32 + 16s + x of the tile, columns
                // bj*32 + 8*grp .. + 7, read transposed from block (bj, bi) in the slot of the
                // wave whose region holds it
                const int x = lane & 15, grp = lane >> 4;
                const int ax = x & 3, mx = x >> 2;
                uint16_t* otile = out + (int64_t)(ti * TILE) * p.ldo + (int64_t)(ti * TILE);
#pragma unroll 1
                for (int u = wave; u < 56; u += NW) {
                    int k = u >> 1, bi = 1;
                    while (k >= bi) { k -= bi; ++bi; }
                    const int bj = k, sh = u & 1;
                    const int owner = (int)((DIAG_REGION_WAVE >> (4 * (4 * (bj >> 2) + (bi >> 1)))) & 15u);
                    const int lr0 = (bj & 3) * 32, lc0 = (bi & 1) * 32 + 16 * sh;
                    const int h = lr0 >> 6, sr0 = (lr0 & 63) + 8 * grp;
                    const char* osl = smem + ((owner < 4) ? (h ? RP_B : 0) : (h ? OFF_B + B_STAGE : OFF_B)) +
                                      (owner & 3) * 8192;
                    const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(osl + soff(sr0 + mx, lc0 + 4 * ax)));
                    const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(osl + soff(sr0 + 4 + mx, lc0 + 4 * ax)));
                    const bf16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    *reinterpret_cast<bf16x8*>(otile + (int64_t)(bi * 32 + 16 * sh + x) * p.ldo + bj * 32 + 8 * grp) = v8;
                }
            }
        }
    };
    if constexpr (HAS_E) {
        epilogue_per_wave();
    } else {
    // SYRK: the whole tile goes through LDS (row r at r * 512 bytes, 16-byte granule G stored
    // at granule G ^ (r & 31)) between workgroup barriers and leaves in whole 512-byte rows,
    // its mirror in 64-byte row pieces assembled with transposing reads.
    char* T = smem;
    auto tb = [](int r, int c) { return r * 512 + (((c >> 3) ^ (r & 31)) << 4) + (c & 7) * 2; };
    lds_wait_barrier();                                   // every wave is done with the K stages
    // the next tile: the atomic goes out now and its result is published to the workgroup
    // at the barrier after the result tile is staged
    if (PERSIST && threadIdx.x == 0) grabbed = grab_tile(p.sched, blockIdx.x % NUM_XCD, p.total_tiles);
    uint2 res[FM][FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] = acc[i][j][4 * q + w];
                res[i][j][q].x = dev::f32x2_to_bf16x2(v[0], v[1]);
                res[i][j][q].y = dev::f32x2_to_bf16x2(v[2], v[3]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2*>(T + tb(wm0 + 32 * i + er, wn0 + 32 * j + 8 * q + ec)) = res[i][j][q];
    if (PERSIST && threadIdx.x == 0) next_slot = grabbed;
    lds_wait_barrier();
    if (PERSIST) b_next = next_slot;
    if (PF) prefetch_next();
    // the tile: 256 rows x 32 granules, whole rows per 32 lanes
    uint16_t* orow = out + (int64_t)ti * TILE * p.ldo + (int64_t)tj * TILE;
#pragma unroll
    for (int s2 = 0; s2 < TILE * 32 / NT; ++s2) {
        const int gi = tid + NT * s2;
        const int r = gi >> 5, g = gi & 31;
        // a diagonal tile's blocks below the diagonal were not computed: mirrored below
        if (ti == tj && (g >> 2) < (r >> 5)) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(T + r * 512 + ((g ^ (r & 31)) << 4));
        *reinterpret_cast<uint4*>(orow + (int64_t)r * p.ldo + g * 8) = v;
    }
    // the mirrored tile (symmetric products): row c of it is column c of the tile.  Off the
    // diagonal it goes to tile (tj, ti) whole; on the diagonal its blocks below the diagonal
    // fill those of the tile itself.  A transposing read over 16 lanes turns 4 tile rows x 16
    // columns into 16 mirrored rows x 4 elements; two of them give each lane 16 bytes of one
    // mirrored row.
    {
        uint16_t* omir = out + (int64_t)tj * TILE * p.ldo + (int64_t)ti * TILE;
        const int x = lane & 15, grp = lane >> 4;
        const int ax = x & 3, mx = x >> 2;
#pragma unroll 2
        for (int u0 = 0; u0 < 128; u0 += NW) {            // 16 columns x 32 rows per unit
            const int u = u0 + wave;
            // mirrored rows c0 .. c0 + 15 (block (u & 15) / 2), columns of tile rows block u / 16
            if (ti == tj && ((u & 15) >> 1) <= (u >> 4)) continue;
            const int c0 = (u & 15) * 16, r0 = (u >> 4) * 32 + 8 * grp;
            const bf16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(T + tb(r0 + mx, c0 + 4 * ax)));
            const bf16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(T + tb(r0 + 4 + mx, c0 + 4 * ax)));
            const bf16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            *reinterpret_cast<bf16x8*>(omir + (int64_t)(c0 + x) * p.ldo + r0) = v8;
        }
    }
    }
  }
  // The launch's last workgroup to finish sets the counters back to zero for the next
  // launch (every other workgroup has taken its last, empty, grab before counting itself
  // finished, so nothing reads them afterwards in this launch).
  if (PERSIST && threadIdx.x == 0) {
      __threadfence();
      if (atomicAdd(&p.sched[NUM_XCD], 1u) == gridDim.x - 1) {
#pragma unroll
          for (int x = 0; x <= NUM_XCD; ++x) atomicExch(&p.sched[x], 0u);
      }
  }
}

// Persistent launches of the 256-tile kernel (one workgroup per CU) when every workgroup
// gets at least two tiles: no workgroup exit and relaunch between tiles, and a tile's
// stores drain while the next tile's first loads go out.  Measured on gfx950: the axpy
// 2.8 % and SYRK/POLY 0.7 % faster at 2048 x 2048 x 128.
constexpr int PERSIST_GRID = 256;

template <int MODE, int TILE, int WM, int WN, int BK, int STAGES>
hipError_t launch_cfg(const NsArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ns_gemm_kernel<MODE, TILE, WM, WN, BK, STAGES>), dim3((unsigned)a.total_tiles),
                       dim3(64 * WM * WN), 0, s, a);
    return hipGetLastError();
}

template <int MODE, bool NORM>
void launch_vs(const NsArgs& a, hipStream_t s) {
    if (a.total_tiles >= 2 * PERSIST_GRID)
        hipLaunchKernelGGL((ns_vs_kernel<MODE, VS_WM, VS_WN, true, NORM>), dim3((unsigned)PERSIST_GRID),
                           dim3(64 * VS_WM * VS_WN), 0, s, a);
    else
        hipLaunchKernelGGL((ns_vs_kernel<MODE, VS_WM, VS_WN, false, NORM>), dim3((unsigned)a.total_tiles),
                           dim3(64 * VS_WM * VS_WN), 0, s, a);
}

template <int MODE>
hipError_t launch_mode(int32_t tile, const NsArgs& a, hipStream_t s) {
    switch (tile) {
        case TILE_256:
            if constexpr (MODE != NS_POLY) {
                if (a.inv) launch_vs<MODE, true>(a, s);
                else launch_vs<MODE, false>(a, s);
            } else {
                if (a.inv) return hipErrorInvalidValue;
                launch_vs<MODE, false>(a, s);
            }
            return hipGetLastError();
        case TILE_128:
            if (a.inv) return hipErrorInvalidValue;   // the direct-to-LDS tiles do not normalise
            return launch_cfg<MODE, 128, 2, 2, 64, 2>(a, s);
        case TILE_64:
            if (a.inv) return hipErrorInvalidValue;
            return launch_cfg<MODE, 64, 2, 2, 64, 2>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Two workgroups per CU (64 KB of LDS each), at most one queue entry each per round.
constexpr int GROUPED_GRID = 512;

template <int MODE>
hipError_t launch_grouped_mode(const GroupedNsArgs& g, hipStream_t s) {
    const int grid = g.total_tiles < GROUPED_GRID ? g.total_tiles : GROUPED_GRID;
    hipLaunchKernelGGL((ns_grouped_kernel<MODE>), dim3((unsigned)grid), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_ns(NsMode mode, int32_t tile, const NsArgs& a, hipStream_t s) {
    switch (mode) {
        case NS_SYRK: return launch_mode<NS_SYRK>(tile, a, s);
        case NS_POLY: return launch_mode<NS_POLY>(tile, a, s);
        case NS_AXPY: return launch_mode<NS_AXPY>(tile, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ns_grouped(NsMode mode, const GroupedNsArgs& g, hipStream_t s) {
    if (g.n_jobs < 1 || g.n_jobs > GROUPED_MAX_JOBS || g.total_tiles < 1) return hipErrorInvalidValue;
    for (int j = 0; j < g.n_jobs; ++j)
        if ((g.job[j].tile != TILE_128 && g.job[j].tile != TILE_64) || g.job[j].a.inv) return hipErrorInvalidValue;
    switch (mode) {
        case NS_SYRK: return launch_grouped_mode<NS_SYRK>(g, s);
        case NS_POLY: return launch_grouped_mode<NS_POLY>(g, s);
        case NS_AXPY: return launch_grouped_mode<NS_AXPY>(g, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace muon
