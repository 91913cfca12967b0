// Launch wrappers for the libmuon kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_internal.h"

namespace muon {

struct MomentumArgs {
    const MatEntry* tbl;   // the chunk's table rows (device)
    uint16_t* xq;          // X0 destination: count matrices of mp x np bf16
    double* partials;      // count * ew_tiles sums of squares
    int64_t mat_stride;    // mp * np
    int64_t np;
    int64_t ew_tiles;
    int64_t total_tiles;   // count * ew_tiles
    float beta, omb;       // beta and (1 - beta), both as the caller's float32
    const float* dev_scalars;  // nullable device {beta, lr, wd}: beta is read from it instead
    int32_t nesterov;      // 1: X0 = bf16(f32(beta*M_new + (1-beta)*G)) instead of bf16(M_new)
};

// Words of a chunk's tile-queue block (8 per-XCD counters and a finished count).
constexpr int SCHED_WORDS = 9;

struct FinalizeArgs {
    const double* partials;
    double* inv;           // per matrix: the float32 normalisation scale of 1 / (sqrt(sum) + eps)
    int64_t ew_tiles;
    double eps;
    // the chunk's tile-queue block, zeroed here before its product launches: in a region
    // shared with other chunks, their data may have overwritten it since its last use
    uint32_t* sched;
    // nullable: X0 (count matrices of mp x np bf16, valid m x n) whose padding is zeroed
    // here, for chunks whose first iteration normalises X0 as it loads it
    uint16_t* x0;
    int64_t m, n, mp, np;
};

struct NormalizeArgs {
    const uint16_t* src;   // X0 (valid m x n region, row stride np)
    uint16_t* dst;         // X, whole mp x np region (pads zeroed); may equal src
    const double* inv;
    int64_t m, n, mp, np;
    int64_t total_units;   // count * mp * np / 8
};

struct ApplyArgs {
    const MatEntry* tbl;
    const uint16_t* xo;    // O: count matrices of mp x np bf16 (canonical orientation)
    int64_t mat_stride;
    int64_t np;
    int64_t ew_tiles;
    int64_t total_tiles;
    double d;              // 1 - lr*wd, formed in float64
    float lr;
    const float* dev_scalars;  // nullable device {beta, lr, wd}: lr and wd are read from it instead
};

struct AdamArgs {
    const AdamEntry* entries;
    const AdamSeg* segs;
    int64_t n_segs;
    double lr, wd, beta1, omb1, beta2, omb2, eps, bc1, bc2;   // float32 inputs, widened
    const float* dev_scalars;   // nullable device {lr, wd, bc1, bc2}
};

// Newton–Schulz GEMM kernels.  opa/opb are matrix-0 bases; every matrix of the chunk
// sits `stride_*` elements after the previous one.
enum NsMode : int32_t { NS_SYRK = 0, NS_POLY = 1, NS_AXPY = 2 };

struct NsArgs {
    const uint16_t* opa;   // SYRK: X; POLY: A; AXPY: B   (row panels, K contiguous)
    const uint16_t* opb;   // SYRK: X; POLY: A; AXPY: X   (AXPY: K x N, N contiguous)
    const uint16_t* ep;    // epilogue input: POLY: A; AXPY: X; SYRK: unused
    uint16_t* out;         // SYRK: A; POLY: B; AXPY: X'
    int64_t stride_a, stride_b, stride_o;
    int32_t lda, ldb, ldo;
    int32_t K;             // reduction length (multiple of 64)
    int32_t tiles_m;       // tiles along M (SYRK/POLY: along the side)
    int32_t tiles_n;       // AXPY: tiles along N
    int32_t tiles_per_mat;
    int32_t total_tiles;
    float alpha;           // POLY: b (times A); AXPY: a (times X)
    float gamma;           // POLY: c (times the product); AXPY: 1
    // persistent launches: 8 per-XCD tile counters and a finished count, zero at launch
    // (the finalize kernel zeroes them before a chunk's first product launch, and each
    // launch's last workgroup sets them back to zero for the next)
    uint32_t* sched;
    // Normalisation fused into the first iteration's loads (256-tile SYRK and AXPY only):
    // when set, every X operand value is read as X0 and used as bf16(X0 * (float)inv[matrix])
    // (the separate normalize pass's arithmetic); X0's padding must be zero (the finalize
    // kernel zeroes it for such chunks).
    const double* inv;
    // Nonzero: the 256-row tile kernels take the chunk's matrices in reverse order (the
    // tiles of each matrix in the usual order); the other tile sizes ignore it.
    int32_t reverse;
};

// Every small tiled chunk (128- or 64-row tiles) of a plan in one launch per product: job
// j is one chunk's NsArgs (as for launch_ns) and its first entry in the launch's tile queue.
constexpr int GROUPED_MAX_JOBS = 12;

struct GroupedJob {
    NsArgs a;
    int32_t tile;          // TILE_128 or TILE_64
    int32_t first;         // queue index of the job's tile 0
};

struct GroupedNsArgs {
    GroupedJob job[GROUPED_MAX_JOBS];
    int32_t n_jobs;
    int32_t total_tiles;
};

// The normalisation of small tiled chunks in one launch: per matrix, the normaliser summed
// and searched as the finalize kernel does, then X = bf16(X0 * scale) as the normalize kernel does
// it, the matrix's units spread over `blocks` workgroups (each sums the partials itself).
constexpr int PREP_MAX_JOBS = 12;
struct PrepJob {
    const double* partials;
    const uint16_t* src;   // X0
    uint16_t* dst;         // X (may equal src)
    int64_t ew_tiles;
    int64_t m, n, mp, np;
    int64_t blocks;        // workgroups per matrix
    int64_t first;         // first workgroup of this job
};
struct PrepGroupArgs {
    PrepJob job[PREP_MAX_JOBS];
    int32_t n_jobs;
    int64_t total_blocks;
    double eps;
};

// Whole Newton–Schulz of small matrices (canonical m <= 64, padded n <= SMALL_NS_MAX_N,
// see plan_internal.h),
// one workgroup per matrix; every job is one chunk of such matrices.

constexpr int SMALL_NS_MAX_JOBS = 8;
constexpr int SMALL_NS_MAX_STEPS = 32;   // longest coefficient schedule the fused kernel holds

struct SmallJob {
    const uint16_t* xq;        // X0: count matrices of 64 x np bf16
    uint16_t* xp;              // O: count matrices of 64 x np bf16
    const double* partials;    // count * ew_tiles sums of squares
    int64_t ew_tiles;
    int32_t m, n, np;
    int32_t first;             // first workgroup of this job
};

struct SmallNsArgs {
    SmallJob job[SMALL_NS_MAX_JOBS];
    int32_t n_jobs;
    int32_t steps;
    float abc[SMALL_NS_MAX_STEPS][3];   // (a, b, c) of each iteration
    double eps;
};

hipError_t launch_momentum(const MomentumArgs& a, int32_t grad_dtype, hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, int64_t count, hipStream_t s);
hipError_t launch_normalize(const NormalizeArgs& a, hipStream_t s);
hipError_t launch_apply(const ApplyArgs& a, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, hipStream_t s);
// Side-stream variants (same results; sized to run beside the Newton–Schulz products).
hipError_t launch_momentum_side(const MomentumArgs& a, int32_t grad_dtype, hipStream_t s);
hipError_t launch_normalize_side(const NormalizeArgs& a, hipStream_t s);
hipError_t launch_apply_side(const ApplyArgs& a, hipStream_t s);
hipError_t launch_ns(NsMode mode, int32_t tile, const NsArgs& a, hipStream_t s);
hipError_t launch_ns_small(const SmallNsArgs& a, int64_t total, hipStream_t s);
hipError_t launch_ns_grouped(NsMode mode, const GroupedNsArgs& g, hipStream_t s);
hipError_t launch_prep_grouped(const PrepGroupArgs& g, hipStream_t s);
// Zero `units` 16-byte units at `dst` (a kernel, so it may sit in a captured graph).
hipError_t launch_zero(void* dst, uint64_t units, hipStream_t s);

}  // namespace muon
