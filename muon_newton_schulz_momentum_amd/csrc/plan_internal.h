// Internal plan layout shared by the host planner (plan.cpp, HIP-free) and the launch
// layer (api.hip).  Not part of the public ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/muon.h"

namespace muon {

// One matrix as the device kernels see it.  The table of these lives in the workspace
// (uploaded once by muon_plan_bind); it is the one-GPU form of the pages' cached
// resharding metadata.  64 bytes per row.
struct MatEntry {
    float* w;             // weight, rows x cols fp32
    float* m;             // momentum, rows x cols fp32
    const void* g;        // gradient, rows x cols (fp32 or bf16)
    int64_t rows;
    int64_t cols;
    int32_t trans;        // 1: canonical X is the transpose (rows > cols)
    float scale;          // update scale s_i
    int64_t pad_[2];
};
static_assert(sizeof(MatEntry) == 64, "MatEntry layout");

// Newton–Schulz tile configurations (square output tiles of edge `tile`).
enum TileCfg : int32_t { TILE_256 = 256, TILE_128 = 128, TILE_64 = 64 };

struct Chunk {
    int32_t bucket;
    int32_t grad_dtype;
    int64_t m, n;            // canonical shape
    int64_t mp, np;          // padded shape: multiples of the tile
    int32_t tile;
    bool fused = false;      // the whole NS runs in the fused small-matrix kernel
    bool grouped = false;    // a small tiled chunk: NS in the grouped launches of all such chunks
    int64_t count;           // matrices in this chunk
    int64_t first;           // first row of this chunk in the matrix table
    // elementwise tiling: 64 x 64 tiles over rows x cols (same count for both orientations)
    int64_t ew_tiles;
    // workspace layout (byte offsets from the workspace base); region_base identifies the
    // region the chunk's buffers live in (grouped small chunks share one, back to back)
    uint64_t region_off, region_bytes, region_base;
    uint64_t off_xp, off_xq, off_a, off_b, off_part, off_inv;
    uint64_t off_sched;      // tile-queue counters of the persistent product kernels (zero between launches)
    uint64_t off_table;      // this chunk's first table row
};

// A parameter that takes AdamW (64 B), and one segment of ADAM_SEG of its elements.
struct AdamEntry {
    float* w;
    float* m;
    float* v;
    const void* g;
    int64_t numel;
    int32_t grad_dtype;
    int32_t pad[3];
};
struct AdamSeg {
    int32_t entry;
    int32_t pad;
    int64_t start;
};
constexpr int64_t ADAM_SEG = 4096;   // elements per AdamW segment (one block's work)

struct ParamRec {
    int32_t ndim;
    int32_t grad_dtype;
    int64_t rows, cols;
    float* w;
    float* m;
    const void* g;
    float* v = nullptr;      // AdamW second moment
    int32_t included;        // 1 Muon, 2 AdamW, 0 excluded
    int32_t chunk;           // Muon: chunk; AdamW: index in the AdamW table
    int64_t slot;
    int32_t trans;
};

struct TimingState {
    int32_t capacity = 0;
    int32_t used = 0;
    std::vector<void*> ev_begin, ev_end;       // hipEvent_t, created lazily by the launch layer
    std::vector<int32_t> kind;
    std::vector<double> work;
};

}  // namespace muon

struct muon_plan {
    std::vector<muon::ParamRec> params;
    std::vector<muon::Chunk> chunks;
    std::vector<muon::MatEntry> table;  // host copy, chunk-major
    int32_t n_buckets = 0;
    int64_t n_included = 0, n_excluded = 0;
    bool shared_regions = false;
    uint32_t flags = 0;      // MUON_PLAN_* bits
    uint64_t table_bytes = 0;    // matrix table + AdamW tables (the start of the workspace)
    std::vector<muon::AdamEntry> adam;
    std::vector<muon::AdamSeg> adam_segs;
    int64_t adam_elements = 0;
    uint64_t off_adam = 0, off_adam_segs = 0;
    uint64_t ws_bytes = 0;
    // bind state
    void* ws = nullptr;
    uint64_t ws_given = 0;
    bool bound = false;
    muon::TimingState timing;
    // the two-stream pipeline: a second stream and its ordering events, created at bind
    void* side = nullptr;                 // hipStream_t
    std::vector<void*> pipe_events;       // hipEvent_t, timing disabled
    // per chunk, in the order calls were enqueued: 1 when the workspace holds a fresh X0 =
    // bf16(M) from muon_momentum_update that no Newton–Schulz call has consumed yet (the
    // iterations overwrite X0 with their ping-pong buffers)
    std::vector<uint8_t> x0_fresh;
};

// An instantiated graph of one whole step.  It holds the device addresses of the
// workspace it was captured against, not the host plan.
struct muon_graph {
    void* graph = nullptr;   // hipGraph_t
    void* exec = nullptr;    // hipGraphExec_t
    int64_t nodes = 0;
    void* ws = nullptr;
};

namespace muon {

// Thread-local error message shared by both translation units.
muon_status set_error(muon_status s, const std::string& msg);
void clear_error();

constexpr int EW_TILE = 64;          // elementwise tile edge
constexpr int SMALL_NS_MAX_N = 1024; // widest padded n of the fused small-matrix kernel
constexpr uint64_t WS_ALIGN = 256;   // workspace sub-buffer alignment
constexpr uint64_t SCHED_BYTES = 256; // per region: 8 per-XCD tile counters and a finished count (uint32)
// MUON_PLAN_PIPELINE chunking: at most this many chunks per bucket, each with at least this
// many SYRK workgroups
constexpr int64_t PIPE_MAX_SPLIT = 8;
constexpr int64_t PIPE_MIN_WG = 2048;
// chunks per bucket the planner may make: the pipeline split and two edge chunks
constexpr int64_t PIPE_MAX_CHUNKS = PIPE_MAX_SPLIT + 2;

// Estimates for the two-stream step (placement on the side stream at step time, edge
// chunks at plan time), near the rates measured on gfx950 with the side kernels running:
// the products' algorithmic rate by the short side m (about 0.9 PFLOP/s at m = 1024, 1.0
// at 2048, 1.1 from 4096 on), the side kernels 1.34-1.92 TB/s (normaliser, apply,
// momentum).  A single conservative 1.2 PFLOP/s and 1.5 TB/s left applies that would have
// fitted on the caller's stream: the 261 GB MoE slice ran 2.4 % slower with them, and one
// 1.0 PFLOP/s for every shape cost the MoE bucket (m = 1024) 1.8 %.
inline double est_ns_rate(int64_t m) {      // FLOP/s, the product kernels
    return m >= 4096 ? 1.1e15 : m >= 2048 ? 1.0e15 : m >= 1024 ? 0.9e15 : 0.5e15;
}
constexpr double EST_SIDE_BW = 1.6e12;      // B/s, the side-stream elementwise kernels
constexpr double EST_FULL_BW = 5.0e12;      // B/s, the full-speed elementwise kernels
constexpr double EST_CHUNK_S = 1.0e-4;      // s, fixed cost of one more chunk (launches, ramps)
constexpr double EST_SIDE_COST = 0.5;       // what side work costs the products beside it, as a
                                            // fraction of its one-stream time (measured)
constexpr int64_t EST_CUS = 256;            // compute units: one 256-tile workgroup each
constexpr int32_t EST_STEPS = 5;            // Newton–Schulz iterations assumed at plan time

// Algorithmic FLOPs of one Newton–Schulz iteration over `count` canonical m x n matrices
// (the three products, the symmetric ones on one triangle).
inline double ns_iter_flops(int64_t count, int64_t m_, int64_t n_) {
    const double m = (double)m_, n = (double)n_;
    return (double)count * (m * (m + 1.0) * n + m * m * (m + 1.0) + 2.0 * m * m * n);
}
// Bytes per element of the elementwise passes: momentum with the normaliser, and apply.
inline double prep_bytes_per_elem(int32_t grad_dtype) { return (grad_dtype == MUON_DTYPE_F32 ? 14.0 : 12.0) + 4.0; }
constexpr double APPLY_BYTES_PER_ELEM = 10.0;

// Side-stream placement of the two-stream step, for tiled chunks 0 .. T-1 in step order.
// window[j]: estimated time of chunk j's products; prep[j], apply[j]: estimated side-stream
// time of chunk j's momentum with normaliser, and of its apply.  Window j takes P_{j+1} and
// A_{j-1} if both fit, else whichever of the two fits (P first: a P left on the main stream
// holds up the next window), else neither.  Sets p_side[j] / a_side[j] for the tasks that
// go to the side stream.
inline void pipe_place(const std::vector<double>& window, const std::vector<double>& prep,
                       const std::vector<double>& apply, std::vector<char>& p_side, std::vector<char>& a_side) {
    const size_t T = window.size();
    p_side.assign(T, 0);
    a_side.assign(T, 0);
    for (size_t j = 0; j < T; ++j) {
        const bool has_p = j + 1 < T, has_a = j > 0;
        const double tp = has_p ? prep[j + 1] : 0.0, ta = has_a ? apply[j - 1] : 0.0;
        if (has_p && has_a && tp + ta <= window[j]) {
            p_side[j + 1] = a_side[j - 1] = 1;
        } else if (has_p && tp <= window[j]) {
            p_side[j + 1] = 1;
        } else if (has_a && ta <= window[j]) {
            a_side[j - 1] = 1;
        }
    }
}

inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace muon
