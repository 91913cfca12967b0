// Host planner: shape buckets, chunks, workspace layout and the per-matrix tables.
//
// This translation unit makes no HIP call; it builds with any C++17 compiler so the
// planner can be tested on a machine without a GPU (and under sanitizers).
//
// The pages batch same-shape momentum matrices before the exchange and cache the
// resharding index metadata because a MoE model has thousands of same-shape experts
// ("Frontier Pre-training at Microsoft AI", method details section 5, resharding step 2
// and the tuning notes after it).  On one GPU the same idea is the plan: computed once,
// uploaded once, reused every step.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <new>
#include <tuple>

#include "plan_internal.h"

namespace muon {

namespace {
thread_local std::string g_last_error;
}

muon_status set_error(muon_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

void clear_error() { g_last_error.clear(); }

namespace {

// Which optimizer a parameter takes (see muon_param_desc).
constexpr int32_t ROLE_NONE = 0, ROLE_MUON = 1, ROLE_ADAMW = 2;
int32_t param_role(const muon_param_desc& d) {
    if (d.optimizer == MUON_OPT_ADAMW) return ROLE_ADAMW;
    if (d.optimizer == MUON_OPT_NONE) return ROLE_NONE;
    if (d.ndim == 2) return ROLE_MUON;
    return d.exp_avg_sq ? ROLE_ADAMW : ROLE_NONE;
}

// The update scale of a shape rule (MUON_SCALE_*), computed in float64 and rounded once
// to float32.
float rule_scale(int32_t mode, int64_t rows, int64_t cols) {
    const double r = (double)rows, c = (double)cols;
    switch (mode) {
        case MUON_SCALE_ASPECT: return (float)std::sqrt(r / c > 1.0 ? r / c : 1.0);
        case MUON_SCALE_RMS_MATCH: return (float)(0.2 * std::sqrt(r > c ? r : c));
        default: return 1.0f;
    }
}

int32_t pick_tile(int64_t m) {
    if (m >= 1024) return TILE_256;
    if (m > 128) return TILE_128;
    return TILE_64;
}

// Bytes one matrix adds to a chunk region: two X buffers, A and B, and the norm partials.
uint64_t per_matrix_bytes(int64_t mp, int64_t np, int64_t ew_tiles) {
    return 2ull * (uint64_t)mp * (uint64_t)np * 2ull      // X ping-pong (bf16)
         + 2ull * (uint64_t)mp * (uint64_t)mp * 2ull      // A and B (bf16)
         + (uint64_t)ew_tiles * 8ull                      // per-tile sums of squares (fp64)
         + 8ull;                                          // 1/(||X0|| + eps) (fp64)
}

void layout_region(Chunk& c, uint64_t base) {
    uint64_t off = base;
    const uint64_t xb = (uint64_t)c.count * c.mp * c.np * 2ull;
    const uint64_t ab = (uint64_t)c.count * c.mp * c.mp * 2ull;
    c.off_xp = off; off = align_up(off + xb, WS_ALIGN);
    c.off_xq = off; off = align_up(off + xb, WS_ALIGN);
    c.off_a = off;  off = align_up(off + ab, WS_ALIGN);
    c.off_b = off;  off = align_up(off + ab, WS_ALIGN);
    c.off_part = off; off = align_up(off + (uint64_t)c.count * c.ew_tiles * 8ull, WS_ALIGN);
    c.off_inv = off;  off = align_up(off + (uint64_t)c.count * 8ull, WS_ALIGN);
    c.off_sched = off; off = align_up(off + SCHED_BYTES, WS_ALIGN);
    c.region_off = base;
    c.region_bytes = off - base;
    c.region_base = base;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// One shape bucket: canonical and padded shape, product tile, elementwise tiles per
// matrix, gradient dtype and its parameters in plan order.
struct BucketGeo { int64_t m, n, mp, np, ew; int32_t tile, gdt; std::vector<int64_t> members; };

// The estimated time of a two-stream step over tiled chunks (bucket, count) in step order:
// the first chunk's momentum and normaliser and the last one's apply at full speed, every
// chunk's products, a fixed cost per chunk, the side-stream tasks that pipe_place leaves
// on the main stream, and what the tasks it moves beside the products cost them.  Window
// sizes are estimated as at step time (algorithmic FLOPs); a 256-tile chunk's products are
// timed by the waves of tiles each launch runs (x tiles take ceil(x / EST_CUS) tile
// times), so that a split which adds a partial wave costs what it costs.
double est_pipelined_step(const std::vector<std::pair<const BucketGeo*, int64_t>>& seq) {
    const size_t T = seq.size();
    std::vector<double> win(T), prep(T), apply(T), prep_full(T), apply_full(T), ns(T);
    for (size_t j = 0; j < T; ++j) {
        const BucketGeo& g = *seq[j].first;
        const double cu_rate = est_ns_rate(g.m) / (double)EST_CUS;
        const int64_t c = seq[j].second;
        const double el = (double)c * (double)g.m * (double)g.n;
        win[j] = EST_STEPS * ns_iter_flops(c, g.m, g.n) / est_ns_rate(g.m);
        prep[j] = el * prep_bytes_per_elem(g.gdt) / EST_SIDE_BW;
        apply[j] = el * APPLY_BYTES_PER_ELEM / EST_SIDE_BW;
        prep_full[j] = el * prep_bytes_per_elem(g.gdt) / EST_FULL_BW;
        apply_full[j] = el * APPLY_BYTES_PER_ELEM / EST_FULL_BW;
        if (g.tile == TILE_256) {
            const int64_t tm = g.mp / TILE_256, tn = g.np / TILE_256;
            const double t_syrk = 2.0 * TILE_256 * TILE_256 * (double)g.np / cu_rate;
            const double t_sq = 2.0 * TILE_256 * TILE_256 * (double)g.mp / cu_rate;   // POLY, AXPY
            const double w_tri = (double)ceil_div(tm * (tm + 1) / 2 * c, EST_CUS);
            const double w_full = (double)ceil_div(tm * tn * c, EST_CUS);
            ns[j] = EST_STEPS * (w_tri * (t_syrk + t_sq) + w_full * t_sq);
        } else {
            ns[j] = win[j];
        }
    }
    std::vector<char> p_side, a_side;
    pipe_place(win, prep, apply, p_side, a_side);
    double t = prep_full[0] + apply_full[T - 1];
    for (size_t j = 0; j < T; ++j) {
        t += ns[j] + EST_CHUNK_S;
        if (j + 1 < T) t += (p_side[j + 1] ? EST_SIDE_COST : 1.0) * prep_full[j + 1];
        if (j > 0) t += (a_side[j - 1] ? EST_SIDE_COST : 1.0) * apply_full[j - 1];
    }
    return t;
}

struct Interval {
    uintptr_t lo, hi;   // [lo, hi)
    int64_t param;
    int role;           // 0 weight, 1 momentum, 2 grad
};

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

const char* muon_status_string(muon_status s) {
    switch (s) {
        case MUON_OK: return "ok";
        case MUON_ERR_INVALID_ARG: return "invalid argument";
        case MUON_ERR_SHAPE: return "bad shape";
        case MUON_ERR_ALIGNMENT: return "misaligned pointer";
        case MUON_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MUON_ERR_NOT_BOUND: return "plan not bound to a workspace";
        case MUON_ERR_STALE_PLAN: return "stale plan";
        case MUON_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* muon_last_error(void) { return muon::g_last_error.c_str(); }

muon_status muon_plan_buckets(const muon_param_desc* params, int64_t n,
                              const muon_plan_opts* opts, muon_plan** out) {
    clear_error();
    if (!out) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: out is NULL");
    *out = nullptr;
    if (n < 0) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: n < 0");
    if (n > 0 && !params) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: params is NULL");
    const uint64_t cap = opts ? opts->max_workspace_bytes : 0;
    const float* scales = opts ? opts->scale : nullptr;
    const int32_t scale_mode = opts ? opts->scale_mode : MUON_SCALE_NONE;
    if (scale_mode != MUON_SCALE_NONE && scale_mode != MUON_SCALE_ASPECT && scale_mode != MUON_SCALE_RMS_MATCH)
        return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: unknown scale_mode");
    const uint32_t flags = opts ? opts->flags : 0u;
    if ((flags & ~(MUON_PLAN_TILED_SMALL | MUON_PLAN_PIPELINE | MUON_PLAN_UNFUSED_NORMALIZE | MUON_PLAN_UNGROUPED)) != 0)
        return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: unknown flag bits");

    // ---- validate every descriptor -----------------------------------------------------
    std::vector<Interval> ivs;
    for (int64_t i = 0; i < n; ++i) {
        const muon_param_desc& d = params[i];
        const std::string who = "parameter " + std::to_string(i);
        if (d.optimizer != MUON_OPT_DEFAULT && d.optimizer != MUON_OPT_ADAMW && d.optimizer != MUON_OPT_NONE)
            return set_error(MUON_ERR_INVALID_ARG, who + ": unknown optimizer");
        const int32_t role = param_role(d);
        if (role == ROLE_ADAMW) {
            if (d.rows <= 0 || d.cols <= 0)
                return set_error(MUON_ERR_SHAPE, who + ": rows and cols must be positive");
            if (d.rows > (int64_t(1) << 40) || d.cols > (int64_t(1) << 31) || d.rows * d.cols > (int64_t(1) << 40))
                return set_error(MUON_ERR_SHAPE, who + ": more than 2^40 elements");
            if (d.grad_dtype != MUON_DTYPE_F32 && d.grad_dtype != MUON_DTYPE_BF16)
                return set_error(MUON_ERR_INVALID_ARG, who + ": grad_dtype must be F32 or BF16");
            if (!d.weight || !d.momentum || !d.exp_avg_sq || !d.grad)
                return set_error(MUON_ERR_INVALID_ARG, who + ": weight, momentum, exp_avg_sq and grad must be non-NULL");
            if (!aligned16(d.weight) || !aligned16(d.momentum) || !aligned16(d.exp_avg_sq) || !aligned16(d.grad))
                return set_error(MUON_ERR_ALIGNMENT, who + ": buffers must be 16-byte aligned");
            const uint64_t elems = (uint64_t)d.rows * (uint64_t)d.cols;
            const uint64_t gsz = d.grad_dtype == MUON_DTYPE_F32 ? 4 : 2;
            ivs.push_back({(uintptr_t)d.weight, (uintptr_t)d.weight + elems * 4, i, 0});
            ivs.push_back({(uintptr_t)d.momentum, (uintptr_t)d.momentum + elems * 4, i, 1});
            ivs.push_back({(uintptr_t)d.exp_avg_sq, (uintptr_t)d.exp_avg_sq + elems * 4, i, 1});
            ivs.push_back({(uintptr_t)d.grad, (uintptr_t)d.grad + elems * gsz, i, 2});
            continue;
        }
        if (role != ROLE_MUON) continue;
        if (d.rows <= 0 || d.cols <= 0)
            return set_error(MUON_ERR_SHAPE, who + ": rows and cols must be positive");
        if (d.rows > (int64_t(1) << 31) || d.cols > (int64_t(1) << 31))
            return set_error(MUON_ERR_SHAPE, who + ": dimension above 2^31");
        if (d.grad_dtype != MUON_DTYPE_F32 && d.grad_dtype != MUON_DTYPE_BF16)
            return set_error(MUON_ERR_INVALID_ARG, who + ": grad_dtype must be F32 or BF16");
        if (!d.weight || !d.momentum || !d.grad)
            return set_error(MUON_ERR_INVALID_ARG, who + ": weight, momentum and grad must be non-NULL");
        if (!aligned16(d.weight) || !aligned16(d.momentum) || !aligned16(d.grad))
            return set_error(MUON_ERR_ALIGNMENT, who + ": buffers must be 16-byte aligned");
        if (scales && !std::isfinite(scales[i]))
            return set_error(MUON_ERR_INVALID_ARG, who + ": scale must be finite");
        const uint64_t elems = (uint64_t)d.rows * (uint64_t)d.cols;
        const uint64_t gsz = d.grad_dtype == MUON_DTYPE_F32 ? 4 : 2;
        ivs.push_back({(uintptr_t)d.weight, (uintptr_t)d.weight + elems * 4, i, 0});
        ivs.push_back({(uintptr_t)d.momentum, (uintptr_t)d.momentum + elems * 4, i, 1});
        ivs.push_back({(uintptr_t)d.grad, (uintptr_t)d.grad + elems * gsz, i, 2});
    }
    // Weights and momenta are written: none may overlap anything else.  Gradients are
    // read only and may overlap each other.
    std::sort(ivs.begin(), ivs.end(), [](const Interval& a, const Interval& b) {
        return std::tie(a.lo, a.hi) < std::tie(b.lo, b.hi);
    });
    {
        // sweep: track the written interval reaching furthest and any interval reaching furthest
        uintptr_t reach_any = 0, reach_w = 0;
        int64_t who_any = -1, who_w = -1;
        for (const Interval& iv : ivs) {
            const bool written = iv.role != 2;
            if (reach_w > iv.lo || (written && reach_any > iv.lo)) {
                const int64_t other = (reach_w > iv.lo) ? who_w : who_any;
                return set_error(MUON_ERR_INVALID_ARG,
                                 "parameters " + std::to_string(other) + " and " + std::to_string(iv.param) +
                                     ": a weight or momentum buffer overlaps another buffer");
            }
            if (iv.hi > reach_any) { reach_any = iv.hi; who_any = iv.param; }
            if (written && iv.hi > reach_w) { reach_w = iv.hi; who_w = iv.param; }
        }
    }

    muon_plan* p = new (std::nothrow) muon_plan();
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_buckets: out of host memory");
    p->params.resize((size_t)n);

    // ---- AdamW parameters: entries and fixed-size segments --------------------------------
    for (int64_t i = 0; i < n; ++i) {
        const muon_param_desc& d = params[i];
        if (param_role(d) != ROLE_ADAMW) continue;
        ParamRec& r = p->params[(size_t)i];
        r.ndim = d.ndim; r.grad_dtype = d.grad_dtype; r.rows = d.rows; r.cols = d.cols;
        r.w = d.weight; r.m = d.momentum; r.g = d.grad; r.v = d.exp_avg_sq;
        r.included = ROLE_ADAMW; r.chunk = (int32_t)p->adam.size(); r.slot = -1; r.trans = 0;
        AdamEntry e{};
        e.w = d.weight; e.m = d.momentum; e.v = d.exp_avg_sq; e.g = d.grad;
        e.numel = d.rows * d.cols; e.grad_dtype = d.grad_dtype;
        for (int64_t s0 = 0; s0 < e.numel; s0 += ADAM_SEG) p->adam_segs.push_back(AdamSeg{r.chunk, 0, s0});
        p->adam.push_back(e);
        p->adam_elements += e.numel;
    }

    // ---- bucket by canonical (m, n, grad dtype) ----------------------------------------
    std::map<std::tuple<int64_t, int64_t, int32_t>, std::vector<int64_t>> buckets;
    for (int64_t i = 0; i < n; ++i) {
        const muon_param_desc& d = params[i];
        ParamRec& r = p->params[(size_t)i];
        const int32_t role = param_role(d);
        if (role == ROLE_ADAMW) continue;
        r.ndim = d.ndim; r.grad_dtype = d.grad_dtype; r.rows = d.rows; r.cols = d.cols;
        r.w = d.weight; r.m = d.momentum; r.g = d.grad; r.v = nullptr;
        r.included = role == ROLE_MUON ? ROLE_MUON : 0; r.chunk = -1; r.slot = -1; r.trans = 0;
        if (!r.included) { p->n_excluded++; continue; }
        p->n_included++;
        r.trans = d.rows > d.cols;
        const int64_t m = std::min(d.rows, d.cols), nn = std::max(d.rows, d.cols);
        buckets[{m, nn, d.grad_dtype}].push_back(i);
    }
    p->n_buckets = (int32_t)buckets.size();

    // ---- per-bucket geometry and chunking ----------------------------------------------
    std::vector<BucketGeo> geo;
    for (auto& kv : buckets) {
        BucketGeo g;
        g.m = std::get<0>(kv.first); g.n = std::get<1>(kv.first); g.gdt = std::get<2>(kv.first);
        g.tile = pick_tile(g.m);
        g.mp = (int64_t)align_up((uint64_t)g.m, (uint64_t)g.tile);
        g.np = (int64_t)align_up((uint64_t)g.n, (uint64_t)g.tile);
        g.ew = ceil_div(g.m, EW_TILE) * ceil_div(g.n, EW_TILE);
        if ((uint64_t)g.mp * (uint64_t)g.np >= (uint64_t(1) << 31)) {
            delete p;
            return set_error(MUON_ERR_SHAPE, "padded matrix " + std::to_string(g.mp) + "x" +
                                                 std::to_string(g.np) + " exceeds 2^31 elements");
        }
        g.members = kv.second;
        geo.push_back(std::move(g));
    }
    const bool pipeline = (flags & MUON_PLAN_PIPELINE) != 0;
    if (pipeline) {
        // The two-stream step hides each chunk's neighbours' elementwise work behind the
        // chunk's products, so the buckets with little product time per element (the
        // smaller tiles) go last, after the edge chunk that ends the 256-tile buckets.
        std::stable_partition(geo.begin(), geo.end(), [](const BucketGeo& g) { return g.tile == TILE_256; });
    }

    // the start of the workspace: matrix table, AdamW entries, AdamW segments
    p->off_adam = align_up((uint64_t)p->n_included * sizeof(MatEntry), WS_ALIGN);
    p->off_adam_segs = p->off_adam + align_up((uint64_t)p->adam.size() * sizeof(AdamEntry), WS_ALIGN);
    p->table_bytes = p->off_adam_segs + align_up((uint64_t)p->adam_segs.size() * sizeof(AdamSeg), WS_ALIGN);
    uint64_t total = p->table_bytes;
    // each chunk's region adds up to 7 sub-buffer alignments
    const uint64_t chunks_per_bucket = pipeline ? (uint64_t)PIPE_MAX_CHUNKS : 1;
    for (const BucketGeo& g : geo)
        total += per_matrix_bytes(g.mp, g.np, g.ew) * (uint64_t)g.members.size() + 7 * WS_ALIGN * chunks_per_bucket;
    p->shared_regions = cap != 0 && total > cap;
    p->flags = flags;
    const bool double_buffer = p->shared_regions && pipeline;

    // chunk sizes per bucket, in plan order
    std::vector<std::vector<int64_t>> sizes(geo.size());
    std::vector<char> fused_b(geo.size(), 0);
    for (size_t bi = 0; bi < geo.size(); ++bi) {
        const BucketGeo& g = geo[bi];
        int64_t per_chunk = (int64_t)g.members.size();
        const bool fused = !(flags & MUON_PLAN_TILED_SMALL) && g.mp == 64 && g.np <= SMALL_NS_MAX_N;
        fused_b[bi] = fused;
        if (pipeline && !fused) {
            // The two-stream step hides a chunk's neighbours' elementwise work behind its
            // products, which needs several chunks per large bucket: up to PIPE_MAX_SPLIT,
            // each keeping at least PIPE_MIN_WG SYRK workgroups (the smallest product
            // launch), so that every launch still fills the chip many times over.
            const int64_t tm = g.mp / g.tile, tri = tm * (tm + 1) / 2;
            const int64_t n_min = ceil_div(PIPE_MIN_WG, tri);
            const int64_t k = std::max<int64_t>(1, std::min<int64_t>(PIPE_MAX_SPLIT, per_chunk / n_min));
            per_chunk = ceil_div(per_chunk, k);
        }
        if (p->shared_regions) {
            // one region of up to `room` bytes, or two of up to `room` each (double buffering)
            const uint64_t pm = per_matrix_bytes(g.mp, g.np, g.ew);
            const uint64_t slack = (double_buffer ? 14 : 7) * WS_ALIGN;
            uint64_t room = cap > p->table_bytes + slack ? cap - p->table_bytes - slack : 0;
            if (double_buffer) room /= 2;
            const int64_t fit = (int64_t)(room / pm);
            if (fit < 1) {
                const std::string msg = "one " + std::to_string(g.m) + "x" + std::to_string(g.n) +
                                        " matrix needs " +
                                        std::to_string((double_buffer ? 2 : 1) * pm + p->table_bytes + slack) +
                                        " bytes of workspace" + (double_buffer ? " with double buffering" : "") +
                                        "; the cap is " + std::to_string(cap);
                delete p;
                return set_error(MUON_ERR_WORKSPACE_TOO_SMALL, msg);
            }
            per_chunk = std::min(per_chunk, fit);
        }
        const int64_t total_m = (int64_t)g.members.size();
        const int64_t nchunks = ceil_div(total_m, per_chunk);
        // balanced split: chunk sizes differ by at most one
        for (int64_t c = 0; c < nchunks; ++c) sizes[bi].push_back(total_m / nchunks + (c < total_m % nchunks ? 1 : 0));
    }
    if (pipeline) {
        // Edge chunks.  In the two-stream step the first tiled chunk's momentum and
        // normaliser run before any product and the last one's apply after all of them, at
        // full speed and alone.  So a smaller chunk is split off the front of the first
        // 256-tile chunk and off the back of the last one (the same chunk when there is one),
        // each of the size that minimises the estimated step time (0: no split).
        size_t bf = geo.size(), bl = geo.size();
        for (size_t bi = 0; bi < geo.size(); ++bi)
            if (!fused_b[bi] && geo[bi].tile == TILE_256) { if (bf == geo.size()) bf = bi; bl = bi; }
        auto sequence = [&]() {
            std::vector<std::pair<const BucketGeo*, int64_t>> seq;
            for (size_t bi = 0; bi < geo.size(); ++bi)
                if (!fused_b[bi])
                    for (const int64_t c : sizes[bi]) seq.emplace_back(&geo[bi], c);
            return seq;
        };
        if (bf < geo.size()) {
            // sizes[bf] and sizes[bl] with head chunk h and tail chunk t (0: none); the same
            // bucket vector when bf == bl
            const std::vector<int64_t> first = sizes[bf], last = sizes[bl];
            auto apply = [&](int64_t h, int64_t t) {
                sizes[bf] = first;
                if (bl != bf) sizes[bl] = last;
                std::vector<int64_t>& f = sizes[bf];
                if (h > 0) { f.front() -= h; f.insert(f.begin(), h); }
                std::vector<int64_t>& l = sizes[bl];
                if (t > 0) { l.back() -= t; l.push_back(t); }
            };
            // a head h and a tail t of the same single chunk must leave at least one matrix
            const bool one = bf == bl && first.size() == 1;
            const int64_t n_head = first.front();
            auto n_tail = [&](int64_t hh) { return one ? first.back() - hh : last.back(); };
            // coordinate descent: the best head for the current tail, then the best tail for
            // that head, for a few rounds (no round raises the estimate)
            int64_t h = 0, t = 0;
            apply(0, 0);
            double best = est_pipelined_step(sequence());
            for (int round = 0; round < 3; ++round) {
                const int64_t h0 = h, t0 = t;
                for (int64_t e = 1; e < n_head - (one ? t : 0); ++e) {
                    apply(e, t);
                    const double v = est_pipelined_step(sequence());
                    if (v < best) { best = v; h = e; }
                }
                for (int64_t e = 1; e < n_tail(h); ++e) {
                    apply(h, e);
                    const double v = est_pipelined_step(sequence());
                    if (v < best) { best = v; t = e; }
                }
                if (h == h0 && t == t0) break;
            }
            apply(h, t);
        }
    }

    int32_t bucket_id = 0;
    for (size_t bi = 0; bi < geo.size(); ++bi) {
        const BucketGeo& g = geo[bi];
        const bool fused = fused_b[bi];
        int64_t start = 0;
        for (const int64_t cnt : sizes[bi]) {
            Chunk ch{};
            ch.bucket = bucket_id; ch.grad_dtype = g.gdt;
            ch.m = g.m; ch.n = g.n; ch.mp = g.mp; ch.np = g.np; ch.tile = g.tile;
            ch.fused = fused;
            ch.grouped = !fused && g.tile != TILE_256 && !(flags & MUON_PLAN_UNGROUPED);
            ch.count = cnt; ch.first = (int64_t)p->table.size(); ch.ew_tiles = g.ew;
            ch.off_table = (uint64_t)ch.first * sizeof(MatEntry);
            const int32_t cidx = (int32_t)p->chunks.size();
            for (int64_t s = 0; s < cnt; ++s) {
                const int64_t pi = g.members[(size_t)(start + s)];
                ParamRec& r = p->params[(size_t)pi];
                r.chunk = cidx; r.slot = s;
                MatEntry e{};
                e.w = r.w; e.m = r.m; e.g = r.g; e.rows = r.rows; e.cols = r.cols;
                e.trans = r.trans; e.scale = scales ? scales[pi] : rule_scale(scale_mode, r.rows, r.cols);
                p->table.push_back(e);
            }
            start += cnt;
            p->chunks.push_back(ch);
        }
        bucket_id++;
    }

    // ---- workspace layout ---------------------------------------------------------------
    // With shared regions the grouped small chunks (orthogonalised together) sit back to
    // back in one region; if they do not fit in one under the cap, each runs on its own.
    if (p->shared_regions) {
        const uint64_t slack = (double_buffer ? 14 : 7) * WS_ALIGN;
        uint64_t room = cap > p->table_bytes + slack ? cap - p->table_bytes - slack : 0;
        if (double_buffer) room /= 2;
        uint64_t group = 0;
        for (Chunk& c : p->chunks)
            if (c.grouped) {
                layout_region(c, 0);
                group += c.region_bytes;
            }
        if (group > room)
            for (Chunk& c : p->chunks) c.grouped = false;
    }
    // lays the grouped chunks out back to back from `base`; returns the bytes they take
    auto layout_group = [&](uint64_t base) {
        uint64_t o = base;
        for (Chunk& c : p->chunks)
            if (c.grouped) {
                layout_region(c, o);
                c.region_base = base;
                o = c.region_off + c.region_bytes;
            }
        return o - base;
    };
    uint64_t off = p->table_bytes, shared_max = 0;
    for (Chunk& c : p->chunks) {
        if (c.grouped && p->shared_regions) continue;
        if (p->shared_regions) {
            layout_region(c, p->table_bytes);
            shared_max = std::max(shared_max, c.region_bytes);
        } else {
            layout_region(c, off);
            off = c.region_off + c.region_bytes;
        }
    }
    if (p->shared_regions) shared_max = std::max(shared_max, layout_group(p->table_bytes));
    bool second = false;
    if (double_buffer) {
        // the tiled chunks alternate between two regions (the fused small-matrix chunks,
        // which the two-stream step runs one at a time first, stay in the first), so that
        // consecutive tiled chunks never share one; the grouped chunks count as one
        int64_t k = 0;
        bool group_seen = false;
        for (Chunk& c : p->chunks) {
            if (c.fused) continue;
            if (c.grouped) {
                if (group_seen) continue;
                group_seen = true;
                if (k++ & 1) {
                    layout_group(p->table_bytes + shared_max);
                    second = true;
                }
                continue;
            }
            if (k++ & 1) {
                layout_region(c, p->table_bytes + shared_max);
                second = true;
            }
        }
    }
    p->ws_bytes = p->shared_regions ? p->table_bytes + shared_max * (second ? 2 : 1) : off;
    if (p->ws_bytes == 0) p->ws_bytes = WS_ALIGN;
    *out = p;
    return MUON_OK;
}

muon_status muon_plan_workspace_bytes(const muon_plan* plan, uint64_t* bytes) {
    if (!plan || !bytes) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_workspace_bytes: NULL argument");
    *bytes = plan->ws_bytes;
    return MUON_OK;
}

muon_status muon_plan_counts(const muon_plan* plan, int32_t* n_chunks, int32_t* n_buckets,
                             int64_t* n_included, int64_t* n_excluded) {
    if (!plan) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_counts: plan is NULL");
    if (n_chunks) *n_chunks = (int32_t)plan->chunks.size();
    if (n_buckets) *n_buckets = plan->n_buckets;
    if (n_included) *n_included = plan->n_included;
    if (n_excluded) *n_excluded = plan->n_excluded;
    return MUON_OK;
}

muon_status muon_plan_adamw_counts(const muon_plan* plan, int64_t* n_params, int64_t* n_elements) {
    if (!plan) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_adamw_counts: plan is NULL");
    if (n_params) *n_params = (int64_t)plan->adam.size();
    if (n_elements) *n_elements = plan->adam_elements;
    return MUON_OK;
}

muon_status muon_plan_info(const muon_plan* plan, int32_t chunk, muon_chunk_info* out) {
    if (!plan || !out) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_info: NULL argument");
    if (chunk < 0 || chunk >= (int32_t)plan->chunks.size())
        return set_error(MUON_ERR_INVALID_ARG, "muon_plan_info: chunk out of range");
    const Chunk& c = plan->chunks[(size_t)chunk];
    std::memset(out, 0, sizeof(*out));
    out->m = c.m; out->n = c.n; out->m_pad = c.mp; out->n_pad = c.np; out->count = c.count;
    out->bucket = c.bucket; out->tile = c.tile; out->grad_dtype = c.grad_dtype;
    out->shared_region = plan->shared_regions ? 1 : 0;
    out->fused_small = c.fused ? 1 : 0;
    out->grouped_small = c.grouped ? 1 : 0;
    const double m = (double)c.m, n = (double)c.n, k = (double)c.count;
    out->flops_conventional = k * (4.0 * m * m * n + 2.0 * m * m * m);
    out->flops_algorithmic = k * (m * (m + 1.0) * n + m * m * (m + 1.0) + 2.0 * m * m * n);
    const double gsz = c.grad_dtype == MUON_DTYPE_F32 ? 4.0 : 2.0;
    // momentum: read M and G, write M and X0 (bf16); apply: read W and O (bf16), write W
    out->bytes_momentum = k * m * n * (4.0 + gsz + 4.0 + 2.0);
    out->bytes_apply = k * m * n * (4.0 + 2.0 + 4.0);
    out->region_offset = c.region_off;
    out->region_bytes = c.region_bytes;
    return MUON_OK;
}

muon_status muon_plan_param_info(const muon_plan* plan, int64_t param, muon_param_info* out) {
    if (!plan || !out) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_param_info: NULL argument");
    if (param < 0 || param >= (int64_t)plan->params.size())
        return set_error(MUON_ERR_INVALID_ARG, "muon_plan_param_info: parameter index out of range");
    std::memset(out, 0, sizeof(*out));
    const ParamRec& r = plan->params[(size_t)param];
    if (!r.included) return MUON_OK;
    if (r.included == ROLE_ADAMW) {
        out->included = ROLE_ADAMW;
        return MUON_OK;
    }
    const Chunk& c = plan->chunks[(size_t)r.chunk];
    out->included = 1;
    out->chunk = r.chunk;
    out->slot = r.slot;
    out->transposed = r.trans;
    out->scale = plan->table[(size_t)(c.first + r.slot)].scale;
    out->output_offset = c.off_xp + (uint64_t)r.slot * c.mp * c.np * 2ull;
    out->ld = c.np;
    return MUON_OK;
}

muon_status muon_plan_validate(const muon_plan* plan, const muon_param_desc* params, int64_t n) {
    if (!plan) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_validate: plan is NULL");
    if (n != (int64_t)plan->params.size() || (n > 0 && !params))
        return set_error(MUON_ERR_STALE_PLAN, "parameter count differs from the plan's");
    for (int64_t i = 0; i < n; ++i) {
        const muon_param_desc& d = params[i];
        const ParamRec& r = plan->params[(size_t)i];
        const int32_t role = param_role(d);
        if ((role == ROLE_NONE ? 0 : role) != r.included)
            return set_error(MUON_ERR_STALE_PLAN, "parameter " + std::to_string(i) + ": optimizer changed");
        if (role == ROLE_NONE) continue;
        if (d.ndim != r.ndim) return set_error(MUON_ERR_STALE_PLAN, "parameter " + std::to_string(i) + ": ndim changed");
        if (d.rows != r.rows || d.cols != r.cols || d.grad_dtype != r.grad_dtype || d.weight != r.w ||
            d.momentum != r.m || d.grad != r.g || (role == ROLE_ADAMW && d.exp_avg_sq != r.v))
            return set_error(MUON_ERR_STALE_PLAN, "parameter " + std::to_string(i) + ": shape, dtype or buffer changed");
    }
    return MUON_OK;
}

}  // extern "C"

// The launch layer owns device-side state of a plan (timing events); it provides this
// hook.  A host-only build of the planner links without it.
extern "C" __attribute__((weak)) void muon_internal_release(muon_plan* plan);

extern "C" void muon_plan_destroy(muon_plan* plan) {
    if (!plan) return;
    if (muon_internal_release) muon_internal_release(plan);
    delete plan;
}
