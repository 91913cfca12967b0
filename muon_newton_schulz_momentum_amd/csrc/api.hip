// Device-side entry points of libmuon: bind, the three step calls, and kernel timing.
// Argument checks happen here, on the host, before anything is launched; a kernel is
// only launched with shapes the planner has laid out in the workspace.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "plan_internal.h"

using namespace muon;

namespace {

muon_status hip_fail(hipError_t e, const char* what) {
    return set_error(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <class T>
T* at(const muon_plan* p, uint64_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(p->ws) + off);
}

muon_status check_step(const muon_plan* p, int32_t chunk, const char* who) {
    if (!p) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": plan is NULL");
    if (!p->bound) return set_error(MUON_ERR_NOT_BOUND, std::string(who) + ": call muon_plan_bind first");
    if (chunk < -1 || chunk >= (int32_t)p->chunks.size())
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": chunk out of range");
    if (chunk == -1 && p->shared_regions && p->chunks.size() > 1)
        return set_error(MUON_ERR_INVALID_ARG,
                         std::string(who) + ": the chunks share one workspace region; "
                                            "step them one at a time (or use muon_step)");
    return MUON_OK;
}

// X0 bookkeeping (muon_plan::x0_fresh): a Newton–Schulz call consumes the chunk's X0, and
// a momentum update of a chunk overwrites the X0 of every other chunk in its region.
void mark_x0(const muon_plan* p, int32_t chunk, bool fresh) {
    std::vector<uint8_t>& f = const_cast<muon_plan*>(p)->x0_fresh;
    const int32_t n = (int32_t)f.size();
    for (int32_t i = 0; i < n; ++i) {
        if (chunk != -1 && i != chunk) continue;
        if (fresh)
            for (int32_t k = 0; k < n; ++k) {
                const Chunk& a = p->chunks[(size_t)k];
                const Chunk& b = p->chunks[(size_t)i];
                if (a.region_off < b.region_off + b.region_bytes && b.region_off < a.region_off + a.region_bytes)
                    f[(size_t)k] = 0;
            }
        f[(size_t)i] = fresh ? 1 : 0;
    }
}
muon_status check_x0(const muon_plan* p, int32_t chunk, const char* who) {
    for (int32_t i = 0; i < (int32_t)p->x0_fresh.size(); ++i)
        if ((chunk == -1 || i == chunk) && !p->x0_fresh[(size_t)i])
            return set_error(MUON_ERR_INVALID_ARG,
                             std::string(who) + ": chunk " + std::to_string(i) +
                                 " holds no fresh X0 (bf16 momentum): an earlier Newton-Schulz call or step has "
                                 "consumed it, or none was made; call muon_momentum_update first");
    return MUON_OK;
}

// ---- per-launch timing ------------------------------------------------------------------

// Set while this thread records a step into a graph: launches then carry no event pairs,
// since an event recorded inside a graph would be overwritten by every replay.
thread_local bool t_capturing = false;

struct TimedLaunch {
    muon_plan* p;
    int slot = -1;
    TimedLaunch(const muon_plan* plan, int32_t kind, double work, hipStream_t s)
        : p(const_cast<muon_plan*>(plan)) {
        TimingState& t = p->timing;
        if (t_capturing || t.used >= t.capacity) return;
        slot = t.used++;
        t.kind[slot] = kind;
        t.work[slot] = work;
        (void)hipEventRecord((hipEvent_t)t.ev_begin[slot], s);
    }
    void done(hipStream_t s) {
        if (slot >= 0) (void)hipEventRecord((hipEvent_t)p->timing.ev_end[slot], s);
    }
};

// ---- one step's settings ----------------------------------------------------------------

struct StepCfg {
    float beta = 0.f, lr = 0.f, wd = 0.f, eps = 0.f;
    int32_t steps = 0;
    std::vector<float> abc;          // (a, b, c) of each iteration, 3 * steps values
    bool nesterov = false;
    const float* dev = nullptr;      // device {beta, lr, wd}, read by the kernels when set
    bool adam = false;               // also run AdamW with `adam_args`
    AdamArgs adam_args{};
    bool pipeline = false;           // the two-stream order (step_pipelined)
};

// AdamW launch arguments from the public config (validated); tables filled in at launch.
muon_status make_adam(const muon_adamw_config* c, AdamArgs& a, const char* who) {
    if (!c) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": AdamW config is NULL");
    if (c->step < 1) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": AdamW step must be >= 1");
    if (!std::isfinite(c->lr) || !std::isfinite(c->wd) || !std::isfinite(c->eps) || c->eps < 0.f ||
        !std::isfinite(c->beta1) || !std::isfinite(c->beta2) || c->beta1 < 0.f || c->beta1 >= 1.f ||
        c->beta2 < 0.f || c->beta2 >= 1.f)
        return set_error(MUON_ERR_INVALID_ARG,
                         std::string(who) + ": AdamW lr, wd finite, eps >= 0, betas in [0, 1)");
    if (c->dev_scalars && ((uintptr_t)c->dev_scalars & 3u) != 0)
        return set_error(MUON_ERR_ALIGNMENT, std::string(who) + ": AdamW dev_scalars must be 4-byte aligned");
    a.lr = (double)c->lr;
    a.wd = (double)c->wd;
    a.beta1 = (double)c->beta1;
    a.omb1 = (double)(1.0f - c->beta1);
    a.beta2 = (double)c->beta2;
    a.omb2 = (double)(1.0f - c->beta2);
    a.eps = (double)c->eps;
    // bias corrections 1 - beta^t in float64 (pow of the float32 beta, widened)
    a.bc1 = 1.0 - std::pow((double)c->beta1, (double)c->step);
    a.bc2 = 1.0 - std::pow((double)c->beta2, (double)c->step);
    a.dev_scalars = c->dev_scalars;
    return MUON_OK;
}

muon_status adam_run(const muon_plan* p, AdamArgs a, hipStream_t s) {
    if (p->adam_segs.empty()) return MUON_OK;
    a.entries = at<const AdamEntry>(p, p->off_adam);
    a.segs = at<const AdamSeg>(p, p->off_adam_segs);
    a.n_segs = (int64_t)p->adam_segs.size();
    double work = 0.0;
    for (const AdamEntry& e : p->adam) work += (double)e.numel * (e.grad_dtype == MUON_DTYPE_F32 ? 28.0 : 26.0);
    TimedLaunch tl(p, MUON_KERNEL_ADAMW, work, s);
    const hipError_t e = launch_adamw(a, s);
    tl.done(s);
    return e == hipSuccess ? MUON_OK : hip_fail(e, "AdamW kernel launch");
}

void fill_abc(StepCfg& cfg, float a, float b, float c) {
    cfg.abc.resize(3 * (size_t)cfg.steps);
    for (int32_t t = 0; t < cfg.steps; ++t) {
        cfg.abc[3 * (size_t)t] = a;
        cfg.abc[3 * (size_t)t + 1] = b;
        cfg.abc[3 * (size_t)t + 2] = c;
    }
}

bool finite(float v) { return std::isfinite(v); }

constexpr int32_t MAX_NS_STEPS = 1024;

muon_status check_ns(int32_t steps, const float* abc, float eps, const char* who) {
    if (steps < 1 || steps > MAX_NS_STEPS)
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": steps must be in [1, 1024]");
    if (!finite(eps) || eps < 0.f) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": eps must be finite and >= 0");
    for (int32_t i = 0; i < 3 * steps; ++i)
        if (!finite(abc[i])) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": coefficients must be finite");
    return MUON_OK;
}

// ---- the three steps for one chunk --------------------------------------------------------

// Chunks whose matrices have fewer than 2^30 elements may use the side-stream kernels
// (their byte offsets are 32-bit).
bool side_ok(const Chunk& c) { return c.m * c.n < (int64_t(1) << 30); }

muon_status momentum_chunk(const muon_plan* p, const Chunk& c, const StepCfg& cfg, hipStream_t s,
                           bool side = false) {
    MomentumArgs a;
    a.tbl = at<const MatEntry>(p, c.off_table);
    a.xq = at<uint16_t>(p, c.off_xq);
    a.partials = at<double>(p, c.off_part);
    a.mat_stride = c.mp * c.np;
    a.np = c.np;
    a.ew_tiles = c.ew_tiles;
    a.total_tiles = c.count * c.ew_tiles;
    a.beta = cfg.beta;
    a.omb = 1.0f - cfg.beta;
    a.dev_scalars = cfg.dev;
    a.nesterov = cfg.nesterov ? 1 : 0;
    const double gsz = c.grad_dtype == MUON_DTYPE_F32 ? 4.0 : 2.0;
    const bool sk = side && side_ok(c);
    TimedLaunch tl(p, sk ? MUON_KERNEL_MOMENTUM_SIDE : MUON_KERNEL_MOMENTUM, (double)c.count * c.m * c.n * (10.0 + gsz), s);
    const hipError_t e = sk ? launch_momentum_side(a, c.grad_dtype, s) : launch_momentum(a, c.grad_dtype, s);
    tl.done(s);
    return e == hipSuccess ? MUON_OK : hip_fail(e, "momentum kernel launch");
}

// The X buffer the iteration starts in.  It ping-pongs between the two X buffers and must
// end in xp, where the apply step reads O: start in xq (normalised in place) for an odd
// step count.
uint16_t* ns_start(const muon_plan* p, const Chunk& c, int32_t steps) {
    return (steps & 1) ? at<uint16_t>(p, c.off_xq) : at<uint16_t>(p, c.off_xp);
}

// Whether the chunk's normalisation is fused into the first iteration's operand loads:
// the 256-tile kernels with an odd iteration count (X0 is then read where the first
// iteration starts, in xq, and the last iteration ends in xp as the apply expects).
bool fused_norm(const muon_plan* p, const Chunk& c, int32_t steps) {
    return c.tile == TILE_256 && (steps & 1) && !(p->flags & MUON_PLAN_UNFUSED_NORMALIZE);
}

// Step 2 for a chunk: the normaliser from the momentum kernel's partial sums, then
// X = bf16(X0 / (||X0|| + eps)) into the starting buffer (unless the first iteration's
// loads do that themselves).
muon_status ns_prep(const muon_plan* p, const Chunk& c, int32_t steps, float eps, hipStream_t s, bool side = false) {
    uint16_t* xq = at<uint16_t>(p, c.off_xq);
    double* inv = at<double>(p, c.off_inv);
    hipError_t e;
    {
        const bool fused = fused_norm(p, c, steps);
        FinalizeArgs f{at<const double>(p, c.off_part), inv, c.ew_tiles, (double)eps, at<uint32_t>(p, c.off_sched),
                       fused && (c.mp != c.m || c.np != c.n) ? xq : nullptr, c.m, c.n, c.mp, c.np};
        TimedLaunch tl(p, MUON_KERNEL_NORM_FINALIZE, (double)c.count * c.ew_tiles * 8.0, s);
        e = launch_finalize(f, c.count, s);
        tl.done(s);
        if (e != hipSuccess) return hip_fail(e, "norm finalize kernel launch");
    }
    if (fused_norm(p, c, steps)) return MUON_OK;
    {
        NormalizeArgs n{xq, ns_start(p, c, steps), inv, c.m, c.n, c.mp, c.np, c.count * c.mp * c.np / 8};
        TimedLaunch tl(p, side ? MUON_KERNEL_NORMALIZE_SIDE : MUON_KERNEL_NORMALIZE, (double)c.count * c.m * c.n * 4.0, s);
        e = side ? launch_normalize_side(n, s) : launch_normalize(n, s);
        tl.done(s);
        if (e != hipSuccess) return hip_fail(e, "normalize kernel launch");
    }
    return MUON_OK;
}

// The arguments of one product launch over chunk c, X read from `cur`, X' written to `nxt`
// (the same for the chunk's own launches and for the grouped ones).  `norm`: the first
// iteration of a fused_norm chunk.
NsArgs ns_args(const muon_plan* p, const Chunk& c, NsMode mode, uint16_t* cur, uint16_t* nxt, float alpha,
               float gamma, bool norm) {
    uint16_t* am = at<uint16_t>(p, c.off_a);
    uint16_t* bm = at<uint16_t>(p, c.off_b);
    const int32_t tm = (int32_t)(c.mp / c.tile), tn = (int32_t)(c.np / c.tile);
    const int32_t tri = tm * (tm + 1) / 2;
    const int64_t xs = c.mp * c.np, as = c.mp * c.mp;
    NsArgs g{};
    g.sched = at<uint32_t>(p, c.off_sched);
    g.alpha = alpha;
    g.gamma = gamma;
    if (mode == NS_SYRK) {              // A = X X^T
        g.opa = cur; g.opb = cur; g.ep = cur; g.out = am;
        g.stride_a = xs; g.stride_b = xs; g.stride_o = as;
        g.lda = (int32_t)c.np; g.ldb = (int32_t)c.np; g.ldo = (int32_t)c.mp;
        g.K = (int32_t)c.np; g.tiles_m = tm; g.tiles_n = tm; g.tiles_per_mat = tri;
        g.total_tiles = (int32_t)(c.count * tri);
        g.inv = norm ? at<const double>(p, c.off_inv) : nullptr;
    } else if (mode == NS_POLY) {       // B = b A + c A A^T (B is computed from A only)
        g.opa = am; g.opb = am; g.ep = am; g.out = bm;
        g.stride_a = as; g.stride_b = as; g.stride_o = as;
        g.lda = (int32_t)c.mp; g.ldb = (int32_t)c.mp; g.ldo = (int32_t)c.mp;
        g.K = (int32_t)c.mp; g.tiles_m = tm; g.tiles_n = tm; g.tiles_per_mat = tri;
        g.total_tiles = (int32_t)(c.count * tri);
    } else {                            // X' = a X + B X
        g.opa = bm; g.opb = cur; g.ep = cur; g.out = nxt;
        g.stride_a = as; g.stride_b = xs; g.stride_o = xs;
        g.lda = (int32_t)c.mp; g.ldb = (int32_t)c.np; g.ldo = (int32_t)c.np;
        g.K = (int32_t)c.mp; g.tiles_m = tm; g.tiles_n = tn; g.tiles_per_mat = tm * tn;
        g.total_tiles = (int32_t)(c.count * tm * tn);
        g.inv = norm ? at<const double>(p, c.off_inv) : nullptr;
    }
    return g;
}

// Algorithmic FLOPs of one product launch over chunk c.
double mode_flops(const Chunk& c, NsMode mode) {
    const double m = (double)c.m, n = (double)c.n, cnt = (double)c.count;
    return mode == NS_SYRK ? cnt * m * (m + 1.0) * n : mode == NS_POLY ? cnt * m * m * (m + 1.0) : cnt * 2.0 * m * m * n;
}

const char* mode_name(NsMode mode) {
    return mode == NS_SYRK ? "SYRK kernel launch" : mode == NS_POLY ? "SYRK+poly kernel launch" : "GEMM+axpy kernel launch";
}

// Step 3 for a chunk: the iterations, from the normalised X.
muon_status ns_iterate(const muon_plan* p, const Chunk& c, const float* abc, int32_t steps, hipStream_t s) {
    uint16_t* xp = at<uint16_t>(p, c.off_xp);
    uint16_t* xq = at<uint16_t>(p, c.off_xq);
    uint16_t* cur = ns_start(p, c, steps);
    static const int32_t kinds[3] = {MUON_KERNEL_SYRK, MUON_KERNEL_SYRK_POLY, MUON_KERNEL_GEMM_AXPY};
    for (int32_t it = 0; it < steps; ++it) {
        const float a_ = abc[3 * it], b_ = abc[3 * it + 1], c_ = abc[3 * it + 2];
        uint16_t* nxt = (cur == xp) ? xq : xp;
        // the first iteration normalises X0 as it loads it (fused_norm)
        const bool norm = it == 0 && fused_norm(p, c, steps);
        const float alpha[3] = {0.f, b_, a_}, gamma[3] = {1.f, c_, 1.f};
        for (int32_t k = 0; k < 3; ++k) {
            const NsMode mode = (NsMode)k;
            NsArgs g = ns_args(p, c, mode, cur, nxt, alpha[k], gamma[k], norm);
            // Consecutive launches sweep the chunk's matrices in alternate directions (the
            // first one against the momentum pass before it), so that each starts on the
            // matrices whose data the previous launch touched last and the device caches
            // still hold.  Results do not depend on the order.
            g.reverse = (3 * it + k) % 2 == 0;
            TimedLaunch tl(p, kinds[k], mode_flops(c, mode), s);
            const hipError_t e = launch_ns(mode, c.tile, g, s);
            tl.done(s);
            if (e != hipSuccess) return hip_fail(e, mode_name(mode));
        }
        cur = nxt;
    }
    return MUON_OK;
}

// ---- the grouped small tiled chunks ----------------------------------------------------------

std::vector<int32_t> grouped_chunks(const muon_plan* p) {
    std::vector<int32_t> g;
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i)
        if (p->chunks[(size_t)i].grouped) g.push_back(i);
    return g;
}

// Step 2 for grouped chunks: one launch (per PREP_MAX_JOBS chunks) computes every matrix's
// normaliser and normalises it into its starting buffer.
muon_status prep_group(const muon_plan* p, const std::vector<int32_t>& idx, int32_t steps, float eps,
                       hipStream_t s) {
    for (size_t g0 = 0; g0 < idx.size(); g0 += PREP_MAX_JOBS) {
        PrepGroupArgs A{};
        A.eps = (double)eps;
        double bytes = 0.0;
        for (size_t k = g0; k < idx.size() && k < g0 + PREP_MAX_JOBS; ++k) {
            const Chunk& c = p->chunks[(size_t)idx[k]];
            PrepJob& J = A.job[A.n_jobs++];
            J.partials = at<const double>(p, c.off_part);
            J.src = at<const uint16_t>(p, c.off_xq);
            J.dst = ns_start(p, c, steps);
            J.ew_tiles = c.ew_tiles;
            J.m = c.m; J.n = c.n; J.mp = c.mp; J.np = c.np;
            J.blocks = ceil_div(c.mp * c.np / 8, 4096);
            J.first = A.total_blocks;
            A.total_blocks += c.count * J.blocks;
            bytes += (double)c.count * ((double)c.m * c.n * 4.0 + (double)c.ew_tiles * 8.0);
        }
        TimedLaunch tl(p, MUON_KERNEL_PREP_GROUPED, bytes, s);
        const hipError_t e = launch_prep_grouped(A, s);
        tl.done(s);
        if (e != hipSuccess) return hip_fail(e, "grouped normalisation kernel launch");
    }
    return MUON_OK;
}

// Step 3 for grouped chunks: per iteration one launch per product (per GROUPED_MAX_JOBS
// chunks) over a single queue of all their tiles.
muon_status iterate_group(const muon_plan* p, const std::vector<int32_t>& idx, const float* abc, int32_t steps,
                          hipStream_t s) {
    std::vector<uint16_t*> cur(idx.size());
    for (size_t k = 0; k < idx.size(); ++k) cur[k] = ns_start(p, p->chunks[(size_t)idx[k]], steps);
    for (int32_t it = 0; it < steps; ++it) {
        const float a_ = abc[3 * it], b_ = abc[3 * it + 1], c_ = abc[3 * it + 2];
        const float alpha[3] = {0.f, b_, a_}, gamma[3] = {1.f, c_, 1.f};
        for (int32_t kk = 0; kk < 3; ++kk) {
            const NsMode mode = (NsMode)kk;
            for (size_t g0 = 0; g0 < idx.size(); g0 += GROUPED_MAX_JOBS) {
                GroupedNsArgs G{};
                double work = 0.0;
                for (size_t k = g0; k < idx.size() && k < g0 + GROUPED_MAX_JOBS; ++k) {
                    const Chunk& c = p->chunks[(size_t)idx[k]];
                    uint16_t* nxt = cur[k] == at<uint16_t>(p, c.off_xp) ? at<uint16_t>(p, c.off_xq) : at<uint16_t>(p, c.off_xp);
                    GroupedJob& J = G.job[G.n_jobs++];
                    J.a = ns_args(p, c, mode, cur[k], nxt, alpha[kk], gamma[kk], false);
                    J.tile = c.tile;
                    J.first = G.total_tiles;
                    G.total_tiles += J.a.total_tiles;
                    work += mode_flops(c, mode);
                }
                TimedLaunch tl(p, MUON_KERNEL_NS_GROUPED, work, s);
                const hipError_t e = launch_ns_grouped(mode, G, s);
                tl.done(s);
                if (e != hipSuccess) return hip_fail(e, "grouped product kernel launch");
            }
        }
        for (size_t k = 0; k < idx.size(); ++k) {
            const Chunk& c = p->chunks[(size_t)idx[k]];
            cur[k] = cur[k] == at<uint16_t>(p, c.off_xp) ? at<uint16_t>(p, c.off_xq) : at<uint16_t>(p, c.off_xp);
        }
    }
    return MUON_OK;
}

muon_status ns_group(const muon_plan* p, const std::vector<int32_t>& idx, const float* abc, int32_t steps, float eps,
                     hipStream_t s) {
    if (idx.empty()) return MUON_OK;
    const muon_status st = prep_group(p, idx, steps, eps, s);
    return st != MUON_OK ? st : iterate_group(p, idx, abc, steps, s);
}

muon_status ns_chunk(const muon_plan* p, const Chunk& c, const float* abc, int32_t steps, float eps,
                     hipStream_t s) {
    const muon_status st = ns_prep(p, c, steps, eps, s);
    return st != MUON_OK ? st : ns_iterate(p, c, abc, steps, s);
}

double ns_iter_flops(const Chunk& c) { return muon::ns_iter_flops(c.count, c.m, c.n); }

// The fused small-matrix kernel over the given chunks (all with Chunk::fused), in
// launches of up to SMALL_NS_MAX_JOBS chunks: normaliser, normalisation and every
// iteration in one launch.  A schedule longer than the kernel's coefficient table goes
// through the tiled kernels instead (bitwise the same result).
muon_status ns_small_chunks(const muon_plan* p, const std::vector<int32_t>& idx, const float* abc, int32_t steps,
                            float eps, hipStream_t s) {
    if (steps > SMALL_NS_MAX_STEPS) {
        for (int32_t i : idx) {
            const muon_status st = ns_chunk(p, p->chunks[(size_t)i], abc, steps, eps, s);
            if (st != MUON_OK) return st;
        }
        return MUON_OK;
    }
    for (size_t g0 = 0; g0 < idx.size(); g0 += SMALL_NS_MAX_JOBS) {
        SmallNsArgs A{};
        int64_t total = 0;
        double work = 0.0;
        for (size_t k = g0; k < idx.size() && k < g0 + SMALL_NS_MAX_JOBS; ++k) {
            const Chunk& ch = p->chunks[(size_t)idx[k]];
            SmallJob& J = A.job[A.n_jobs++];
            J.xq = at<const uint16_t>(p, ch.off_xq);
            J.xp = at<uint16_t>(p, ch.off_xp);
            J.partials = at<const double>(p, ch.off_part);
            J.ew_tiles = ch.ew_tiles;
            J.m = (int32_t)ch.m;
            J.n = (int32_t)ch.n;
            J.np = (int32_t)ch.np;
            J.first = (int32_t)total;
            total += ch.count;
            work += steps * ns_iter_flops(ch);
        }
        A.steps = steps;
        for (int32_t t = 0; t < steps; ++t)
            for (int32_t q = 0; q < 3; ++q) A.abc[t][q] = abc[3 * t + q];
        A.eps = (double)eps;
        TimedLaunch tl(p, MUON_KERNEL_NS_SMALL, work, s);
        const hipError_t e = launch_ns_small(A, total, s);
        tl.done(s);
        if (e != hipSuccess) return hip_fail(e, "fused small-matrix NS kernel launch");
    }
    return MUON_OK;
}

// Newton–Schulz for one chunk, by whichever path the plan chose for it.
muon_status ns_one(const muon_plan* p, int32_t i, const float* abc, int32_t steps, float eps, hipStream_t s) {
    const Chunk& ch = p->chunks[(size_t)i];
    if (ch.fused) return ns_small_chunks(p, std::vector<int32_t>{i}, abc, steps, eps, s);
    if (ch.grouped) return ns_group(p, std::vector<int32_t>{i}, abc, steps, eps, s);
    return ns_chunk(p, ch, abc, steps, eps, s);
}

// Newton–Schulz for every chunk (their regions are distinct): all fused chunks in grouped
// launches, all small tiled chunks in the grouped product launches, then the rest.
muon_status ns_all(const muon_plan* p, const float* abc, int32_t steps, float eps, hipStream_t s) {
    std::vector<int32_t> small;
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i)
        if (p->chunks[(size_t)i].fused) small.push_back(i);
    muon_status st = ns_small_chunks(p, small, abc, steps, eps, s);
    if (st != MUON_OK) return st;
    if ((st = ns_group(p, grouped_chunks(p), abc, steps, eps, s)) != MUON_OK) return st;
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i) {
        const Chunk& ch = p->chunks[(size_t)i];
        if (!ch.fused && !ch.grouped && (st = ns_chunk(p, ch, abc, steps, eps, s)) != MUON_OK) return st;
    }
    return MUON_OK;
}

muon_status apply_chunk(const muon_plan* p, const Chunk& c, const StepCfg& cfg, hipStream_t s,
                        bool side = false) {
    ApplyArgs a;
    a.tbl = at<const MatEntry>(p, c.off_table);
    a.xo = at<const uint16_t>(p, c.off_xp);
    a.mat_stride = c.mp * c.np;
    a.np = c.np;
    a.ew_tiles = c.ew_tiles;
    a.total_tiles = c.count * c.ew_tiles;
    const double lw = (double)cfg.lr * (double)cfg.wd;   // exact
    a.d = 1.0 - lw;                                       // one float64 rounding
    a.lr = cfg.lr;
    a.dev_scalars = cfg.dev;
    const bool sk = side && side_ok(c);
    TimedLaunch tl(p, sk ? MUON_KERNEL_APPLY_SIDE : MUON_KERNEL_APPLY, (double)c.count * c.m * c.n * 10.0, s);
    const hipError_t e = sk ? launch_apply_side(a, s) : launch_apply(a, s);
    tl.done(s);
    return e == hipSuccess ? MUON_OK : hip_fail(e, "apply kernel launch");
}

hipError_t record(const muon_plan* p, size_t k, hipStream_t s) {
    return hipEventRecord((hipEvent_t)p->pipe_events[k], s);
}
hipError_t wait(const muon_plan* p, size_t k, hipStream_t s) {
    return hipStreamWaitEvent(s, (hipEvent_t)p->pipe_events[k], 0);
}

// A unit of the two-stream step: one tiled chunk, or every grouped small chunk together.
using Unit = std::vector<int32_t>;

bool same_region(const muon_plan* p, const Unit& a, const Unit& b) {
    for (int32_t i : a)
        for (int32_t k : b)
            if (p->chunks[(size_t)i].region_base == p->chunks[(size_t)k].region_base) return true;
    return false;
}

// The tiled units, in plan order (the group where its first chunk is), when the two-stream
// pipeline can run them: at least two, and no two consecutive ones in the same workspace
// region.  Empty otherwise.
std::vector<Unit> pipeline_units(const muon_plan* p) {
    std::vector<Unit> t;
    bool group_done = false;
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i) {
        const Chunk& c = p->chunks[(size_t)i];
        if (c.fused) continue;
        if (c.grouped) {
            if (!group_done) t.push_back(grouped_chunks(p));
            group_done = true;
            continue;
        }
        t.push_back(Unit{i});
    }
    if (t.size() < 2 || !p->side || p->pipe_events.size() < 1 + 4 * t.size()) return {};
    for (size_t j = 1; j < t.size(); ++j)
        if (same_region(p, t[j], t[j - 1])) return {};
    return t;
}

// Side-stream placement estimates (the constants and their bias are with the planner's).
double est_ns_s(const Chunk& c, int32_t steps) { return steps * ns_iter_flops(c) / est_ns_rate(c.m); }
double est_prep_s(const Chunk& c) {         // momentum + normalise bytes, side kernels
    return (double)c.count * c.m * c.n * prep_bytes_per_elem(c.grad_dtype) / EST_SIDE_BW;
}
double est_apply_s(const Chunk& c) { return (double)c.count * c.m * c.n * APPLY_BYTES_PER_ELEM / EST_SIDE_BW; }

// A unit's steps: momentum of each chunk; the normalisation (grouped: one launch); the
// iterations (grouped: the grouped launches); the apply of each chunk.
muon_status unit_momentum(const muon_plan* p, const Unit& u, const StepCfg& cfg, hipStream_t s, bool side) {
    for (int32_t i : u) {
        const muon_status st = momentum_chunk(p, p->chunks[(size_t)i], cfg, s, side);
        if (st != MUON_OK) return st;
    }
    return MUON_OK;
}
muon_status unit_prep(const muon_plan* p, const Unit& u, const StepCfg& cfg, hipStream_t s, bool side) {
    if (p->chunks[(size_t)u[0]].grouped) return prep_group(p, u, cfg.steps, cfg.eps, s);
    return ns_prep(p, p->chunks[(size_t)u[0]], cfg.steps, cfg.eps, s, side);
}
muon_status unit_iterate(const muon_plan* p, const Unit& u, const StepCfg& cfg, hipStream_t s) {
    if (p->chunks[(size_t)u[0]].grouped) return iterate_group(p, u, cfg.abc.data(), cfg.steps, s);
    return ns_iterate(p, p->chunks[(size_t)u[0]], cfg.abc.data(), cfg.steps, s);
}
muon_status unit_apply(const muon_plan* p, const Unit& u, const StepCfg& cfg, hipStream_t s, bool side) {
    for (int32_t i : u) {
        const muon_status st = apply_chunk(p, p->chunks[(size_t)i], cfg, s, side);
        if (st != MUON_OK) return st;
    }
    return MUON_OK;
}

// The whole step with two streams.  The pages overlap the exchange of the next batch of
// matrices with the orthogonalisation of the current one ("Frontier Pre-training at
// Microsoft AI", method details section 5, "Scaling Muon to 16K GPUs", the prefetching of
// the next batch).  On one GPU the work beside the products is the HBM-bound part of the
// step: while unit j's Newton–Schulz products run on the caller's stream s, unit j+1's
// momentum and normaliser (P_{j+1}) and unit j-1's apply (A_{j-1}) run on the plan's side
// stream d, in the side-stream kernels sized to share each compute unit with a product
// workgroup.  A task goes to d only if it fits the window (estimates above: side kernels
// are slower than the full-speed ones); otherwise it runs at full speed on s, P_{j+1} after
// NS(u_j) and A_{j-1} before it, so that the step is never much slower than one stream.
//
// For the tiled units u_0 .. u_{T-1} (small fused chunks first, as in the one-stream
// order, on s), with every task on d:
//   s: P_0, [W_0], NS(u_0), [wait P_1], [W_1], NS(u_1), ..., NS(u_{T-1}), A_{T-1}, [join]
//   d: [wait W_0], P_1, [wait NS(u_0)], A_0, [wait W_1], P_2, [wait NS(u_1)], A_1, ...
// W_j marks the start of window j on s: P_{j+1} waits for it, so it never starts before
// NS(u_{j-1}) and an A_{j-1} run on s are done; a P_{j+1} run on s after an A_{j-1} run on
// d waits for that apply when the two units share a region.  Consecutive units are in
// different regions, so what runs side by side never touches the same workspace bytes,
// and two regions are enough.  Events: 0 join, 1 + j W_j, 1 + T + j P_j done,
// 1 + 2T + j NS(u_j) done, 1 + 3T + j A_j done.
muon_status step_pipelined(const muon_plan* p, const std::vector<Unit>& u, const StepCfg& cfg, hipStream_t s) {
    muon_status st;
    hipError_t e = hipSuccess;
    const float* abc = cfg.abc.data();
    const size_t T = u.size();
    hipStream_t d = (hipStream_t)p->side;
    const size_t EV_JOIN = 0, EV_W = 1, EV_P = 1 + T, EV_NS = 1 + 2 * T, EV_A = 1 + 3 * T;

    std::vector<int32_t> small;
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i)
        if (p->chunks[(size_t)i].fused) small.push_back(i);
    if (!p->shared_regions) {
        for (int32_t i : small)
            if ((st = momentum_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
        if ((st = ns_small_chunks(p, small, abc, cfg.steps, cfg.eps, s)) != MUON_OK) return st;
        for (int32_t i : small)
            if ((st = apply_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
    } else {
        for (int32_t i : small) {
            const Chunk& c = p->chunks[(size_t)i];
            if ((st = momentum_chunk(p, c, cfg, s)) != MUON_OK) return st;
            if ((st = ns_one(p, i, abc, cfg.steps, cfg.eps, s)) != MUON_OK) return st;
            if ((st = apply_chunk(p, c, cfg, s)) != MUON_OK) return st;
        }
    }

    // placement of P_{j+1} and A_{j-1} beside NS(u_j) (pipe_place)
    std::vector<double> win(T, 0.0), tp(T, 0.0), ta(T, 0.0);
    for (size_t j = 0; j < T; ++j)
        for (int32_t i : u[j]) {
            const Chunk& c = p->chunks[(size_t)i];
            win[j] += est_ns_s(c, cfg.steps);
            tp[j] += est_prep_s(c);
            ta[j] += est_apply_s(c);
        }
    std::vector<char> p_side, a_side;
    pipe_place(win, tp, ta, p_side, a_side);

    if ((st = unit_momentum(p, u[0], cfg, s, false)) != MUON_OK) return st;
    if ((st = unit_prep(p, u[0], cfg, s, false)) != MUON_OK) return st;
    for (size_t j = 0; j < T; ++j) {
        if (j > 0 && p_side[j] && (e = wait(p, EV_P + j, s)) != hipSuccess) return hip_fail(e, "pipeline wait");
        if (j > 0 && !a_side[j - 1] && (st = unit_apply(p, u[j - 1], cfg, s, false)) != MUON_OK) return st;
        if ((e = record(p, EV_W + j, s)) != hipSuccess) return hip_fail(e, "pipeline record");
        if (j == 0 && (e = wait(p, EV_W, d)) != hipSuccess) return hip_fail(e, "pipeline fork");
        if ((st = unit_iterate(p, u[j], cfg, s)) != MUON_OK) return st;
        if (j + 1 < T) {
            if (p_side[j + 1]) {
                if ((e = wait(p, EV_W + j, d)) != hipSuccess) return hip_fail(e, "pipeline wait");
                if ((st = unit_momentum(p, u[j + 1], cfg, d, true)) != MUON_OK) return st;
                if ((st = unit_prep(p, u[j + 1], cfg, d, true)) != MUON_OK) return st;
                if ((e = record(p, EV_P + j + 1, d)) != hipSuccess) return hip_fail(e, "pipeline record");
            } else {
                if (j > 0 && a_side[j - 1] && same_region(p, u[j + 1], u[j - 1]) &&
                    (e = wait(p, EV_A + j - 1, s)) != hipSuccess)
                    return hip_fail(e, "pipeline wait");
                if ((st = unit_momentum(p, u[j + 1], cfg, s, false)) != MUON_OK) return st;
                if ((st = unit_prep(p, u[j + 1], cfg, s, false)) != MUON_OK) return st;
            }
        }
        if (a_side[j]) {
            if ((e = record(p, EV_NS + j, s)) != hipSuccess || (e = wait(p, EV_NS + j, d)) != hipSuccess)
                return hip_fail(e, "pipeline record");
            if ((st = unit_apply(p, u[j], cfg, d, true)) != MUON_OK) return st;
            if ((e = record(p, EV_A + j, d)) != hipSuccess) return hip_fail(e, "pipeline record");
        }
    }
    if ((st = unit_apply(p, u[T - 1], cfg, s, false)) != MUON_OK) return st;
    if ((e = record(p, EV_JOIN, d)) != hipSuccess || (e = wait(p, EV_JOIN, s)) != hipSuccess)
        return hip_fail(e, "pipeline join");
    return cfg.adam ? adam_run(p, cfg.adam_args, s) : MUON_OK;
}

// Steps 1, 3 and 5 for one chunk, or for every chunk (-1) on one stream.  With distinct
// regions every chunk's momentum runs first, then Newton–Schulz (small chunks grouped),
// then every apply; chunks that share a region go through all three in turn (the grouped
// small chunks, which sit in one region back to back, together).  With `pipeline` (every
// chunk), the two-stream order above where the plan allows it.
muon_status step_chunks(const muon_plan* p, int32_t chunk, const StepCfg& cfg, hipStream_t s) {
    muon_status st;
    const int32_t nc = (int32_t)p->chunks.size();
    const float* abc = cfg.abc.data();
    if (chunk == -1 && cfg.pipeline) {
        const std::vector<Unit> u = pipeline_units(p);
        if (!u.empty()) return step_pipelined(p, u, cfg, s);
    }
    if (chunk == -1 && !p->shared_regions) {
        for (int32_t i = 0; i < nc; ++i)
            if ((st = momentum_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
        if ((st = ns_all(p, abc, cfg.steps, cfg.eps, s)) != MUON_OK) return st;
        for (int32_t i = 0; i < nc; ++i)
            if ((st = apply_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
        return cfg.adam ? adam_run(p, cfg.adam_args, s) : MUON_OK;
    }
    bool group_done = false;
    for (int32_t i = 0; i < nc; ++i) {
        if (chunk != -1 && i != chunk) continue;
        const Chunk& ch = p->chunks[(size_t)i];
        if (chunk == -1 && ch.grouped) {
            if (group_done) continue;
            group_done = true;
            const Unit g = grouped_chunks(p);
            if ((st = unit_momentum(p, g, cfg, s, false)) != MUON_OK) return st;
            if ((st = ns_group(p, g, abc, cfg.steps, cfg.eps, s)) != MUON_OK) return st;
            if ((st = unit_apply(p, g, cfg, s, false)) != MUON_OK) return st;
            continue;
        }
        if ((st = momentum_chunk(p, ch, cfg, s)) != MUON_OK) return st;
        if ((st = ns_one(p, i, abc, cfg.steps, cfg.eps, s)) != MUON_OK) return st;
        if ((st = apply_chunk(p, ch, cfg, s)) != MUON_OK) return st;
    }
    // the AdamW parameters once, with the whole step (not with a single chunk)
    return (cfg.adam && chunk == -1) ? adam_run(p, cfg.adam_args, s) : MUON_OK;
}

// A StepCfg from the public config (validated).
muon_status make_cfg(const muon_step_config* c, StepCfg& cfg, const char* who) {
    if (!c) return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": config is NULL");
    cfg.steps = c->steps;
    if (c->steps < 1 || c->steps > MAX_NS_STEPS)
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": steps must be in [1, 1024]");
    if (c->coeffs) cfg.abc.assign(c->coeffs, c->coeffs + 3 * (size_t)c->steps);
    else fill_abc(cfg, c->a, c->b, c->c);
    muon_status st = check_ns(cfg.steps, cfg.abc.data(), c->eps, who);
    if (st != MUON_OK) return st;
    if (c->nesterov != 0 && c->nesterov != 1)
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": nesterov must be 0 or 1");
    if (!c->dev_scalars && (!finite(c->beta) || !finite(c->lr) || !finite(c->wd)))
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": beta, lr and wd must be finite");
    if (c->dev_scalars && ((uintptr_t)c->dev_scalars & 3u) != 0)
        return set_error(MUON_ERR_ALIGNMENT, std::string(who) + ": dev_scalars must be 4-byte aligned");
    cfg.beta = c->beta;
    cfg.lr = c->lr;
    cfg.wd = c->wd;
    cfg.eps = c->eps;
    cfg.nesterov = c->nesterov == 1;
    cfg.dev = c->dev_scalars;
    if (c->pipeline != 0 && c->pipeline != 1)
        return set_error(MUON_ERR_INVALID_ARG, std::string(who) + ": pipeline must be 0 or 1");
    cfg.pipeline = c->pipeline == 1;
    if (c->adamw) {
        if ((st = make_adam(c->adamw, cfg.adam_args, who)) != MUON_OK) return st;
        cfg.adam = true;
    }
    return MUON_OK;
}

muon_step_config legacy_config(float beta, float a, float b, float c, int32_t steps, float eps, float lr, float wd) {
    muon_step_config k{};
    k.beta = beta; k.lr = lr; k.wd = wd; k.eps = eps; k.steps = steps;
    k.a = a; k.b = b; k.c = c;
    return k;
}

// The tile grid of a chunk must fit the kernels' int32 indexing, one padded matrix (X, A
// or B) the 32-bit byte offsets of the buffer loads, and the chunk's rows the normaliser's
// 32-bit row index.
bool grid_fits(const Chunk& c) {
    const int64_t tm = c.mp / c.tile, tn = c.np / c.tile;
    const int64_t lim = int64_t(1) << 31;
    return c.count * tm * tn < lim && c.count * tm * (tm + 1) / 2 < lim && c.mp * c.np * 2 < lim &&
           c.mp * c.mp * 2 < lim && c.count * c.mp < lim;
}

// ---- the library's static scratch (muon_step_noalloc) -------------------------------------

constexpr uint64_t NOALLOC_BYTES = MUON_NOALLOC_MAX_BYTES;
static_assert(NOALLOC_BYTES % 16 == 0, "scratch is cleared in 16-byte units");

// One copy per GPU, in the code object's device memory.  Host code must not pass the
// array's name to a kernel (on the host it is only a handle for the runtime); it uses the
// device address looked up per device below.
static __device__ __attribute__((aligned(256))) uint8_t scratch[NOALLOC_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The scratch's device address on the current device, looked up on the first call there.
muon_status scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "muon_step_noalloc: hipGetDevice");
    if (dev < 0 || dev >= MAX_DEVICES) return set_error(MUON_ERR_INVALID_ARG, "muon_step_noalloc: device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "muon_step_noalloc: hipGetSymbolAddress(scratch)");
        if (!ptr || ((uintptr_t)ptr & (WS_ALIGN - 1)) != 0)
            return set_error(MUON_ERR_HIP, "muon_step_noalloc: the scratch's device address is not 256-byte aligned");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MUON_OK;
}

}  // namespace

extern "C" {

void muon_internal_release(muon_plan* p) {
    for (void* ev : p->timing.ev_begin) (void)hipEventDestroy((hipEvent_t)ev);
    for (void* ev : p->timing.ev_end) (void)hipEventDestroy((hipEvent_t)ev);
    p->timing = TimingState{};
    for (void* ev : p->pipe_events) (void)hipEventDestroy((hipEvent_t)ev);
    p->pipe_events.clear();
    if (p->side) (void)hipStreamDestroy((hipStream_t)p->side);
    p->side = nullptr;
}

muon_status muon_plan_bind(muon_plan* p, void* ws, uint64_t bytes, void* stream) {
    clear_error();
    if (!p || !ws) return set_error(MUON_ERR_INVALID_ARG, "muon_plan_bind: NULL plan or workspace");
    if (((uintptr_t)ws & (WS_ALIGN - 1)) != 0)
        return set_error(MUON_ERR_ALIGNMENT, "muon_plan_bind: workspace must be 256-byte aligned");
    if (bytes < p->ws_bytes)
        return set_error(MUON_ERR_WORKSPACE_TOO_SMALL, "muon_plan_bind: workspace holds " + std::to_string(bytes) +
                                                           " bytes; the plan needs " + std::to_string(p->ws_bytes));
    for (const Chunk& c : p->chunks)
        if (!grid_fits(c)) return set_error(MUON_ERR_SHAPE, "muon_plan_bind: chunk tile grid exceeds 2^31 tiles or a padded matrix exceeds 2 GiB");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemsetAsync(ws, 0, p->ws_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: hipMemsetAsync");
    if (!p->adam.empty()) {
        e = hipMemcpyAsync(static_cast<char*>(ws) + p->off_adam, p->adam.data(), p->adam.size() * sizeof(AdamEntry),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(static_cast<char*>(ws) + p->off_adam_segs, p->adam_segs.data(),
                               p->adam_segs.size() * sizeof(AdamSeg), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: AdamW table upload");
    }
    if (!p->table.empty() || !p->adam.empty()) {
        if (!p->table.empty())
            e = hipMemcpyAsync(ws, p->table.data(), p->table.size() * sizeof(MatEntry), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: table upload");
        // the host table is pageable memory owned by the plan; make sure the copy has
        // consumed it before the caller can free or change anything
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: stream synchronize");
    }
    // the two-stream pipeline's side stream (default priority) and ordering events, made
    // here so that no step has to create anything (a step may be under graph capture)
    if (!p->side) {
        hipStream_t side = nullptr;
        e = hipStreamCreateWithFlags(&side, hipStreamNonBlocking);
        if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: hipStreamCreateWithFlags");
        p->side = side;
    }
    while (p->pipe_events.size() < 1 + 4 * p->chunks.size()) {
        hipEvent_t ev = nullptr;
        e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
        if (e != hipSuccess) return hip_fail(e, "muon_plan_bind: hipEventCreateWithFlags");
        p->pipe_events.push_back(ev);
    }
    p->ws = ws;
    p->ws_given = bytes;
    p->bound = true;
    p->x0_fresh.assign(p->chunks.size(), 0);
    return MUON_OK;
}

muon_status muon_momentum_update(const muon_plan* p, int32_t chunk, float beta, void* stream) {
    clear_error();
    muon_status st = check_step(p, chunk, "muon_momentum_update");
    if (st != MUON_OK) return st;
    if (!finite(beta)) return set_error(MUON_ERR_INVALID_ARG, "muon_momentum_update: beta must be finite");
    StepCfg cfg;
    cfg.beta = beta;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i) {
        if (chunk != -1 && i != chunk) continue;
        if ((st = momentum_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
    }
    mark_x0(p, chunk, true);
    return MUON_OK;
}

muon_status muon_ns_batched_schedule(const muon_plan* p, int32_t chunk, const float* coeffs, int32_t steps,
                                     float eps, void* stream) {
    clear_error();
    muon_status st = check_step(p, chunk, "muon_ns_batched_schedule");
    if (st != MUON_OK) return st;
    if (!coeffs) return set_error(MUON_ERR_INVALID_ARG, "muon_ns_batched_schedule: coeffs is NULL");
    if (steps < 1 || steps > MAX_NS_STEPS)
        return set_error(MUON_ERR_INVALID_ARG, "muon_ns_batched_schedule: steps must be in [1, 1024]");
    if ((st = check_ns(steps, coeffs, eps, "muon_ns_batched_schedule")) != MUON_OK) return st;
    if ((st = check_x0(p, chunk, "muon_ns_batched_schedule")) != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mark_x0(p, chunk, false);
    if (chunk == -1) return ns_all(p, coeffs, steps, eps, s);
    return ns_one(p, chunk, coeffs, steps, eps, s);
}

muon_status muon_ns_batched(const muon_plan* p, int32_t chunk, float a, float b, float c, int32_t steps,
                            float eps, void* stream) {
    clear_error();
    muon_status st = check_step(p, chunk, "muon_ns_batched");
    if (st != MUON_OK) return st;
    if (steps < 1 || steps > MAX_NS_STEPS)
        return set_error(MUON_ERR_INVALID_ARG, "muon_ns_batched: steps must be in [1, 1024]");
    StepCfg cfg;
    cfg.steps = steps;
    fill_abc(cfg, a, b, c);
    if ((st = check_ns(steps, cfg.abc.data(), eps, "muon_ns_batched")) != MUON_OK) return st;
    if ((st = check_x0(p, chunk, "muon_ns_batched")) != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mark_x0(p, chunk, false);
    if (chunk == -1) return ns_all(p, cfg.abc.data(), steps, eps, s);
    return ns_one(p, chunk, cfg.abc.data(), steps, eps, s);
}

muon_status muon_apply(const muon_plan* p, int32_t chunk, float lr, float wd, void* stream) {
    clear_error();
    muon_status st = check_step(p, chunk, "muon_apply");
    if (st != MUON_OK) return st;
    if (!finite(lr) || !finite(wd)) return set_error(MUON_ERR_INVALID_ARG, "muon_apply: lr and wd must be finite");
    StepCfg cfg;
    cfg.lr = lr;
    cfg.wd = wd;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < (int32_t)p->chunks.size(); ++i) {
        if (chunk != -1 && i != chunk) continue;
        if ((st = apply_chunk(p, p->chunks[(size_t)i], cfg, s)) != MUON_OK) return st;
    }
    return MUON_OK;
}

muon_status muon_step_ex(const muon_plan* p, int32_t chunk, const muon_step_config* config, void* stream) {
    clear_error();
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_step_ex: plan is NULL");
    if (!p->bound) return set_error(MUON_ERR_NOT_BOUND, "muon_step_ex: call muon_plan_bind first");
    if (chunk < -1 || chunk >= (int32_t)p->chunks.size())
        return set_error(MUON_ERR_INVALID_ARG, "muon_step_ex: chunk out of range");
    StepCfg cfg;
    muon_status st = make_cfg(config, cfg, "muon_step_ex");
    if (st != MUON_OK) return st;
    mark_x0(p, chunk, false);      // the step makes and consumes its own X0
    return step_chunks(p, chunk, cfg, static_cast<hipStream_t>(stream));
}

muon_status muon_adamw_step(const muon_plan* p, const muon_adamw_config* config, void* stream) {
    clear_error();
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_adamw_step: plan is NULL");
    if (!p->bound) return set_error(MUON_ERR_NOT_BOUND, "muon_adamw_step: call muon_plan_bind first");
    AdamArgs a{};
    muon_status st = make_adam(config, a, "muon_adamw_step");
    if (st != MUON_OK) return st;
    return adam_run(p, a, static_cast<hipStream_t>(stream));
}

muon_status muon_step_noalloc(const muon_plan* p, const muon_step_config* config, void* stream) {
    clear_error();
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_step_noalloc: plan is NULL");
    StepCfg cfg;
    muon_status st = make_cfg(config, cfg, "muon_step_noalloc");
    if (st != MUON_OK) return st;
    cfg.pipeline = false;
    if (p->ws_bytes > NOALLOC_BYTES)
        return set_error(MUON_ERR_WORKSPACE_TOO_SMALL, "muon_step_noalloc: the plan needs " +
                                                           std::to_string(p->ws_bytes) + " bytes of workspace; the static scratch holds " +
                                                           std::to_string(NOALLOC_BYTES));
    for (const Chunk& c : p->chunks)
        if (!grid_fits(c)) return set_error(MUON_ERR_SHAPE, "muon_step_noalloc: chunk tile grid too large");
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the previous call's contents go: clear what this plan uses, then its tables
    hipError_t e = launch_zero(ws, (p->ws_bytes + 15) / 16, s);
    if (e != hipSuccess) return hip_fail(e, "muon_step_noalloc: clear kernel launch");
    if (!p->adam.empty()) {
        e = hipMemcpyAsync(static_cast<char*>(ws) + p->off_adam, p->adam.data(), p->adam.size() * sizeof(AdamEntry),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(static_cast<char*>(ws) + p->off_adam_segs, p->adam_segs.data(),
                               p->adam_segs.size() * sizeof(AdamSeg), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "muon_step_noalloc: AdamW table copy");
    }
    if (!p->table.empty()) {
        e = hipMemcpyAsync(ws, p->table.data(), p->table.size() * sizeof(MatEntry), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "muon_step_noalloc: table copy");
    }
    // the step's kernels take their addresses from the plan's workspace base: point it at
    // the scratch for the launches (calls on one plan do not overlap), then restore it
    muon_plan* mp = const_cast<muon_plan*>(p);
    void* const saved = mp->ws;
    mp->ws = ws;
    st = step_chunks(mp, -1, cfg, s);
    mp->ws = saved;
    mark_x0(p, -1, false);
    return st;
}

muon_status muon_step(const muon_plan* p, int32_t chunk, float beta, float a, float b, float c, int32_t steps,
                      float eps, float lr, float wd, void* stream) {
    const muon_step_config k = legacy_config(beta, a, b, c, steps, eps, lr, wd);
    return muon_step_ex(p, chunk, &k, stream);
}

// ---- the step as one graph ----------------------------------------------------------------

muon_status muon_graph_capture_ex(const muon_plan* p, const muon_step_config* config, muon_graph** out) {
    clear_error();
    if (!out) return set_error(MUON_ERR_INVALID_ARG, "muon_graph_capture: out is NULL");
    *out = nullptr;
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_graph_capture: plan is NULL");
    if (!p->bound) return set_error(MUON_ERR_NOT_BOUND, "muon_graph_capture: call muon_plan_bind first");
    StepCfg cfg;
    muon_status st = make_cfg(config, cfg, "muon_graph_capture");
    if (st != MUON_OK) return st;

    // A private stream: the caller's stream may be the null stream, which cannot capture.
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "muon_graph_capture: hipStreamCreateWithFlags");
    hipGraph_t graph = nullptr;
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return hip_fail(e, "muon_graph_capture: hipStreamBeginCapture");
    }
    t_capturing = true;
    st = step_chunks(p, -1, cfg, cs);
    t_capturing = false;
    mark_x0(p, -1, false);         // every replay makes and consumes its own X0
    const std::string launch_error = st == MUON_OK ? std::string() : std::string(muon_last_error());
    e = hipStreamEndCapture(cs, &graph);
    (void)hipStreamDestroy(cs);
    if (st != MUON_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return set_error(st, "muon_graph_capture: " + launch_error);
    }
    if (e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return hip_fail(e, "muon_graph_capture: hipStreamEndCapture");
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return hip_fail(e, "muon_graph_capture: hipGraphInstantiate");
    }
    size_t nodes = 0;
    (void)hipGraphGetNodes(graph, nullptr, &nodes);
    muon_graph* g = new muon_graph;
    g->graph = graph;
    g->exec = exec;
    g->nodes = (int64_t)nodes;
    g->ws = p->ws;
    *out = g;
    return MUON_OK;
}

muon_status muon_graph_capture(const muon_plan* p, float beta, float a, float b, float c, int32_t steps, float eps,
                               float lr, float wd, muon_graph** out) {
    const muon_step_config k = legacy_config(beta, a, b, c, steps, eps, lr, wd);
    return muon_graph_capture_ex(p, &k, out);
}

muon_status muon_graph_launch(const muon_graph* g, void* stream) {
    clear_error();
    if (!g) return set_error(MUON_ERR_INVALID_ARG, "muon_graph_launch: graph is NULL");
    const hipError_t e = hipGraphLaunch((hipGraphExec_t)g->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MUON_OK : hip_fail(e, "muon_graph_launch: hipGraphLaunch");
}

muon_status muon_graph_node_count(const muon_graph* g, int64_t* nodes) {
    clear_error();
    if (!g || !nodes) return set_error(MUON_ERR_INVALID_ARG, "muon_graph_node_count: bad argument");
    *nodes = g->nodes;
    return MUON_OK;
}

void muon_graph_destroy(muon_graph* g) {
    if (!g) return;
    (void)hipGraphExecDestroy((hipGraphExec_t)g->exec);
    (void)hipGraphDestroy((hipGraph_t)g->graph);
    delete g;
}

muon_status muon_timing_enable(muon_plan* p, int32_t capacity) {
    clear_error();
    if (!p || capacity < 0) return set_error(MUON_ERR_INVALID_ARG, "muon_timing_enable: bad argument");
    TimingState& t = p->timing;
    while ((int32_t)t.ev_begin.size() < capacity) {
        hipEvent_t b0, e0;
        hipError_t e = hipEventCreate(&b0);
        if (e != hipSuccess) return hip_fail(e, "muon_timing_enable: hipEventCreate");
        e = hipEventCreate(&e0);
        if (e != hipSuccess) {
            (void)hipEventDestroy(b0);
            return hip_fail(e, "muon_timing_enable: hipEventCreate");
        }
        t.ev_begin.push_back(b0);
        t.ev_end.push_back(e0);
    }
    t.kind.assign((size_t)capacity, -1);
    t.work.assign((size_t)capacity, 0.0);
    t.capacity = capacity;
    t.used = 0;
    return MUON_OK;
}

muon_status muon_timing_reset(muon_plan* p) {
    if (!p) return set_error(MUON_ERR_INVALID_ARG, "muon_timing_reset: plan is NULL");
    p->timing.used = 0;
    return MUON_OK;
}

muon_status muon_timing_read(muon_plan* p, int32_t kernel, double* total_ms, int64_t* launches, double* work) {
    clear_error();
    if (!p || kernel < 0 || kernel >= MUON_KERNEL_COUNT)
        return set_error(MUON_ERR_INVALID_ARG, "muon_timing_read: bad argument");
    double ms = 0.0, wk = 0.0;
    int64_t n = 0;
    TimingState& t = p->timing;
    for (int32_t i = 0; i < t.used; ++i) {
        if (t.kind[(size_t)i] != kernel) continue;
        hipError_t e = hipEventSynchronize((hipEvent_t)t.ev_end[(size_t)i]);
        if (e != hipSuccess) return hip_fail(e, "muon_timing_read: hipEventSynchronize");
        float f = 0.f;
        e = hipEventElapsedTime(&f, (hipEvent_t)t.ev_begin[(size_t)i], (hipEvent_t)t.ev_end[(size_t)i]);
        if (e != hipSuccess) return hip_fail(e, "muon_timing_read: hipEventElapsedTime");
        ms += f;
        wk += t.work[(size_t)i];
        ++n;
    }
    if (total_ms) *total_ms = ms;
    if (launches) *launches = n;
    if (work) *work = wk;
    return MUON_OK;
}

const char* muon_kernel_name(int32_t k) {
    switch (k) {
        case MUON_KERNEL_MOMENTUM: return "momentum";
        case MUON_KERNEL_NORM_FINALIZE: return "norm_finalize";
        case MUON_KERNEL_NORMALIZE: return "normalize";
        case MUON_KERNEL_SYRK: return "syrk";
        case MUON_KERNEL_SYRK_POLY: return "syrk_poly";
        case MUON_KERNEL_GEMM_AXPY: return "gemm_axpy";
        case MUON_KERNEL_APPLY: return "apply";
        case MUON_KERNEL_NS_SMALL: return "ns_small";
        case MUON_KERNEL_ADAMW: return "adamw";
        case MUON_KERNEL_MOMENTUM_SIDE: return "momentum_side";
        case MUON_KERNEL_NORMALIZE_SIDE: return "normalize_side";
        case MUON_KERNEL_APPLY_SIDE: return "apply_side";
        case MUON_KERNEL_NS_GROUPED: return "ns_grouped";
        case MUON_KERNEL_PREP_GROUPED: return "prep_grouped";
        default: return "unknown";
    }
}

}  // extern "C"
