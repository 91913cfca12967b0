/*
 * libmuon — one Muon optimizer step on an AMD Instinct MI355X (gfx950).
 *
 * The step the pages describe ("Frontier Pre-training at Microsoft AI", method details
 * section 5, "Scaling Muon to 16K GPUs", resharding steps 1, 3 and 5; the same step in
 * "Microsoft Reveals MAI-Base-2 Training Recipe ...", section "How to Make Parameter
 * Updates Faster and More Stable?"):
 *
 *   1. each GPU updates its FP32 momentum and casts it to BF16;
 *   3. each GPU orthogonalises whole momentum matrices, batched by shape, with a
 *      Newton–Schulz operator built for the symmetric intermediates;
 *   5. the update is cast back to FP32 and applied to the weights.
 *
 * On one GPU the all-to-all exchanges of steps 2 and 4 have no counterpart: this library
 * takes one GPU's share of whole matrices.  Two points of that section become the plan
 * below: matrices of one shape are processed together as a batch, and the indexing
 * metadata of the resharding is worked out once and then reused every step.
 *
 * Memory and ownership
 *   The caller owns every device buffer: weights W, momenta M, gradients G and the
 *   workspace.  The library owns only the host-side plan object.  It never allocates or
 *   frees device memory.  All step calls are asynchronous on the given stream, never
 *   synchronise, and can be captured in a HIP graph.
 *
 * Errors
 *   Every call returns a muon_status synchronously; MUON_OK is 0.  muon_last_error()
 *   gives a message for the last failing call on the calling thread.  Device faults
 *   surface at the caller's next synchronisation.  NaN and Inf are data, not errors:
 *   they stay inside the matrix they occur in.
 *
 * Threading
 *   A bound plan's layout never changes.  Step calls on one plan must not overlap on
 *   different streams: they share the workspace.
 *
 * Streams are passed as `void*` holding a hipStream_t (NULL = the null stream).
 */
#ifndef LIBMUON_MUON_H
#define LIBMUON_MUON_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MUON_API __attribute__((visibility("default")))
#else
#define MUON_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t muon_status;
#define MUON_OK 0
#define MUON_ERR_INVALID_ARG 1         /* null pointer, bad enum, bad chunk or scalar     */
#define MUON_ERR_SHAPE 2               /* zero or oversized dimension                     */
#define MUON_ERR_ALIGNMENT 3           /* device pointer not 16-byte aligned              */
#define MUON_ERR_WORKSPACE_TOO_SMALL 4 /* workspace below muon_plan_workspace_bytes()     */
#define MUON_ERR_NOT_BOUND 5           /* step call before muon_plan_bind()               */
#define MUON_ERR_STALE_PLAN 6          /* descriptors no longer match the plan            */
#define MUON_ERR_HIP 7                 /* a HIP runtime call failed (message in last_error) */

#define MUON_DTYPE_F32 0
#define MUON_DTYPE_BF16 1

/* One parameter as the caller holds it.  The pages apply Muon to every 2-D matrix that is
 * not an embedding and AdamW to the rest, scalars and embeddings ("Frontier Pre-training
 * at Microsoft AI", setup section 4; "Microsoft Reveals MAI-Base-2 Training Recipe ...",
 * section "How to Make Parameter Updates Faster and More Stable?").  `optimizer` says
 * which one a parameter takes:
 *   MUON_OPT_DEFAULT  ndim == 2: Muon; otherwise AdamW when exp_avg_sq is non-NULL,
 *                     else excluded (its pointers are then not read);
 *   MUON_OPT_ADAMW    AdamW whatever ndim (embeddings);
 *   MUON_OPT_NONE     excluded.
 * Muon: weight, momentum are rows x cols float32, grad rows x cols of grad_dtype, all
 * row-major, contiguous, device, 16-B aligned.  AdamW: weight, momentum (the first
 * moment), exp_avg_sq (the second moment) are float32 and grad of grad_dtype, each
 * rows * cols contiguous elements (a parameter of another ndim passes rows = its
 * element count and cols = 1), device, 16-B aligned.  Written buffers (weight,
 * momentum, exp_avg_sq) must not overlap each other, any other parameter's, or a grad. */
typedef struct muon_param_desc {
    int32_t ndim;
    int32_t grad_dtype; /* MUON_DTYPE_F32 or MUON_DTYPE_BF16 */
    int64_t rows;
    int64_t cols;
    float* weight;
    float* momentum;
    const void* grad;
    float* exp_avg_sq;  /* AdamW only */
    int32_t optimizer;  /* MUON_OPT_* */
    int32_t reserved;
} muon_param_desc;

#define MUON_OPT_DEFAULT 0
#define MUON_OPT_ADAMW 1
#define MUON_OPT_NONE 2

/* Plan options.  A zero-filled struct (or NULL) means: no workspace cap, scale 1. */
typedef struct muon_plan_opts {
    /* Upper bound on the workspace in bytes; 0 = no bound.  Above the bound, buckets
     * are split into chunks that share one workspace region and must then be stepped
     * one chunk at a time (momentum, NS, apply for chunk i before chunk i+1). */
    uint64_t max_workspace_bytes;
    /* Host, nullable: per-parameter update scale s_i (n entries, indexed like the
     * descriptors; entries of excluded parameters are ignored).  NULL means s_i = 1.
     * The pages give no scale rule; the scale is a free per-matrix factor. */
    const float* scale;
    /* MUON_PLAN_* bits; 0 for the defaults.  Other bits: INVALID_ARG. */
    uint32_t flags;
    /* Update-scale rule used where `scale` is NULL (MUON_SCALE_*).  The pages give no
     * rule: one of them notes only that careful per-parameter scaling of the update
     * was a key to scaling Muon, in the prior work it names ("MAI-Base-2 в 4–12 раз
     * экономнее DeepSeek на предобучении", section "Muon обошёл AdamW, но потребовал
     * пересобирать матрицы между GPU"). */
    int32_t scale_mode;
} muon_plan_opts;

/* s_i = 1. */
#define MUON_SCALE_NONE 0
/* s_i = sqrt(max(1, rows / cols)) of the parameter as stored (rows = outputs): the
 * scale of the original Muon write-up, which keeps tall matrices' per-element update
 * size in line with square ones. */
#define MUON_SCALE_ASPECT 1
/* s_i = 0.2 * sqrt(max(rows, cols)): gives the orthogonalised update an RMS of about
 * 0.2, the range of AdamW's updates (the rule of Moonshot AI's Muon scaling paper). */
#define MUON_SCALE_RMS_MATCH 2

/* Orthogonalise small matrices with the tiled kernels too, instead of the fused
 * whole-iteration kernel (both give bitwise the same result; this exists to show it). */
#define MUON_PLAN_TILED_SMALL 1u
/* Plan for the two-stream step (muon_step_config.pipeline), which hides one chunk's
 * neighbours' elementwise work behind its Newton–Schulz products and so needs several
 * chunks: a large bucket is split into up to 8 chunks, as many as keep at least 2048
 * SYRK workgroups per launch (sizes differing by at most one).  The buckets of 256-row
 * output tiles (m >= 1024) come first, and a smaller chunk may be split off the front of
 * the first such chunk and off the back of the last one (their elementwise work is the
 * part nothing hides), sized by an estimate of the step time that the plan computes from
 * the shapes alone.  With a workspace cap that splits buckets anyway, the chunks are laid
 * out in two regions of at most half the remaining cap each, alternating between
 * consecutive tiled chunks, so that one chunk can be prepared while the previous one is
 * orthogonalised.  Results do not depend on the chunking. */
#define MUON_PLAN_PIPELINE 2u
/* Normalise in a separate pass instead of in the first iteration's operand loads.  By
 * default a chunk of 256-row output tiles (m >= 1024) run for an odd number of iterations
 * never writes the normalised X: its first SYRK and GEMM+axpy read X0 and normalise each
 * value on its way into LDS, with the same arithmetic as the pass (bitwise the same
 * result; this exists to show it). */
#define MUON_PLAN_UNFUSED_NORMALIZE 4u
/* Run each small tiled chunk (128- or 64-row tiles: 64 < m < 1024, or m <= 64 with a
 * padded n above 1024, e.g. routers and gates) on its own.  By default all of a plan's
 * small tiled chunks are orthogonalised together: one launch normalises them all and one
 * launch per product and iteration works through a single queue of all their tiles (the
 * pages treat router weights apart from the bulk of the experts: "Frontier Pre-training
 * at Microsoft AI", method details section 5).  Both give bitwise the same result; this
 * exists to show it. */
#define MUON_PLAN_UNGROUPED 8u

typedef struct muon_plan muon_plan;

/* Per-chunk facts, for reporting. */
typedef struct muon_chunk_info {
    int64_t m, n;          /* canonical shape: m = min(rows, cols), n = max(rows, cols) */
    int64_t m_pad, n_pad;  /* padded workspace shape of every matrix in the chunk       */
    int64_t count;         /* matrices in the chunk                                    */
    int32_t bucket;        /* bucket id (chunks of one bucket share it)                */
    int32_t tile;          /* Newton–Schulz output tile edge                           */
    int32_t grad_dtype;
    int32_t shared_region; /* 1 when this chunk shares its workspace region            */
    int32_t fused_small;   /* 1 when one fused kernel runs this chunk's whole NS        */
    int32_t grouped_small; /* 1 when the chunk's products run in the grouped launches of
                              every small tiled chunk (MUON_PLAN_UNGROUPED)              */
    double flops_conventional; /* per NS iteration: 4 m^2 n + 2 m^3, times count        */
    double flops_algorithmic;  /* per NS iteration: m(m+1)n + m^2(m+1) + 2 m^2 n, x count */
    double bytes_momentum;     /* algorithmic HBM bytes of the momentum kernel          */
    double bytes_apply;        /* algorithmic HBM bytes of the apply kernel             */
    uint64_t region_offset;    /* byte offset of the chunk's region in the workspace    */
    uint64_t region_bytes;
} muon_chunk_info;

/* Where one parameter's orthogonalised update O lives after muon_ns_batched. */
typedef struct muon_param_info {
    int32_t included;       /* 1: Muon; 2: AdamW; 0: excluded (for 0 and 2 the rest is 0) */
    int32_t chunk;
    int64_t slot;           /* index of the matrix inside its chunk                   */
    int32_t transposed;     /* 1 when rows > cols: O is stored as the m x n transpose */
    float scale;            /* the update scale s_i the apply step uses               */
    uint64_t output_offset; /* byte offset of O (bf16, m x n, row stride ld) in the workspace */
    int64_t ld;             /* row stride of O in elements (= n_pad)                  */
} muon_param_info;

/* ---- plan (host only; no device calls) ---------------------------------------------- */

/* Build a plan for n parameters: exclude ndim != 2, canonicalise each matrix to
 * (m, n) = (min, max) with a transpose flag when rows > cols, group by (m, n, grad
 * dtype) into buckets, split buckets into chunks under the workspace cap, lay out the
 * workspace and build the per-matrix tables.  On success *out owns a new plan.
 * Errors: INVALID_ARG (null params with n > 0, null out, bad dtype, null or
 * overlapping buffers), SHAPE (rows or cols <= 0, or a padded matrix above 2^31
 * elements), ALIGNMENT (a buffer not 16-B aligned), WORKSPACE_TOO_SMALL (one matrix of
 * some bucket does not fit under the cap). */
MUON_API muon_status muon_plan_buckets(const muon_param_desc* params, int64_t n,
                              const muon_plan_opts* opts, muon_plan** out);

/* Bytes of device workspace the plan needs (256-B aligned start required). */
MUON_API muon_status muon_plan_workspace_bytes(const muon_plan* plan, uint64_t* bytes);

/* Number of chunks and buckets; counts of the parameters that take Muon (included) and
 * of those that take neither optimizer (excluded).  Any pointer may be NULL. */
MUON_API muon_status muon_plan_counts(const muon_plan* plan, int32_t* n_chunks, int32_t* n_buckets,
                             int64_t* n_included, int64_t* n_excluded);
/* Count and total elements of the parameters that take AdamW (any pointer may be NULL). */
MUON_API muon_status muon_plan_adamw_counts(const muon_plan* plan, int64_t* n_params, int64_t* n_elements);

MUON_API muon_status muon_plan_info(const muon_plan* plan, int32_t chunk, muon_chunk_info* out);

MUON_API muon_status muon_plan_param_info(const muon_plan* plan, int64_t param, muon_param_info* out);

/* STALE_PLAN when the descriptors differ from those the plan was built from (count,
 * ndim, shape, dtype or any pointer), else OK. */
MUON_API muon_status muon_plan_validate(const muon_plan* plan, const muon_param_desc* params, int64_t n);

/* ---- bind (device) ------------------------------------------------------------------- */

/* Attach a caller-owned device workspace (>= muon_plan_workspace_bytes, 256-B aligned)
 * and upload the plan's tables, ordered on `stream`.  Also zero-fills the workspace.
 * May be called again with another workspace.  Errors: INVALID_ARG, ALIGNMENT,
 * WORKSPACE_TOO_SMALL, SHAPE (a chunk needs 2^31 or more tiles, or one padded matrix
 * takes 2 GiB or more: about 32768 x 32768), HIP. */
MUON_API muon_status muon_plan_bind(muon_plan* plan, void* workspace, uint64_t bytes, void* stream);

/* ---- the step (device, asynchronous on `stream`) --------------------------------------- */

/* Step 1.  For every matrix of `chunk` (-1 = every chunk; not allowed when chunks share
 * a region): M <- beta*M + (1-beta)*G with both products and the sum in float64 and one
 * float32 store; X0 = bf16(M) (round to nearest even) written to the workspace in
 * canonical orientation; per-tile sums of X0^2 for the normaliser.  beta = 0 copies G
 * into M.  Errors: INVALID_ARG (chunk, non-finite beta), NOT_BOUND, HIP. */
MUON_API muon_status muon_momentum_update(const muon_plan* plan, int32_t chunk, float beta, void* stream);

/* Step 3.  For every matrix of `chunk`: X = bf16(X0 / (||X0||_F + eps)) (the norm summed
 * in float64; X0 times the reciprocal, the float64 product rounded once to bf16, which
 * float32 products reach through a per-matrix float32 scale chosen for it), then `steps`
 * quintic Newton–Schulz iterations, each
 *     A = X X^T (bf16),  B = b A + c A A (bf16),  X = a X + B X (bf16),
 * with bf16 MFMA products accumulated in float32.  A and B are symmetric; only their
 * upper-triangle tiles are computed and then mirrored.  The result O is left in the
 * workspace (see muon_plan_param_info).  The pages give no coefficients or step count;
 * (3.4445, -4.7750, 2.0315), 5 steps and eps = 1e-7 are the usual choice.  ("Frontier
 * Pre-training at Microsoft AI", method details section 5, resharding step 3: the
 * orthogonalisation of whole same-shape matrices with an operator for symmetric
 * intermediates.)  For chunks of 256-row tiles (m >= 1024) and an odd step count the
 * normalisation happens inside the first iteration's loads (bitwise the same X).
 * The call consumes X0: the iterations overwrite it, so each call needs a muon_momentum_update
 * of the chunk after the last Newton–Schulz call or step that touched it (or that touched
 * another chunk in the same workspace region); the plan tracks this in the order calls are
 * made and refuses the call otherwise.
 * Errors: INVALID_ARG (chunk, steps < 1, non-finite scalars, no fresh X0), NOT_BOUND, HIP. */
MUON_API muon_status muon_ns_batched(const muon_plan* plan, int32_t chunk, float a, float b, float c,
                            int32_t steps, float eps, void* stream);

/* Step 5.  For every matrix of `chunk`: W <- f32((1 - lr*wd) * W - lr*s_i*O), each
 * product and the difference rounded to float64 separately (no fused multiply-add),
 * O read back in the parameter's own orientation.  Decoupled weight decay: the decay's
 * time scale is 1/(lr*wd) ("Frontier Pre-training at Microsoft AI", method details
 * section 3), so lr and wd are plain arguments and wd = 17.04/(steps*lr) plugs in.
 * Errors: INVALID_ARG (chunk, non-finite lr or wd), NOT_BOUND, HIP. */
MUON_API muon_status muon_apply(const muon_plan* plan, int32_t chunk, float lr, float wd, void* stream);

/* Steps 1, 3 and 5 for `chunk` (-1 = every chunk, in order), with the arguments above. */
MUON_API muon_status muon_step(const muon_plan* plan, int32_t chunk, float beta, float a, float b,
                      float c, int32_t steps, float eps, float lr, float wd, void* stream);

/* ---- variants the pages leave open ------------------------------------------------------ */

/* Step 3 with its own coefficients per iteration: `coeffs` (host) holds 3*steps floats
 * (a_t, b_t, c_t), t = 1..steps; iteration t runs A = X X^T, B = b_t A + c_t A A,
 * X = a_t X + B X.  The pages fix neither the coefficients nor their schedule;
 * muon_ns_batched is this call with the same (a, b, c) every iteration.
 * Errors: INVALID_ARG (chunk, coeffs NULL, steps outside [1, 1024], non-finite values,
 * eps < 0, no fresh X0 as for muon_ns_batched), NOT_BOUND, HIP. */
MUON_API muon_status muon_ns_batched_schedule(const muon_plan* plan, int32_t chunk, const float* coeffs,
                                     int32_t steps, float eps, void* stream);

/* AdamW for the parameters that take it (the pages' companion optimizer, see
 * muon_param_desc), decoupled weight decay as in the Muon apply.  Per element, float64
 * arithmetic with every operation rounded once, in this order, then float32 stores:
 *     m = beta1*m + (1-beta1)*g;   v = beta2*v + (1-beta2)*(g*g);
 *     w = (1 - lr*wd)*w - (lr * (m / bc1)) / (sqrt(v / bc2) + eps),
 * with bc1 = 1 - beta1^t, bc2 = 1 - beta2^t formed in float64 on the host (the float32 m
 * and v are the values stored).  The pages give no AdamW hyper-parameters. */
typedef struct muon_adamw_config {
    float lr, beta1, beta2, eps, wd;
    int32_t reserved;
    int64_t step;              /* t >= 1, for the bias corrections                      */
    /* Device, nullable, 4-byte aligned: {lr, wd, bc1, bc2} as four floats, read by the
     * kernel when it runs instead of lr, wd and the bias corrections from `step` (for
     * graph replays; bc1 and bc2 are then float32 values). */
    const float* dev_scalars;
} muon_adamw_config;

/* AdamW over every AdamW parameter of the plan, one launch.  Errors: INVALID_ARG (NULL
 * config, step < 1, non-finite or out-of-range hyper-parameters), ALIGNMENT, NOT_BOUND,
 * HIP.  Nothing is launched when the plan has no AdamW parameter. */
MUON_API muon_status muon_adamw_step(const muon_plan* plan, const muon_adamw_config* config, void* stream);

/* Everything one step takes, for muon_step_ex and muon_graph_capture_ex. */
typedef struct muon_step_config {
    float beta;                /* momentum coefficient                                     */
    float lr, wd;              /* learning rate, decoupled weight decay                    */
    float eps;                 /* added to the Frobenius norm (>= 0)                       */
    int32_t steps;             /* Newton–Schulz iterations, 1..1024                        */
    float a, b, c;             /* each iteration's coefficients when `coeffs` is NULL      */
    const float* coeffs;       /* host, nullable: 3*steps floats (a_t, b_t, c_t)           */
    /* 0: Newton–Schulz takes bf16(M_new), the momentum itself (the pages' step 1).
     * 1: it takes the Nesterov look-ahead bf16(f32(beta*M_new + (1-beta)*G)), formed like
     *    the momentum (float64 products and sum, one float32 rounding).  The stored
     *    momentum is M_new either way. */
    int32_t nesterov;
    /* Device, nullable, 4-byte aligned: {beta, lr, wd} as three floats, read by the
     * kernels when they run instead of the fields above (whose values are then
     * ignored).  A captured graph then follows a learning-rate or decay schedule: write
     * the new values into this buffer, ordered before each launch.  Non-finite values
     * are not checked; they propagate as data. */
    const float* dev_scalars;
    /* Host, nullable: also run AdamW over the plan's AdamW parameters (after the Muon
     * step, on the same stream), so one call updates every parameter. */
    const muon_adamw_config* adamw;
    /* 0: one stream, phase by phase.  1: the two-stream pipeline, for whole steps
     * (chunk -1): while one chunk's Newton–Schulz products run on `stream`, the next
     * chunk's momentum and normaliser and the previous chunk's apply run on a second
     * stream that the plan owns (created at bind, default priority), in kernels small
     * enough to share the compute units with the products; the call returns with all of
     * it ordered before later work on `stream`.  The pages overlap the next batch's
     * exchange with the current batch's orthogonalisation ("Frontier Pre-training at
     * Microsoft AI", method details section 5, "Scaling Muon to 16K GPUs").  Results are
     * bitwise those of 0.  It needs at least two tiled chunks, no two consecutive ones
     * in one workspace region (always so without a binding cap; with one, plan with
     * MUON_PLAN_PIPELINE); otherwise the step runs as with 0.  Steps of one plan
     * must not overlap: the second stream is shared by every call on the plan. */
    int32_t pipeline;
} muon_step_config;

/* muon_step with a muon_step_config.  Errors: INVALID_ARG (NULL config, chunk, steps,
 * non-finite scalars or coefficients, nesterov or pipeline not 0/1), ALIGNMENT
 * (dev_scalars), NOT_BOUND, HIP. */
MUON_API muon_status muon_step_ex(const muon_plan* plan, int32_t chunk, const muon_step_config* config,
                         void* stream);

/* ---- the whole step as one graph ------------------------------------------------------- */

/* The pages count kernel-dispatch overhead among the causes of the gap between the
 * measured optimizer step and its communication limit ("Frontier Pre-training at
 * Microsoft AI", method details section 5, "Scaling Muon to 16K GPUs", overhead
 * analysis; the same list in "MAI-Base-2 в 4–12 раз экономнее DeepSeek на
 * предобучении", its optimizer section).
 * A step issues 2 + 3*steps + 2 launches per chunk; as a graph it is one launch.
 *
 * muon_graph_capture records muon_step(plan, -1, ...) on a private stream into a HIP
 * graph and instantiates it.  Nothing runs during capture.  The graph holds the device
 * addresses of W, M, G and of the workspace bound at capture time, and the scalars
 * given here: a later muon_plan_bind does not move it, and the caller keeps all of
 * those buffers alive and in place while the graph exists.  New gradients are picked
 * up by writing them into the same G buffers before each launch.  Kernel timing is not
 * recorded inside graphs.  Errors: INVALID_ARG, NOT_BOUND, HIP (capture or
 * instantiation failed; nothing is left allocated). */
typedef struct muon_graph muon_graph;
MUON_API muon_status muon_graph_capture(const muon_plan* plan, float beta, float a, float b, float c,
                               int32_t steps, float eps, float lr, float wd, muon_graph** out);
/* muon_graph_capture with a muon_step_config (schedules, Nesterov, device scalars). */
MUON_API muon_status muon_graph_capture_ex(const muon_plan* plan, const muon_step_config* config,
                                  muon_graph** out);
/* Launch one step, ordered on `stream` (the null stream is allowed).  Launches of one
 * graph, or of graphs of one plan, must not overlap on different streams. */
MUON_API muon_status muon_graph_launch(const muon_graph* graph, void* stream);
/* Number of nodes in the captured graph (one per kernel launch). */
MUON_API muon_status muon_graph_node_count(const muon_graph* graph, int64_t* nodes);
/* Free the graph; the caller makes sure no launch of it is still running. */
MUON_API void muon_graph_destroy(muon_graph* graph);

/* ---- a step that allocates nothing ------------------------------------------------------ */

/* Bytes of the library's own static device scratch (one copy per GPU, held until the
 * process ends). */
#define MUON_NOALLOC_MAX_BYTES (64ull << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): muon_step_ex for every chunk, on one
 * stream, with the library's static scratch array on the current device as the workspace
 * instead of a bound one.  The plan need not be bound; it must need at most
 * MUON_NOALLOC_MAX_BYTES of workspace (muon_plan_workspace_bytes).  Each call clears the
 * part of the scratch the plan uses (with a kernel) and copies the plan's tables into it
 * (hipMemcpyAsync from the plan's host memory, which the plan owns), then runs the step;
 * config->pipeline is ignored (one stream).  Calls no hipMalloc or hipFree.  Every call
 * on one GPU shares that GPU's scratch and leaves its contents there: calls that overlap
 * on one GPU (different streams or threads) race, and the result O cannot be read back
 * (muon_plan_param_info refers to a bound workspace).  The first call on a device looks
 * the scratch's address up on that device.
 * Errors: INVALID_ARG (NULL plan, config as for muon_step_ex), WORKSPACE_TOO_SMALL (the
 * plan needs more than MUON_NOALLOC_MAX_BYTES), SHAPE, HIP. */
MUON_API muon_status muon_step_noalloc(const muon_plan* plan, const muon_step_config* config, void* stream);

/* ---- per-kernel timing (HIP events on the launching stream) --------------------------- */

#define MUON_KERNEL_MOMENTUM 0
#define MUON_KERNEL_NORM_FINALIZE 1
#define MUON_KERNEL_NORMALIZE 2
#define MUON_KERNEL_SYRK 3
#define MUON_KERNEL_SYRK_POLY 4
#define MUON_KERNEL_GEMM_AXPY 5
#define MUON_KERNEL_APPLY 6
#define MUON_KERNEL_NS_SMALL 7
#define MUON_KERNEL_ADAMW 8
/* the side-stream kernels of the two-stream step (muon_step_config.pipeline) */
#define MUON_KERNEL_MOMENTUM_SIDE 9
#define MUON_KERNEL_NORMALIZE_SIDE 10
#define MUON_KERNEL_APPLY_SIDE 11
/* the grouped launches of the small tiled chunks (all three products; the normalisation) */
#define MUON_KERNEL_NS_GROUPED 12
#define MUON_KERNEL_PREP_GROUPED 13
#define MUON_KERNEL_COUNT 14

/* Start recording a HIP event pair around every kernel launch of this plan (up to
 * `capacity` launches; later ones go unrecorded).  capacity = 0 stops recording.
 * Not for use while a graph is being captured. */
MUON_API muon_status muon_timing_enable(muon_plan* plan, int32_t capacity);
/* Wait for the recorded events and return, for one kernel kind, the summed duration
 * in milliseconds, the launch count and the summed algorithmic work of those launches
 * (FLOPs for the Newton–Schulz kernels, HBM bytes for the others).  Clears nothing. */
MUON_API muon_status muon_timing_read(muon_plan* plan, int32_t kernel, double* total_ms,
                             int64_t* launches, double* work);
/* Forget recorded launches (events are kept for reuse). */
MUON_API muon_status muon_timing_reset(muon_plan* plan);
MUON_API const char* muon_kernel_name(int32_t kernel);

/* ---- teardown and errors ------------------------------------------------------------ */

MUON_API void muon_plan_destroy(muon_plan* plan);
MUON_API const char* muon_status_string(muon_status status);
MUON_API const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMUON_MUON_H */
