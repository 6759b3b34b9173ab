/*
 * libdmuon_ns -- the owner-side Muon step on one MI355X (gfx950), C ABI.
 *
 * What the library computes.  For every matrix of a batch, independently:
 *   M' = beta M + G;  U = G + beta M' (Nesterov) or U = M';
 *   X  = U / (||U||_F + eps), taken on the short side (U^T when rows > cols);
 *   ns_steps times:  A = X X^T;  B = b A + c A A;  X = a X + B X;
 *   O  = X in the stored orientation;  W' = W (1 - lr wd) - lr s O,
 *   s  = sqrt(max(1, rows / cols)).
 * The pages describe this as the work of a matrix's single owner: it runs the
 * Newton-Schulz (NS) iteration and the optimizer update once, on the full
 * matrix (DMuon abstract, arXiv 2611.07084 listing; DMuon explainer on
 * gist.science, "Technische Samenvatting" section 2.1 Owner-Centric
 * Executiestrategie), on the momentum-aggregated gradient (explainer section 1
 * Probleemstelling), in the m x m Gram space of the short side with the
 * symmetric product X X^T computed as one triangle (explainer, second section
 * 2.1, Efficiente Gram Newton-Schulz Iteratie), with similar shapes batched to
 * amortise dispatch (same section, "Batching").  The user-facing form on the
 * pages is dmuon.Muon(model, lr=0.02, ns_steps=5, ...) (DMuon docs, section
 * "LLM 预训练").  The pages print no coefficients; the workloads use
 * (a, b, c) = (3.4445, -4.7750, 2.0315), beta = 0.95, lr = 0.02, 5 steps.
 *
 * Conventions shared by every entry point.
 *  - Every function returns a dmuon_status; no C++ exception crosses the ABI.
 *  - Matrices are dense, row-major, rows x cols, contiguous (leading
 *    dimension = cols).  Every device pointer must be 16-byte aligned.
 *  - "Device pointer" = memory of the HIP device current on the calling
 *    thread; pointer arrays themselves are HOST arrays, in the order of the
 *    plan's descriptors.
 *  - The caller owns every device buffer (gradients, momenta, parameters,
 *    outputs, workspace).  The step entry points allocate no device memory;
 *    they only enqueue work on `stream` (a hipStream_t, NULL = the default
 *    stream) and return.  Buffers must stay alive until the stream has passed
 *    that point.
 *  - Arguments are checked before anything is enqueued, and every host
 *    allocation of a call is made before its first enqueue: on an
 *    INVALID_ARG, UNSUPPORTED, WORKSPACE or ALLOC return nothing has been
 *    enqueued.  A launch failure returns DMUON_ERR_HIP (work enqueued before
 *    it may have run).
 *  - No buffer a call writes (momentum, parameter, output, workspace) may
 *    overlap any other buffer of the call, byte range against byte range;
 *    read-only inputs may overlap each other.  Violations are INVALID_ARG.
 *  - Results are deterministic: same plan, inputs and device give bitwise
 *    identical outputs (no floating-point atomics).
 *  - NaN and Inf in the inputs are not masked; they propagate.
 *  - Calls that share a workspace must not overlap in time; a plan may be
 *    shared by threads and streams if each call has its own workspace.
 */
#ifndef DMUON_NS_H
#define DMUON_NS_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DMUON_API __attribute__((visibility("default")))
#else
#define DMUON_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DMUON_OK = 0,
    DMUON_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad dtype, bad index */
    DMUON_ERR_UNSUPPORTED = -2, /* valid request outside the library's limits (e.g. a dim >= 2^30) */
    DMUON_ERR_WORKSPACE = -3,   /* workspace missing, too small or not 256-byte aligned */
    DMUON_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
    DMUON_ERR_ALLOC = -5        /* host allocation failed (nothing was enqueued) */
} dmuon_status;

typedef enum { DMUON_F32 = 0, DMUON_BF16 = 1 } dmuon_dtype;

/* One matrix of the batch.  grad_dtype selects the precision path: a bf16
 * gradient runs NS with bf16 MFMA operands and fp32 accumulation; an fp32
 * gradient runs NS in fp32 throughout.  param_dtype is the dtype of the
 * parameter (muon_step_batched) or of the output (ns_orthogonalize_batched).
 * Momentum buffers are always fp32. */
typedef struct {
    int64_t rows;        /* stored rows (output features), >= 1 */
    int64_t cols;        /* stored cols (input features), >= 1 */
    int32_t grad_dtype;  /* dmuon_dtype */
    int32_t param_dtype; /* dmuon_dtype */
} dmuon_matrix_desc;

/* Step hyper-parameters.  ns_steps >= 0 (0: O is the normalised U).
 * nesterov != 0 selects U = G + beta M'.  eps is added to the Frobenius norm. */
typedef struct {
    float lr;
    float beta;
    float weight_decay;
    float eps;
    float a, b, c;
    int32_t ns_steps;
    int32_t nesterov;
} dmuon_hparams;

typedef struct dmuon_plan dmuon_plan; /* opaque, host memory only, immutable once built */

/* How a bucket runs its Newton-Schulz iterations. */
typedef enum {
    DMUON_ALGO_AUTO = 0,  /* plan option: Gram space where it saves work, else short side */
    DMUON_ALGO_SHORT_SIDE = 1,
    /* The iteration carried in the m x m Gram space (DMuon explainer on
     * gist.science, second section 2.1 Efficiente Gram Newton-Schulz
     * Iteratie): X_k = P_k X_0 with A_0 = X_0 X_0^T and, per iteration,
     * Q = a I + b A + c A A, P <- Q P, A <- Q A Q.  All of these are
     * polynomials in A_0, hence symmetric and commuting, and each product is
     * computed on one triangle.  Every gram_restart iterations (and after the
     * last) the recurrence restarts from the actual iterate X = P X_0 with a
     * fresh Gram matrix X X^T: with A's rounding amplified by P^2 along
     * directions that X_0 barely spans, the Gram space in bf16 resolves small
     * singular values far worse than the short side, and restarts bound that
     * loss.  A segment of L iterations costs 3 m^2 n + (4 L - 3) m^3 flops
     * (the short side: 3 m^2 n + m^3 per iteration), so 5 iterations as 3 + 2
     * take 6 m^2 n + 14 m^3 instead of 15 m^2 n + 5 m^3: cheaper whenever n > m
     * (as 2 + 2 + 1, 9 m^2 n + 11 m^3: cheaper once n > 1.5 m). */
    DMUON_ALGO_GRAM_SPACE = 2
} dmuon_algo;

/* A per-shape configuration (tuning cache entry): how the plan runs a bucket of
 * the given path and padded dims (the padded dims the default tile granularity
 * gives).  The pages autotune kernel configurations per matrix shape and cache
 * the result, and balance work by measured per-shape cost (DMuon explainer on
 * gist.science, sections 2.3 and 2.4); muon_autotune measures these entries on
 * the device, and muon_plan_ex applies them. */
#define DMUON_XCD_REMAP_DEFAULT 0xFFFFFFFFu
typedef struct {
    int32_t path;            /* DMUON_BF16 | DMUON_F32 (key) */
    int32_t tile;            /* output tile edge: bf16 128 or 256 (dividing both padded dims), fp32 64;
                                0: the default granularity */
    int64_t padded_m;        /* key: padded short side */
    int64_t padded_n;        /* key: padded long side */
    int32_t algo;            /* dmuon_algo for the bucket; DMUON_ALGO_AUTO: the plan option's rule.
                                DMUON_ALGO_GRAM_SPACE is accepted on the bf16 path only; under
                                the DMUON_ALGO_AUTO plan option it applies only to a bucket that
                                the automatic rule would run in the Gram space (entries are keyed
                                by padded dims, so the bucket's real members may differ from
                                those it was measured on), else the bucket keeps the short side */
    int32_t gram_restart;    /* Gram-space iterations between restarts; 0: the plan option's */
    uint32_t xcd_remap;      /* bf16 path: bit per phase (1 Gram, 2 square, 4 B X, 8 prod) whose launch
                                gives each XCD a contiguous run of the bucket's tiles (neighbouring tiles
                                share operand panels in that XCD's L2); DMUON_XCD_REMAP_DEFAULT: B X only */
    int32_t apply_pass;      /* 0 (default): the kernel that ends the iteration writes the update (or
                                the output) and X is never written back: in a resident bucket the
                                resident kernel, for every member; otherwise, on the bf16 path, the
                                last B X launch's epilogue, for every member with a bf16 parameter
                                (output) and cols a multiple of 8;
                                1: a separate elementwise pass writes it from the final X for every
                                member, as it does for the other members.  The two give identical
                                bits; other values are INVALID_ARG */
    double cost_ms_per_matrix; /* measured time of one matrix's Newton-Schulz iterations; when every
                                  bucket of a plan has one > 0, buckets are ordered by count times it
                                  instead of the dense cost */
} dmuon_tune_entry;

typedef struct {
    int32_t algo;         /* dmuon_algo; DMUON_ALGO_AUTO (the default) picks the Gram space for
                             bf16 buckets with padded n > padded m and padded m >= 1024 whose
                             members all have n >= 3 m (in bf16 the Gram space resolves small
                             singular values worse; there it saves the most work for the
                             least accuracy), else the short side;
                             DMUON_ALGO_GRAM_SPACE forces it on every bf16 bucket;
                             DMUON_ALGO_SHORT_SIDE forces the short side everywhere.  fp32
                             buckets always run the short side. */
    int32_t gram_restart; /* Gram-space iterations between restarts, >= 1; 0: the default per
                             bucket, 2 for a padded short side up to 1024 and 3 above (the
                             more accurate of the two on each side of that size, measured
                             against the fp64 reference).  Larger values save m^2 n work and
                             lose accuracy on ill-conditioned inputs; 1 is the short side. */
    const dmuon_tune_entry* tuned; /* host array of per-shape entries (NULL: none); for each bucket
                             the first entry with its key applies, entries matching no bucket are
                             ignored.  Only read during the call. */
    int32_t tuned_count;
} dmuon_plan_opts;

/* Build the batch plan (host only, no device work): step one of the owner's
 * work, which batches matrices of similar shape so that their Newton-Schulz
 * iterations run jointly and amortise kernel dispatch (DMuon explainer on
 * gist.science, second section 2.1, "Batching"), and orders the work by its
 * computational cost, as owners are balanced by cost (DMuon abstract; the
 * explainer's section 2.3 on load balancing).  Per matrix: m = min(rows,
 * cols), n = max(rows, cols), transposed = rows > cols (square matrices are
 * not transposed).  Tile granularity g = 64 on the fp32 path; on the bf16 path
 * g = 128 when m <= 128, else 256.  Padded dims are m, n rounded up to g (the
 * padding is zero and leaves the result unchanged); the GEMM tile is g unless
 * a tuned entry picks another that divides the padded dims.  Matrices with the same
 * (path, padded m, padded n) share a bucket and run jointly.  Buckets are
 * ordered by executed cost, the sum of 4 m_pad^2 n_pad + 2 m_pad^3 over their
 * members (or the measured cost, with tuned entries: see dmuon_tune_entry),
 * descending, ties in order of first appearance; members keep input order.
 * count == 0 gives an empty plan.  Errors: INVALID_ARG for count < 0,
 * descs == NULL with count > 0, out == NULL, a dim < 1 or an unknown dtype;
 * UNSUPPORTED for a dim >= 2^30, a side > 2^27 with a bf16 gradient, or a
 * bucket whose B X launch would need more than 2^31 - 1 tiles; ALLOC
 * on host allocation failure.
 * On success *out owns the plan; release it with muon_plan_destroy. */
DMUON_API dmuon_status muon_plan(const dmuon_matrix_desc* descs, int32_t count, dmuon_plan** out);

/* muon_plan with options (opts == NULL: the defaults).  INVALID_ARG also for
 * an unknown opts->algo, opts->gram_restart < 0, tuned_count < 0 (or > 0 with
 * tuned == NULL), or an applied entry with a tile that does not divide the
 * bucket's padded dims, an unknown algo, the Gram space on the fp32 path, a
 * negative restart, remap bits beyond the four phases or reserved != 0. */
DMUON_API dmuon_status muon_plan_ex(const dmuon_matrix_desc* descs, int32_t count, const dmuon_plan_opts* opts,
                                    dmuon_plan** out);

/* Bytes of device workspace a step or orthogonalisation with this plan needs
 * (0 for an empty plan).  The workspace holds the per-bucket X (two copies),
 * A and B operands (and, for Gram-space buckets, three more m x m matrices
 * per member), per-matrix norms and a small descriptor table;
 * its contents need no initialisation and are garbage after a call. */
DMUON_API dmuon_status muon_plan_workspace_bytes(const dmuon_plan* plan, size_t* bytes);

/* Number of matrices and buckets of the plan. */
DMUON_API dmuon_status muon_plan_info(const dmuon_plan* plan, int32_t* count, int32_t* num_buckets);

/* Per-matrix plan entry: bucket index (execution order), slot within the
 * bucket, transposed flag, padded short/long dims, and the dense NS cost
 * 4 m^2 n + 2 m^3 of the real shape, the cost by which the work is balanced
 * (DMuon abstract; DMuon explainer on gist.science, section 2.3).  The cost
 * is an exact integer (int64), and the slot is reported as well, for tests
 * that check the plan element by element.  Any output pointer may be NULL.
 * INVALID_ARG for idx outside [0, count). */
DMUON_API dmuon_status muon_plan_query(const dmuon_plan* plan, int32_t idx, int32_t* bucket, int32_t* slot,
                             int32_t* transposed, int64_t* padded_m, int64_t* padded_n,
                             int64_t* ns_cost);

/* Per-bucket plan entry: precision path (dmuon_dtype of its gradients),
 * padded dims, member count and tile granularity. */
DMUON_API dmuon_status muon_plan_bucket(const dmuon_plan* plan, int32_t bucket, int32_t* path,
                              int64_t* padded_m, int64_t* padded_n, int32_t* count,
                              int32_t* tile);

/* The dmuon_algo a bucket runs (DMUON_ALGO_SHORT_SIDE or DMUON_ALGO_GRAM_SPACE) and its
 * iterations per Gram-space segment (1 on the short side).  A call with ns_steps
 * iterations runs Gram-space buckets as segments of gram_restart iterations, the
 * last one shorter if needed; if |a|^gram_restart > 2^64 (P grows like a^k along
 * directions that X_0 barely spans) the call runs them on the short side instead.
 * Either pointer may be NULL. */
DMUON_API dmuon_status muon_plan_bucket_algo(const dmuon_plan* plan, int32_t bucket, int32_t* algo,
                                             int32_t* gram_restart);

/* Whether a bucket runs resident: every short-side iteration of each of its
 * matrices in one workgroup, with the matrix held in LDS, one launch for all
 * such buckets of a call (1), or as grouped tiled launches per phase (0).
 * Resident buckets are the bf16 buckets of padded short side 128 and padded
 * long side at most 512 that run the short side; their product launches would
 * be latency-bound.  Same arithmetic and roundings either way. */
DMUON_API dmuon_status muon_plan_bucket_resident(const dmuon_plan* plan, int32_t bucket, int32_t* resident);

/* Where a step (or orthogonalisation) with ns_steps iterations writes matrix
 * idx's update (output): 1 from the kernel that ends its iteration, which
 * then never writes the final X back, 0 in the separate elementwise pass.
 * The owner applies the update right after the matrix's Newton-Schulz
 * iteration (DMuon abstract; DMuon explainer on gist.science, section 2.1
 * Owner-Centric Executiestrategie); written by the kernel that ends the
 * iteration, the orthogonalised matrix makes no round trip through memory.
 * With ns_steps > 0 and the bucket's apply_pass 0: the resident kernel takes
 * every member of a resident bucket (muon_plan_bucket_resident), any
 * parameter type and shape; the last B X launch's epilogue takes a bf16
 * parameter (output) with cols a multiple of 8 in a bucket of tiled bf16
 * launches.  The two routes give identical bits.  Host only.  Errors:
 * INVALID_ARG (null plan or fused, idx out of range, ns_steps < 0). */
DMUON_API dmuon_status muon_plan_update_fused(const dmuon_plan* plan, int32_t idx, int32_t ns_steps,
                                              int32_t* fused);

/* The configuration a bucket runs with, as a tuning entry (key, tile, algo,
 * restart, remap bits; cost_ms_per_matrix as given to the plan, else 0). */
DMUON_API dmuon_status muon_plan_bucket_config(const dmuon_plan* plan, int32_t bucket, dmuon_tune_entry* out);

/* Workspace muon_autotune needs for these descs and opts (the largest of its
 * trial plans, the whole batch with every bucket in its largest form included). */
DMUON_API dmuon_status muon_autotune_workspace_bytes(const dmuon_matrix_desc* descs, int32_t count,
                                                     const dmuon_plan_opts* opts, size_t* bytes);

/* Measure candidate configurations of every bucket that muon_plan_ex(descs,
 * count, opts) forms, ignoring opts->tuned, and write the fastest for each into
 * out[0 .. *out_count) (bucket order of that plan).  Each candidate runs the
 * bucket's members alone through ns_orthogonalize_batched: one untimed call,
 * then reps (>= 1) calls timed with HIP events on `stream`.  Candidates: on the
 * bf16 path tiles 256 (where it divides the padded dims) and 128, remap bits 0,
 * 4 and 15; the short side, and the Gram space with opts' restart where the
 * plan options would allow it (forced forms are kept); fp32 buckets and
 * resident ones (muon_plan_bucket_resident) have one candidate.  Then, if some bucket picked the Gram space, the whole batch is
 * timed twice the same way: with the picked entries, and with every Gram-space
 * entry replaced by its bucket's fastest short-side one.  The faster set is
 * returned.  The Gram-space buckets add product launches that the other
 * buckets lack, and in batches of small matrices that latency can cost more
 * than the Gram space saves.  inputs / outputs: device pointers as for ns_orthogonalize_batched
 * (trial data; outputs are overwritten).  The call blocks until the trials
 * are done.  Errors: INVALID_ARG (also out_capacity below the bucket count),
 * WORKSPACE (below muon_autotune_workspace_bytes), HIP, ALLOC. */
DMUON_API dmuon_status muon_autotune(const dmuon_matrix_desc* descs, int32_t count, const dmuon_plan_opts* opts,
                                     const void* const* inputs, void* const* outputs, int32_t ns_steps,
                                     float a, float b, float c, int32_t reps, void* workspace,
                                     size_t workspace_bytes, void* stream, dmuon_tune_entry* out,
                                     int32_t out_capacity, int32_t* out_count);

/* Release a plan (NULL is a no-op). */
DMUON_API void muon_plan_destroy(dmuon_plan* plan);

/* One fused Muon step over every matrix of the plan: the owner's whole work
 * on each of its matrices -- the Newton-Schulz iteration and the optimizer
 * update, once, on the full matrix (DMuon abstract; DMuon explainer on
 * gist.science, section 2.1 Owner-Centric Executiestrategie) -- applied to
 * the momentum-aggregated gradient (explainer, section 1).  Momentum (in
 * place in momenta[i], fp32), normalisation, ns_steps NS iterations on the
 * short side (or in the Gram space, per bucket: dmuon_algo), and the
 * in-place parameter update of params[i] (param_dtype; bf16 results are
 * rounded to nearest even once, from fp32), written by the kernel that
 * ends the iteration (resident kernel, or last B X launch) where
 * muon_plan_update_fused says so, else by an elementwise pass.
 *   grads[i]   device, rows x cols, grad_dtype, read only, must not alias
 *   momenta[i] device, rows x cols, fp32, read and written
 *   params[i]  device, rows x cols, param_dtype, read and written
 *   hp         host, step hyper-parameters (ns_steps >= 0)
 *   workspace  device, >= muon_plan_workspace_bytes, 256-byte aligned
 *   stream     hipStream_t (NULL = default stream)
 * Errors: INVALID_ARG (null plan/hp/array/pointer, misaligned pointer,
 * ns_steps < 0, overlapping buffers), WORKSPACE, ALLOC, HIP. */
DMUON_API dmuon_status muon_step_batched(const dmuon_plan* plan, const void* const* grads,
                               float* const* momenta, void* const* params,
                               const dmuon_hparams* hp, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Orthogonalise every matrix of the plan without momentum or update: the
 * Newton-Schulz iteration alone, which drives the singular values of each
 * input towards a uniform spectrum (DMuon explainer on gist.science, section
 * 1), on the short side or in the m x m Gram space with X X^T computed as one
 * triangle (explainer, second section 2.1).
 * outputs[i] = NS(inputs[i]) with ns_steps iterations of coefficients
 * (a, b, c) after normalisation by ||input||_F + eps, in the input's own
 * orientation.  inputs[i] are device rows x cols in grad_dtype (read only);
 * outputs[i] are device rows x cols in param_dtype and must not alias the
 * inputs.  Errors as for muon_step_batched. */
DMUON_API dmuon_status ns_orthogonalize_batched(const dmuon_plan* plan, const void* const* inputs,
                                      void* const* outputs, int32_t ns_steps, float a, float b,
                                      float c, float eps, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---- the step for callers that cannot allocate ------------------------------
 * For callers that cannot allocate device memory or hand over a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The step of muon_step_batched, with its workspace taken from a
 * static device array of DMUON_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on until the process ends; the call itself
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * The caller passes the inputs and outputs as for muon_step_batched.  Every
 * call on a GPU shares that GPU's array, so calls on one GPU that overlap in
 * time (other streams, other threads) race and must be serialised by the
 * caller.  Errors as for muon_step_batched; WORKSPACE when the plan needs more
 * than DMUON_NOALLOC_SCRATCH_BYTES (muon_plan_workspace_bytes), UNSUPPORTED
 * for a device index beyond 255, HIP if the array's address cannot be found. */
#define DMUON_NOALLOC_SCRATCH_BYTES (64u << 20)
DMUON_API dmuon_status muon_step_batched_noalloc(const dmuon_plan* plan, const void* const* grads,
                                                 float* const* momenta, void* const* params,
                                                 const dmuon_hparams* hp, void* stream);

/* ---- AdamW for the parameters that do not go through Muon -------------------
 * The optimizer takes a separate AdamW learning rate for the parameters that
 * its predicate does not route to Muon (DMuon project documentation,
 * quick-start snippet and the VLA/VLM paragraph); the other hyper-parameters
 * are the caller's.  step is the 1-based count of steps including this one. */
typedef struct {
    double lr;
    double beta1, beta2; /* double: 1 - beta loses 3 digits in float (1 - (float)0.999 is off by 1.3e-5) */
    double eps;
    double weight_decay;
    int64_t step;
} dmuon_adamw_hparams;

/* One AdamW step on each of `count` tensors, updated in place:
 *   p <- p (1 - lr wd);  m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr m / (1 - beta1^step) / (sqrt(v / (1 - beta2^step)) + eps)
 * Every array holds `count` entries (host arrays of device pointers):
 * params[i] (param_dtypes[i]: DMUON_F32 | DMUON_BF16, stored rounded to nearest
 * even) and grads[i] (grad_dtypes[i], read only) of numels[i] elements,
 * exp_avgs[i] / exp_avg_sqs[i] fp32 moments of the same length.  Tensors are
 * flat; numels[i] may be 0 (skipped).  The four buffers of a tensor are
 * distinct and 16-byte aligned.  Arithmetic is fp32 on the device; 1 - beta,
 * 1 - lr wd and the bias corrections are formed on the host in double and
 * handed to the device rounded once to fp32.  Enqueued on `stream`;
 * nothing is allocated.  Errors: INVALID_ARG (null or misaligned pointer,
 * unknown dtype, negative numel, aliasing buffers, step < 1, beta outside
 * [0, 1), eps <= 0, non-finite lr or weight decay), HIP. */
DMUON_API dmuon_status adamw_step_batched(int32_t count, const int64_t* numels, const int32_t* param_dtypes,
                                          const int32_t* grad_dtypes, void* const* params,
                                          const void* const* grads, float* const* exp_avgs,
                                          float* const* exp_avg_sqs, const dmuon_adamw_hparams* hp,
                                          void* stream);

/* ---- profiling ------------------------------------------------------------
 * The step of muon_step_batched, with a HIP event recorded on `stream` at each
 * phase boundary so that the caller can time every kernel phase live:
 * events[0] before the first launch, then one event after each phase, the
 * phases being: prep (momentum, cast, norms), then for every iteration four
 * phases -- Gram (short-side buckets; Gram-space buckets in the first
 * iteration only), square (every bucket), products (the Gram-space buckets'
 * P and A updates), B X (short-side buckets; Gram-space buckets' O = P X_0 in
 * the last iteration) -- each a set of grouped launches, some possibly empty,
 * then the update.  Needs num_events >= muon_step_event_count(hp->ns_steps)
 * event handles (hipEvent_t, e.g. from dmuon_events_create); nothing is
 * synchronised.  Errors as for muon_step_batched, INVALID_ARG for too few or
 * NULL events. */
DMUON_API dmuon_status muon_step_batched_profiled(const dmuon_plan* plan, const void* const* grads,
                                                  float* const* momenta, void* const* params,
                                                  const dmuon_hparams* hp, void* workspace,
                                                  size_t workspace_bytes, void* stream,
                                                  void* const* events, int32_t num_events);

/* Events muon_step_batched_profiled records: 3 + 4 ns_steps (-1 if ns_steps < 0 or
 * the count would not fit an int32). */
DMUON_API int32_t muon_step_event_count(int32_t ns_steps);

/* Create n HIP events (timing enabled) into events[0..n); the caller destroys
 * them with dmuon_events_destroy.  HIP on failure (none is left created). */
DMUON_API dmuon_status dmuon_events_create(int32_t n, void** events);

/* Milliseconds between two recorded events; waits for `stop` to complete. */
DMUON_API dmuon_status dmuon_events_elapsed_ms(void* start, void* stop, float* ms);

/* Destroy n events created by dmuon_events_create (NULL entries skipped). */
DMUON_API dmuon_status dmuon_events_destroy(int32_t n, void** events);

/* ---- measurement ------------------------------------------------------------
 * Two kernels that measure the practical ceilings the benchmark reports next
 * to the published peaks, on the same device in the same run (the project's
 * benchmark section states hardware, precision and method for every figure:
 * DMuon project documentation, "基准测试").  Both only enqueue on `stream`.
 *
 * dmuon_diag_copy: copy `bytes` (a multiple of 16, > 0) from src to dst
 * (device, 16-byte aligned, not overlapping) with streaming 16-byte accesses:
 * the HBM read + write rate a bandwidth-bound pass can reach.  INVALID_ARG for
 * bad pointers or sizes, HIP on a launch failure. */
DMUON_API dmuon_status dmuon_diag_copy(void* dst, const void* src, size_t bytes, void* stream);

/* dmuon_diag_mfma: `blocks` workgroups of 512 threads, each wave running
 * `iters` (a multiple of 8) rounds of 8 independent v_mfma_f32_32x32x16_bf16
 * (32768 flops each) on pseudo-random bf16 operands that change every
 * instruction, with no memory traffic: 8 * blocks * iters * 8 * 32768 flops,
 * the matrix-core rate the chip sustains within its power limit.  out: device,
 * blocks * 512 floats (per-thread sums that keep the products live).
 * INVALID_ARG for bad arguments, HIP on a launch failure. */
DMUON_API dmuon_status dmuon_diag_mfma(float* out, int32_t blocks, int32_t iters, void* stream);

/* dmuon_diag_mix: the byte mix of one of the library's bandwidth-bound
 * passes on flat contiguous arrays of n elements (n > 0, a multiple of 4), so
 * that a pass can be compared with what its own traffic reaches untiled.
 * kind 0 (prep): reads a (bf16, n) and b (fp32, n), writes b and c (bf16, n):
 * 12 bytes an element.  kind 1 (apply): reads a and b (bf16, n), writes b; c
 * unused: 6 bytes.  kind 2 (AdamW): reads a and b (bf16, n) and c (fp32,
 * 2 n), writes a and c: 22 bytes.  Device pointers, 16-byte aligned, regions
 * not overlapping; the arrays' contents are overwritten with bounded values.
 * INVALID_ARG for bad arguments, HIP on a launch failure. */
DMUON_API dmuon_status dmuon_diag_mix(int32_t kind, void* a, void* b, void* c, size_t n, void* stream);

/* dmuon_diag_clock: one wave that records `samples` (>= 2) pairs (shader-clock
 * cycles, 100 MHz wall-clock ticks) into out (device, 2 * samples int64), the
 * k-th pair k * interval wall ticks (>= 1) after the first; it runs for
 * samples x interval ticks, at most 1e10 (100 s).  Launched on a stream of its
 * own beside other work, the pairs give the shader clock of the XCD it ran on
 * while that work ran.  INVALID_ARG for bad arguments, HIP on a launch
 * failure. */
DMUON_API dmuon_status dmuon_diag_clock(long long* out, int32_t samples, int32_t interval, void* stream);

/* Static, human-readable name of a status code. */
DMUON_API const char* dmuon_status_string(dmuon_status status);

/* Library version, "major.minor.patch". */
DMUON_API const char* dmuon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_NS_H */
