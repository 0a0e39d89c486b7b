/*
 * dmuon.h -- C ABI of libdmuon: batched Gram Newton-Schulz orthogonalisation
 * and the fused Muon optimizer step on one AMD Instinct MI355X (gfx950).
 *
 * Source of the method: "DMuon: Efficient Distributed Muon Training with
 * Near-Adam Overhead", as summarised on gist.science (Portuguese and French
 * technical summaries) and on shd-paper.top (with the authors' English
 * abstract).  Sections cited below are those of the gist.science technical
 * summary.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Matrices are dense, row-major, contiguous: element (r, c) of a rows x cols
 *    matrix sits at offset r * cols + c.  Device pointers must be 16-byte
 *    aligned for the vectorised path; other alignments fall back to a slower
 *    element-wise path with the same results.
 *  - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16).
 *  - "stream" is a hipStream_t passed as void*; NULL selects the null stream.
 *    Every compute call only enqueues work on that stream and returns without
 *    synchronising; results are valid once the stream reaches that point.
 *  - The caller owns every matrix, gradient and momentum buffer and must keep
 *    them alive until the enqueued work completes.  The library owns plans and
 *    their device workspace, and never frees caller memory.
 *  - Arguments are validated before anything is enqueued: a call that returns
 *    an error has enqueued nothing.  No C++ exception crosses this boundary.
 *    dmuon_last_error() returns a thread-local message for the last failure.
 *  - NaN or Inf inputs are not detected; they propagate to the outputs.
 *  - Calls that share a plan or the implicit workspace must be ordered on one
 *    stream (or externally synchronised): the workspace is reused per call.
 */
#ifndef DMUON_H
#define DMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  DMUON_OK = 0,
  DMUON_EINVAL = -1,       /* bad argument (null pointer, non-positive size, ...) */
  DMUON_EUNSUPPORTED = -2, /* valid request the library does not implement        */
  DMUON_EHIP = -3,         /* a HIP runtime call failed; see dmuon_last_error()   */
  DMUON_ENOMEM = -4,       /* device workspace allocation failed or over the cap  */
  DMUON_EPLAN = -5         /* the plan does not match the call                    */
};

/* Element types of caller matrices. */
enum { DMUON_BF16 = 0, DMUON_F32 = 1 };

/* Arithmetic used for the matrix products.
 *   AUTO : for bf16 inputs, per recurrence bucket (short side k): F32 when
 *          k <= 128 and some member has long side < 2k (16-bit Gram state
 *          misses the accuracy bar on small near-square matrices); otherwise
 *          F16 when the host-side range check of the recurrence passes
 *          (always for the quintic coefficients; it fails when a state would
 *          overflow fp16, or when Q's power-of-two scale, which keeps its
 *          fastest-growing direction in range, would exceed 2^12 and push
 *          the converged directions below fp16's normal range -- e.g. the
 *          cubic (1.5, -0.5, 0) from 43 steps on), else BF16.  F32 for
 *          f32 inputs.
 *   F16  : fp16 MFMA operands, fp32 accumulation.  bf16 inputs are converted
 *          exactly (power-of-two scaling); the m x m state is kept in fp16
 *          with a fixed power-of-two scale.
 *   BF16 : bf16 MFMA operands and bf16 state, fp32 accumulation.
 *   F32  : fp32 MFMA, fp32 state (f32 inputs only). */
enum { DMUON_PREC_AUTO = 0, DMUON_PREC_F16 = 1, DMUON_PREC_BF16 = 2, DMUON_PREC_F32 = 3 };

/* Factor applied to the orthogonalised update in dmuon_step.
 *   SQRT_RATIO : sqrt(max(1, rows / cols)) of the caller's (rows, cols).
 *   NONE       : 1. */
enum { DMUON_SCALE_SQRT_RATIO = 0, DMUON_SCALE_NONE = 1 };

/* ---------------------------------------------------------------------------
 * dmuon_ns_batched -- Newton-Schulz orthogonalisation of `batch` same-shape
 * bf16 matrices, in place.
 *
 * Defines the operation of DMuon's Gram-space iteration (technical summary
 * section 2.2: the recurrence runs on G = X X^T, m x m, instead of the m x n
 * matrix; symmetric products compute only the lower triangle; matrices of like
 * shape are processed together).  For each matrix M (rows m x cols n):
 *   X0 = M' / (||M||_F + 1e-7), where M' = M if m <= n, else M^T (short side
 *   k = min(m, n));  A = X0 X0^T;  Q = I;
 *   repeat `steps` times:  P = a I + b A + c A^2;  A = P A P;  Q = P Q;
 *   result = Q X0 (transposed back when m > n), written over M.
 *
 *  ptrs   host array of `batch` device pointers, each an m x n bf16 matrix.
 *         The matrices must not overlap.  The array itself is read during the
 *         call only.
 *  m, n   rows and cols of every matrix (> 0).
 *  batch  number of matrices (> 0).
 *  steps  number of iterations (>= 0; 0 returns the normalised input).
 *  a,b,c  polynomial coefficients, e.g. the quintic (3.4445, -4.7750, 2.0315).
 *  stream hipStream_t as void*.
 * Precision is DMUON_PREC_AUTO.  Device workspace comes from a per-device cache
 * that grows on demand with hipMalloc (geometrically, at least 1.5x).  An
 * outgrown buffer is retired, never freed behind the caller's back: work still
 * enqueued, or a HIP graph that captured an earlier call, may address it.
 * Retired buffers are released only by dmuon_release_workspace().  Such a
 * call may be captured in a HIP graph once the cache has grown for its shape
 * (make one call of that shape first); a call that would have to grow the
 * cache while its stream is being captured fails with EUNSUPPORTED and
 * enqueues nothing.
 * Errors: EINVAL for a null ptrs array or null entry, m/n/batch <= 0,
 * steps < 0; ENOMEM if the workspace cannot grow; EUNSUPPORTED for growth
 * during capture; EHIP on a launch failure.
 * ------------------------------------------------------------------------- */
int dmuon_ns_batched(void* const* ptrs, int64_t m, int64_t n, int64_t batch,
                     int steps, float a, float b, float c, void* stream);

/* Bytes of the statically allocated device scratch of
 * dmuon_ns_batched_noalloc (128 MiB, held by every device the library runs
 * on until the process ends). */
#define DMUON_NOALLOC_SCRATCH_BYTES (128ull * 1024ull * 1024ull)

/* dmuon_ns_batched_noalloc -- dmuon_ns_batched for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, operation, launch sequence and results as
 * dmuon_ns_batched (bitwise), but its workspace is a file-scope device array
 * of DMUON_NOALLOC_SCRATCH_BYTES (one per device) instead of the implicit
 * cache: the call never calls hipMalloc, hipFree or a synchronising function.
 * The first call on a device looks up the array's address there
 * (hipGetSymbolAddress); later calls reuse it.
 * All calls on one device share that device's array, and it keeps the last
 * call's contents (nothing in it needs to start at zero): calls that can
 * overlap on one device -- on different streams without ordering, or from
 * several threads -- race on it and must be ordered by the caller.
 * Errors: those of dmuon_ns_batched, and ENOMEM (nothing enqueued) when the
 * batch needs more workspace than the array holds -- for example one
 * 4096 x 4096 matrix (224 MiB of workspace) does not fit; one 2048 x 8192
 * matrix (104 MiB) or eight 1024 x 1024 matrices (112 MiB) do. */
int dmuon_ns_batched_noalloc(void* const* ptrs, int64_t m, int64_t n, int64_t batch,
                             int steps, float a, float b, float c, void* stream);

/* Release the implicit workspace of the current device (its live buffer and
 * every retired one): synchronises the device, then frees them.  The next
 * plan-free call allocates again.  A HIP graph that captured a plan-free call
 * must not be replayed after this.  EHIP if the synchronisation or a free
 * fails. */
int dmuon_release_workspace(void);

/* Sizes of the implicit workspace of the current device: the live buffer's
 * bytes, the retired buffers' total bytes and their number (each output
 * nullable).  Host bookkeeping only; EHIP if the current device cannot be
 * read. */
int dmuon_workspace_info(int64_t* live_bytes, int64_t* retired_bytes, int32_t* retired_count);

/* Same operation on f32 matrices, computed with fp32 MFMA (DMUON_PREC_F32). */
int dmuon_ns_batched_f32(void* const* ptrs, int64_t m, int64_t n, int64_t batch,
                         int steps, float a, float b, float c, void* stream);

/* Same operation with an explicit element type (DMUON_BF16 / DMUON_F32) and
 * precision (DMUON_PREC_*).  DMUON_PREC_F32 needs f32 input; F16 and BF16
 * need bf16 input (EUNSUPPORTED otherwise). */
int dmuon_ns_batched_ex(void* const* ptrs, int64_t m, int64_t n, int64_t batch,
                        int dtype, int precision, int steps, float a, float b,
                        float c, void* stream);

/* ---------------------------------------------------------------------------
 * Plans: shape bucketing, tile choice and workspace for repeated steps.
 *
 * Follows the batching and autotuning passages of DMuon (technical summary
 * section 2.2, batching bullet; section 2.4: a tile configuration is chosen
 * per matrix shape and cached for later steps).  The Gram product and the
 * final product are grouped by the caller's exact (rows, cols), since a
 * matrix with more rows than columns is processed transposed; the k x k
 * recurrence (k = min(rows, cols)) is grouped by k alone, so matrices of
 * different long side or orientation share its launches.  The tile
 * configuration of every launch comes from a table keyed by k and the number
 * of matrices in the bucket (built in; a JSON file named by opts->tune_path or
 * the DMUON_TUNE_TABLE environment variable -- for example one written by
 * dmuon_tune -- overrides it).
 * ------------------------------------------------------------------------- */
typedef struct dmuon_plan dmuon_plan_t; /* opaque, library-owned */

typedef struct dmuon_plan_opts {
  int precision;         /* DMUON_PREC_*; default AUTO                         */
  int scale_mode;        /* DMUON_SCALE_*; default SQRT_RATIO                  */
  int no_device;         /* 1: plan on the host only (no workspace, no HIP call);
                            such a plan can be described but not stepped      */
  float eps;             /* added to the Frobenius norm; <= 0 selects 1e-7     */
  int64_t max_workspace; /* bytes; 0 = no cap.  Over the cap -> ENOMEM        */
  const char* tune_path; /* JSON tune table or NULL                           */
  int form;              /* DMUON_FORM_*; default AUTO                         */
  float pad_ratio;       /* similar-shape batching (technical summary section
                            2.2, batching bullet): short sides within a factor
                            1 + pad_ratio share one recurrence bucket, its size
                            the largest of them rounded up to 64 (when that
                            stays within the factor) with zero padding.  0
                            (default) batches equal short sides only; at most
                            1.  fp32 buckets are not padded.  Results are
                            those of the unpadded matrices: zero rows add zero
                            eigenvalues, which never mix with the others     */
  int storage;           /* DMUON_STORAGE_*; default AUTO                      */
  int fused;             /* DMUON_FUSED_*; default AUTO                        */
} dmuon_plan_opts;

/* Storage of the symmetric k x k states of a GRAM bucket (A, P, R, Q; the
 * technical summary, section 2.2, computes only their lower triangle):
 *   FULL : both triangles are written (the products mirror each lower tile).
 *   AUTO : only the lower triangle of tile x tile blocks is written, and the
 *          products read the rest of a row panel transposed from the stored
 *          blocks below the diagonal, wherever every product of the bucket
 *          runs the direct-load kernel (16-bit products, tiles of 128 or 256
 *          covering every dimension exactly); FULL elsewhere.  Results are
 *          bitwise identical to FULL: the same values reach the same MFMAs
 *          in the same order.  The state buffers are library workspace, so
 *          the choice is invisible to the caller. */
enum { DMUON_STORAGE_AUTO = 0, DMUON_STORAGE_FULL = 1 };

/* Kernel of a GRAM bucket with short side k <= 128 (the batching and
 * occupancy case of the technical summary, section 2.2: many small matrices):
 *   AUTO : when the bucket runs fp16 state (DMUON_PREC_F16, or AUTO for wide
 *          members), its members are bf16, not transposed (rows <= cols)
 *          and steps is 1 .. 64, one launch runs the whole map -- Gram
 *          product, every recurrence step and the final product (or the
 *          update) -- with one workgroup per matrix and the k x k states in
 *          LDS, up to 256 matrices (one per CU) per launch.  The momentum
 *          pass of dmuon_step stays a launch of its own (per 64 matrices).
 *          The arithmetic is that of the grouped kernels (same operand
 *          types, scales and accumulation precision); the summation order
 *          differs, so results agree to rounding, not bitwise.  A group of
 *          at most 64 matrices of short side above 64 runs the map as two
 *          launches instead (Gram product and recurrence, then the final
 *          product with one workgroup per 128 output columns), so that a
 *          small batch occupies more CUs; the results are the same bits.
 *   OFF  : the grouped product kernels, as for every other bucket.
 *   ONE  : the fused kernel, always as one launch.
 *   SPLIT: the fused kernel, always as the two launches. */
enum { DMUON_FUSED_AUTO = 0, DMUON_FUSED_OFF = 1, DMUON_FUSED_ONE = 2, DMUON_FUSED_SPLIT = 3 };

/* Form of the iteration per recurrence bucket (a bucket is the matrices of one
 * short side k):
 *   GRAM     : the k x k Gram-space recurrence (technical summary section
 *              2.2), then one final product.
 *   STANDARD : the plain iteration on the k x n matrix every step:
 *              A = X X^T, X <- a X + (b A + c A^2) X.  Same flops as GRAM
 *              when n = k, more when n > k; it never forms Q, so it does not
 *              amplify rounding noise in the Gram spectrum.  16-bit buckets
 *              only: fp32 buckets (f32 data, or near-square k <= 128 under AUTO
 *              precision) always run GRAM.
 *   AUTO     : STANDARD for 16-bit buckets that run plain bf16 products
 *              (DMUON_PREC_BF16) with every member's long side n <= 2k --
 *              there the Gram form with bf16 state misses the 2e-2 accuracy
 *              bar on square matrices and saves at most a quarter of the
 *              flops -- GRAM otherwise. */
enum { DMUON_FORM_AUTO = 0, DMUON_FORM_GRAM = 1, DMUON_FORM_STANDARD = 2 };

/* Fill *opts with the defaults (AUTO, SQRT_RATIO, device plan, eps 1e-7, no
 * cap, built-in table, AUTO form, no padding, AUTO storage, AUTO fused). */
void dmuon_plan_opts_default(dmuon_plan_opts* opts);

/*  rows, cols  host arrays of `count` positive sizes (caller's orientation).
 *  dtype       DMUON_BF16 (bf16 params and grads) or DMUON_F32.
 *  opts        NULL for defaults.
 *  out         receives the plan; set to NULL on failure.
 * Allocates the device workspace on the current device unless opts->no_device.
 * May be called while other streams run; it synchronises nothing. */
int dmuon_plan(const int64_t* rows, const int64_t* cols, int64_t count, int dtype,
               const dmuon_plan_opts* opts, dmuon_plan_t** out);

/* Frees the plan and its workspace (NULL is a no-op).  The caller must make
 * sure no enqueued step still uses it. */
int dmuon_plan_destroy(dmuon_plan_t* plan);

/* JSON description of the plan: buckets, member indices, tile configs,
 * precision and workspace bytes.  Writes at most `len` bytes including the
 * terminating NUL; returns the full length needed (excluding NUL), or a
 * negative error code. */
int64_t dmuon_plan_describe(const dmuon_plan_t* plan, char* buf, size_t len);

/* ---------------------------------------------------------------------------
 * dmuon_step -- one fused Muon update of every matrix of the plan.
 *
 * Muon applies Newton-Schulz to momentum-aggregated gradients, and DMuon keeps
 * that update rule unchanged (technical summary sections 1 and 5).  For each
 * matrix i, in plan registration order:
 *   buf <- mu buf + G
 *   U   <- G + mu buf   if nesterov, else U <- buf
 *   O   <- dmuon_ns_batched(U) with (steps, a, b, c) and the plan's eps
 *   W   <- W (1 - lr weight_decay) - lr s(rows, cols) O
 *
 *  params   host array of `count` device pointers to W (dtype of the plan),
 *           updated in place.
 *  grads    host array of device pointers to G (dtype of the plan), read only.
 *  momenta  host array of device pointers to fp32 buffers, updated in place.
 *  All three arrays are read during the call only.
 * Errors: EPLAN for a NULL plan or a host-only plan; EINVAL for null arrays or
 * entries, steps < 0; EHIP on a launch failure.
 * ------------------------------------------------------------------------- */
int dmuon_step(const dmuon_plan_t* plan, void* const* params,
               const void* const* grads, void* const* momenta, float lr,
               float weight_decay, float mu, int nesterov, int steps, float a,
               float b, float c, void* stream);

/* ---------------------------------------------------------------------------
 * dmuon_plan_ns -- the Gram Newton-Schulz map of every matrix of the plan, in
 * place: the operation of dmuon_ns_batched (technical summary section 2.2:
 * Gram product, the recurrence P = aI + bA + cA^2, A <- P A P, Q <- P Q in
 * Gram space, one final product), over matrices of several shapes at once.
 * Matrices of one short side share the recurrence's launches (batching
 * bullet of section 2.2), as in dmuon_step, where separate dmuon_ns_batched
 * calls per shape would each run their own.  No shape factor is applied.
 *
 *  mats     host array of `count` device pointers (dtype of the plan), in plan
 *           registration order, each overwritten with its orthogonalised
 *           matrix; read during the call only.
 * Errors: EPLAN for a NULL plan, a host-only plan or another device;
 * EINVAL for a NULL array or entry, steps < 0; EUNSUPPORTED when a bucket
 * the plan forces to fp16 state cannot hold these coefficients; EHIP on a
 * launch failure.
 * ------------------------------------------------------------------------- */
int dmuon_plan_ns(const dmuon_plan_t* plan, void* const* mats, int steps, float a, float b,
                  float c, void* stream);

/* ---------------------------------------------------------------------------
 * dmuon_adamw_step -- one fused AdamW step over `count` tensors, in place.
 *
 * AdamW is the element-wise optimizer DMuon's cost is measured against
 * (technical summary section 4: the per-step overhead over AdamW); this call
 * provides it on the same GPU for that comparison.  Adam with decoupled
 * weight decay and bias-corrected moments, per element (t = step):
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   W <- W (1 - lr weight_decay)
 *        - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 * computed in fp32 (bias corrections evaluated on the host in double); bf16
 * parameters are rounded to nearest even.
 *
 *  params      host array of `count` device pointers to W (dtype), updated.
 *  grads       host array of device pointers to g (dtype), read only.
 *  exp_avg     host array of device pointers to fp32 m, updated.
 *  exp_avg_sq  host array of device pointers to fp32 v, updated.
 *  numel       host array of element counts (any shape: the update is
 *              element-wise; each tensor is contiguous).
 *  dtype       DMUON_BF16 or DMUON_F32 (parameters and gradients).
 *  step        1-based step count of the bias corrections.
 * Tensors must not overlap.  16-byte aligned tensors take 16-byte accesses;
 * others are processed element by element with the same results.  The
 * pointer arrays are read during the call only; one launch per 64 tensors,
 * no workspace.  eps = 0 with a zero second moment gives NaN, as the formula
 * does.
 * Errors: EINVAL for null arrays or entries, count <= 0, numel outside
 * [1, 2^40], unknown dtype, step < 1, betas outside [0, 1), eps < 0 or
 * non-finite lr, weight_decay or eps; EHIP on a launch failure.
 * ------------------------------------------------------------------------- */
int dmuon_adamw_step(void* const* params, const void* const* grads, void* const* exp_avg,
                     void* const* exp_avg_sq, const int64_t* numel, int64_t count, int dtype, float lr,
                     float beta1, float beta2, float eps, float weight_decay, int64_t step, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics: per-launch kernel timing.
 *
 * When enabled, every kernel launch made by the calls above is bracketed by a
 * pair of hipEvents recorded on the launch's stream, and the launch is
 * counted with its algorithmic work (flops for products, counting a
 * symmetric output's lower triangle only; bytes for the elementwise kernels).
 * Process-wide; not for concurrent use from several threads.
 * ------------------------------------------------------------------------- */

/* 1 enables recording, 0 disables it (records are kept).  Returns DMUON_OK. */
int dmuon_timing_enable(int enable);

/* JSON summary of the recorded launches grouped by kernel:
 *   {"kernels": [{"kernel": name, "launches": n, "total_ms": t, "avg_ms": t/n,
 *                 "flops": f, "bytes": b}, ...]}
 * Waits for the recorded events, then clears the records, on every call: pass
 * a buffer large enough for the whole report.  Writes at most `len` bytes
 * including the terminating NUL and returns the full length (excluding NUL);
 * a return value >= len means the text was cut.  EHIP if an event query
 * fails. */
int64_t dmuon_timing_report(char* buf, size_t len);

/* ---------------------------------------------------------------------------
 * Owner assignment (technical summary section 2.3).  In distributed DMuon
 * every matrix has exactly one owner rank, which keeps its optimizer state and
 * runs its Newton-Schulz update once; owners are chosen so that the predicted
 * maximum per-rank time (the makespan) is as small as possible, from costs
 * measured per distinct shape (dmuon_profile_costs) rather than flop counts.
 *
 * Cost model: matrices of one shape that share an owner run as one batch.
 * T_s(k), the time of a batch of k matrices of shape s, is the
 * piecewise-linear curve through (0, 0) and the points
 * (batches[p], times[s * npts + p]), extended past the last point with the
 * last segment's slope (negative values clamp to 0).  A rank's load is the
 * sum over shapes of T_s(k_s) for the counts k_s it owns.
 *
 *   shape_of   : count entries, the shape index of each matrix (0 <= . < nshapes)
 *   batches    : npts strictly increasing batch sizes, each >= 1
 *   times      : nshapes x npts costs (any unit), finite and >= 0
 *   ranks      : number of owners, 1 .. 2^20
 *   method     : DMUON_ASSIGN_EXACT  -- branch and bound over the per-rank
 *                                       counts; optimal unless it runs out of
 *                                       nodes (then the best assignment found,
 *                                       never worse than the greedy one)
 *                DMUON_ASSIGN_GREEDY -- one matrix at a time (shapes by
 *                                       decreasing single-matrix time) to the
 *                                       rank whose load after taking it is
 *                                       smallest, lowest rank on ties
 *                DMUON_ASSIGN_AUTO   -- EXACT for count <= 64, else GREEDY
 *   node_limit : search nodes for EXACT (<= 0: one million)
 *   owner      : out, count entries in [0, ranks): within one shape, matrices
 *                in index order fill rank 0 first, then rank 1, and so on
 *   makespan   : out (nullable), the predicted maximum load
 *   optimal    : out (nullable), 1 when the search proved the makespan minimal
 *
 * Host-only: touches no device, allocates only host memory, deterministic.
 * Errors: EINVAL (NULL pointer, non-positive size, index or cost out of range).
 */
enum { DMUON_ASSIGN_AUTO = 0, DMUON_ASSIGN_EXACT = 1, DMUON_ASSIGN_GREEDY = 2 };
int dmuon_assign_owners(const int32_t* shape_of, int64_t count, const int32_t* batches, int32_t npts,
                        const double* times, int32_t nshapes, int32_t ranks, int32_t method,
                        int64_t node_limit, int32_t* owner, double* makespan, int32_t* optimal);

/* dmuon_profile_costs -- measure the cost table on the current device
 * (technical summary section 2.3: the runtime of several batch sizes is
 * profiled per distinct shape at initialisation).
 *
 * For each shape (rows[s], cols[s]) and batch size batches[p] it runs
 * dmuon_ns_batched (bf16, AUTO precision, the given steps and coefficients)
 * on deterministic pseudo-random matrices: `warmup` untimed calls, then
 * `repeats` timed ones bracketed by HIP events on `stream`.  times[s*npts + p]
 * receives the median in milliseconds.
 *
 * Allocates and frees its own device buffers (the largest batch of each shape
 * in turn) and synchronises the stream: an initialisation-time call, not for
 * the training loop.  Errors: EINVAL (batch sizes outside [1, 4096] or not
 * increasing, non-positive shapes, repeats < 1), ENOMEM, EHIP, and any error
 * of dmuon_ns_batched. */
int dmuon_profile_costs(const int64_t* rows, const int64_t* cols, int32_t nshapes, const int32_t* batches,
                        int32_t npts, int steps, float a, float b, float c, int32_t warmup, int32_t repeats,
                        double* times, void* stream);

/* dmuon_tune -- measure tile configurations on the current device and write
 * a tune table (technical summary section 2.4: tile configurations are
 * searched per matrix shape on the target hardware, and the best one is
 * cached and reused on later steps).
 *
 * The `count` matrices (caller orientation rows x cols, as for dmuon_plan)
 * are grouped into recurrence buckets as dmuon_plan groups them.  For each
 * bucket on its own, every tile configuration -- the recurrence tile and the
 * Gram/final-product tile, each 64, 128 or 256; configurations that the
 * planner would run identically are timed once -- is timed on
 * deterministic pseudo-random bf16 matrices of the bucket's shapes:
 * `warmup` untimed dmuon_ns_batched-equivalent runs, then `repeats` timed
 * ones between HIP events on `stream`, median.  The fastest configuration of
 * each bucket becomes a table entry {max_m: m, max_batch: bucket size}, and
 * the JSON written to out_path also lists every candidate's time, the
 * device and the coefficients.  A plan reads such a file through
 * opts->tune_path or DMUON_TUNE_TABLE.
 *
 * Allocates and frees its own device memory and synchronises the stream: an
 * initialisation-time call.  Errors: EINVAL (NULL arguments, count <= 0,
 * shapes outside [1, 2^20], repeats < 1, warmup < 0, bad coefficients, an
 * unwritable out_path), ENOMEM, EHIP. */
int dmuon_tune(const int64_t* rows, const int64_t* cols, int64_t count, int steps, float a, float b, float c,
               int32_t warmup, int32_t repeats, const char* out_path, void* stream);

/* Thread-local description of the last error ("" if none). */
const char* dmuon_last_error(void);

/* Library version string. */
const char* dmuon_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_H */
