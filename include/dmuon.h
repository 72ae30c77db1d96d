/*
 * dmuon.h - C ABI of the MI355X (gfx950) per-owner Muon optimizer step.
 *
 * The library runs, on one GPU and batched over many owned 2D matrices, the
 * part of DMuon's Muon optimizer that the owner rank executes (DMuon
 * "HSDP Training (Multi-Node)", "What Happens Under the Hood": only the
 * owner runs momentum, Newton-Schulz, weight decay and the update on the
 * parameters it owns; DMuon "API Reference", Muon.step: momentum + NS +
 * update on owned dedicated params).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are dense, row-major, leading dimension == n (no stride
 *   argument).  Pointers are device pointers on the current HIP device,
 *   aligned at least to their element size.
 * - The caller owns every buffer (params, grads, momentum buffers, outputs,
 *   workspace).  The library keeps no pointer after the enqueued work ends.
 *   It keeps one per-device cache of launch tables keyed by the shapes and
 *   options of a call (never by its pointers): the first call with a new
 *   batch layout allocates and uploads that layout's table (a hipMalloc and
 *   a blocking copy); every later call with the same layout, whatever its
 *   buffers and workspace, allocates nothing and does not synchronize.  The
 *   call's buffer pointers travel to the device in kernel arguments (a
 *   small upload kernel writes them into the workspace) ahead of the
 *   call's kernels on `stream`.  Past 256 distinct layouts per process the
 *   least recently used table is freed (after a device synchronization).
 * - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *   the default stream).  The workspace must stay alive until that work
 *   completes.
 * - Validation is synchronous and happens before anything is enqueued: on
 *   any error no buffer is touched.  Errors are reported as a status code
 *   plus a thread-local message (dmuon_last_error).  No C++ exception
 *   crosses the ABI.  Faults inside kernels surface at the caller's next
 *   synchronization, or as DMUON_E_HIP from a later call.
 * - NaN and Inf propagate; nothing is clamped.  Results are bitwise
 *   reproducible run to run for the same inputs (fixed reduction orders, no
 *   floating-point atomics).
 * - count == 0 is a valid no-op.
 */
#ifndef DMUON_H
#define DMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DMUON_OK = 0,
  DMUON_E_INVALID = 1,     /* bad argument (shape, dtype, pointer, alias) */
  DMUON_E_UNSUPPORTED = 2, /* well-formed but outside the supported range */
  DMUON_E_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  DMUON_E_HIP = 4          /* HIP runtime error while enqueueing */
} dmuon_status_t;

/* Element types of caller buffers. */
typedef enum { DMUON_F32 = 0, DMUON_BF16 = 1 } dmuon_dtype_t;

/*
 * Newton-Schulz arithmetic.
 *   DMUON_NS_F32          fp32 operands on fp32 MFMA, fp32 accumulate.
 *   DMUON_NS_BF16         fp32 master copy of X; bf16 copies of X, A = X X^T
 *                         and B = bA + cA^2 as MFMA operands; fp32
 *                         accumulate and fp32 epilogues.
 *   DMUON_NS_BF16_SPLIT   as DMUON_NS_BF16, with A and B carried as bf16
 *                         hi + lo pairs (A^2 from three products, B X from
 *                         two).
 *   DMUON_NS_BF16_SPLIT_A as DMUON_NS_BF16 with only A split (A^2 from three
 *                         products, B X from one).
 *   DMUON_NS_F16          as DMUON_NS_BF16 for the first iteration (its
 *                         input is not normalized yet, and bf16 has fp32's
 *                         exponent range), then fp16 copies of X, A and B
 *                         (3 more fraction bits than bf16; the normalized
 *                         iterates stay inside fp16's range) on the
 *                         same-rate fp16 MFMA.  No operand is split.
 *   DMUON_NS_AUTO         per matrix by its tile class: DMUON_NS_F16 on
 *                         64- and 128-wide tiles (min side below 1024, or
 *                         where 256-wide tiles would pad more than 1/8),
 *                         DMUON_NS_BF16 on 256-wide tiles (fp16 products run
 *                         a few percent slower there and plain bf16 is well
 *                         within tolerance at those sizes).  Nothing is
 *                         split.
 */
typedef enum {
  DMUON_NS_F32 = 0,
  DMUON_NS_BF16 = 1,
  DMUON_NS_BF16_SPLIT = 2,
  DMUON_NS_AUTO = 3,
  DMUON_NS_BF16_SPLIT_A = 4,
  DMUON_NS_F16 = 5
} dmuon_prec_t;

/* One matrix: m rows, n columns, row-major, device pointer. */
typedef struct {
  int64_t m;
  int64_t n;
  void* ptr;
} dmuon_mat_t;

/* A batch of matrices of one element type; `mats` is a host array. */
typedef struct {
  const dmuon_mat_t* mats;
  int32_t count;
  int32_t dtype; /* dmuon_dtype_t */
} dmuon_batch_t;

/*
 * How the NS polynomial is evaluated (DMuon "API Reference", NewtonSchulz
 * backend "direct" or "gram").
 *   DMUON_NS_DIRECT  X <- a X + (b A + c A^2) X with A = X X^T, per step.
 *   DMUON_NS_GRAM    Gram space (gram_newton_schulz): per restart window,
 *                    A = X X^T, then per step P = a I + b A + c A^2,
 *                    Q <- P Q, A <- P A P, and X <- Q X at the window's
 *                    end.  Equal to DIRECT in exact arithmetic.  Operands:
 *                    fp32 (prec F32, or AUTO, which resolves to F32), or
 *                    fp16 (prec F16; DMuon "API Reference", the
 *                    newton_schulz module note: the mixed-precision Gram
 *                    pipeline in fp16), with X normalized before the first
 *                    window, A and P A stored times 2^12, P and Q times
 *                    2^10, fp32 accumulation, and the fp32 A kept for the
 *                    b A term.  The Q factor amplifies the rounding of X in
 *                    the small singular directions: relative Frobenius
 *                    error about 3e-3 on Gaussian inputs, up to 2e-2 on
 *                    low-rank ones with the default restart.  With F16 the
 *                    coefficients must keep |Q| below 48 over each window
 *                    (eigenvalues of A in [0, 1.25]): the quintic does
 *                    (40.9 over three steps); other tables are rejected
 *                    with DMUON_E_UNSUPPORTED.  Other precisions:
 *                    DMUON_E_UNSUPPORTED.
 */
typedef enum { DMUON_NS_DIRECT = 0, DMUON_NS_GRAM = 1 } dmuon_ns_backend_t;

/*
 * Newton-Schulz configuration (DMuon "API Reference", direct_newton_schulz:
 * per-step (a, b, c) coefficients whose list length is the number of
 * iterations; eps is added to the Frobenius norm used to normalize;
 * gram_newton_schulz: restart_iterations, default [2]).
 *   coeffs     host array of 3 * ns_steps floats (a0, b0, c0, a1, ...), or
 *              NULL for (3.4445, -4.7750, 2.0315) at every step.
 *   ns_steps   1..16.
 *   eps        >= 0 and finite (1e-7 in DMuon's signature).
 *   prec       dmuon_prec_t.
 *   backend    dmuon_ns_backend_t.
 *   restarts   GRAM only: host array of nrestarts step indices where a new
 *              window starts (indices outside 1..ns_steps-1 have no
 *              effect; negative ones are rejected), or NULL for [2].
 */
typedef struct {
  const float* coeffs;
  int32_t ns_steps;
  float eps;
  int32_t prec;
  int32_t backend;
  int32_t nrestarts;
  const int32_t* restarts;
} dmuon_ns_cfg_t;

/*
 * Workspace bytes needed by dmuon_ns_orthogonalize / dmuon_muon_step for a
 * batch of these shapes.  Only the shapes, count, cfg->prec and
 * cfg->backend matter (the pointers of `g` are not read; they may be NULL).
 * Pure host computation.
 */
dmuon_status_t dmuon_ns_workspace_size(const dmuon_batch_t* g,
                                       const dmuon_ns_cfg_t* cfg,
                                       size_t* bytes);

/*
 * out[i] = NS(g[i]) for every matrix of the batch (DMuon "API Reference",
 * direct_newton_schulz: G is transposed when it has more rows than columns,
 * normalized by ||G||_F + eps, then X <- a X + b (X X^T) X + c (X X^T)^2 X
 * per coefficient row; the result has G's shape and dtype).
 *   g, out    same count, same shapes, same dtype.  out[i] may be exactly
 *             g[i] (in place); any other overlap is rejected.
 *   ws        device workspace of at least dmuon_ns_workspace_size bytes,
 *             256-byte aligned.  Its contents on entry are ignored.
 */
dmuon_status_t dmuon_ns_orthogonalize(const dmuon_batch_t* g,
                                      const dmuon_batch_t* out,
                                      const dmuon_ns_cfg_t* cfg,
                                      void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * One Muon step on every owned matrix of the batch (DMuon "API Reference",
 * Muon: lr, momentum, weight_decay, ns_steps, nesterov; the nesterov
 * argument's lookahead feeds grad + momentum * buf to Newton-Schulz):
 *   buf <- momentum * buf + grad
 *   u   <- grad + momentum * buf      if nesterov, else buf
 *   O   <- NS(u)                      as in dmuon_ns_orthogonalize
 *   p   <- p - lr * weight_decay * p - lr * O
 * params: F32 or BF16, updated in place (the new value is rounded to the
 * param dtype, round-to-nearest-even).  grads: F32 or BF16, read only.
 * bufs: F32, updated in place.  The three batches have the same count and
 * per-index shapes; no two of the buffers overlap.
 */
dmuon_status_t dmuon_muon_step(const dmuon_batch_t* params,
                               const dmuon_batch_t* grads,
                               const dmuon_batch_t* bufs,
                               const dmuon_ns_cfg_t* cfg,
                               float momentum, float lr, float weight_decay,
                               int32_t nesterov,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * dmuon_muon_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the workspace, the call's
 * pointer slots and its launch tables live in a static device array of
 * 64 MiB per GPU, which the library holds from its first use on that GPU
 * until the process ends.  The call allocates nothing, on the device or
 * through any library, and its result is bitwise the one dmuon_muon_step
 * gives for the same arguments.
 *   - Batches whose workspace plus launch tables exceed 64 MiB are rejected
 *     with DMUON_E_UNSUPPORTED (e.g. the fp32 TinyMLP d=256 step fits; one
 *     TinyMLP d=512 layer fits; the whole 4-layer d=512 step does not).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     behind: two calls that overlap in time on one GPU (other streams,
 *     other threads) race and give wrong results.  Calls on one stream are
 *     ordered and safe.  Nothing in the array needs clearing between calls.
 * Arguments and errors as dmuon_muon_step.
 */
dmuon_status_t dmuon_muon_step_noalloc(const dmuon_batch_t* params,
                                       const dmuon_batch_t* grads,
                                       const dmuon_batch_t* bufs,
                                       const dmuon_ns_cfg_t* cfg,
                                       float momentum, float lr, float weight_decay,
                                       int32_t nesterov, void* stream);

/*
 * Recorded calls (HIP graphs), for batches whose step is short enough that
 * launching its kernels one by one costs a visible share of it (the
 * TinyMLP shapes of DMuon "Quick Start"; many small owned matrices).
 *
 * dmuon_muon_step_graph / dmuon_ns_orthogonalize_graph validate exactly as
 * dmuon_muon_step / dmuon_ns_orthogonalize, then record the kernels that
 * call would enqueue -- with these buffer pointers, this workspace and these
 * hyperparameters -- into an executable graph (nothing runs yet).
 * dmuon_graph_launch enqueues one replay on `stream`: the same operation,
 * bitwise the same result as the direct call would give on the buffers'
 * contents at that point of the stream.
 *   - The graph keeps the pointers: params, grads, bufs (or g, out) and ws
 *     must stay allocated, unmoved, until dmuon_graph_destroy; refill the
 *     gradient buffers between replays.  A new lr, momentum or gradient
 *     buffer needs a new graph (recording costs a few host milliseconds and
 *     no device synchronization).
 *   - Replays of one graph share its workspace: replays that overlap in time
 *     (different streams without ordering) race.
 *   - Launch with the recording device current, on any stream of it.
 *   - The graph holds a reference to its launch tables; they outlive the
 *     table cache's eviction until the graph is destroyed.
 *   - Recording must not happen inside another stream capture; an empty
 *     batch is DMUON_E_INVALID (there is nothing to record).
 * dmuon_graph_destroy waits for the device to finish outstanding work, then
 * frees the graph; NULL is a no-op.
 */
typedef struct dmuon_graph_s* dmuon_graph_t;

dmuon_status_t dmuon_muon_step_graph(const dmuon_batch_t* params,
                                     const dmuon_batch_t* grads,
                                     const dmuon_batch_t* bufs,
                                     const dmuon_ns_cfg_t* cfg,
                                     float momentum, float lr, float weight_decay,
                                     int32_t nesterov,
                                     void* ws, size_t ws_bytes,
                                     dmuon_graph_t* graph);

dmuon_status_t dmuon_ns_orthogonalize_graph(const dmuon_batch_t* g,
                                            const dmuon_batch_t* out,
                                            const dmuon_ns_cfg_t* cfg,
                                            void* ws, size_t ws_bytes,
                                            dmuon_graph_t* graph);

dmuon_status_t dmuon_graph_launch(dmuon_graph_t graph, void* stream);

void dmuon_graph_destroy(dmuon_graph_t graph);

/*
 * Gram-space NS of matrices held as column shards of their oriented view
 * (DMuon "API Reference", gram_newton_schulz_distributed_local and its
 * batched variant: the shard group rebuilds only the small Gram matrix by
 * an all-reduce, and each rank gets its own block of the full NS output).
 *
 * g[i] is this rank's block of matrix i in the stored layout.  transposed
 * (0 or 1, one flag for the batch) is the FULL matrix's orientation: when 1,
 * g[i]^T is the block of the oriented matrix, so p = g[i].n and the block's
 * width is g[i].m; when 0, p = g[i].m.  Every rank of a group passes the same
 * flag, the same p per matrix and the same batch order; block widths may
 * differ.  cfg->backend must be DMUON_NS_GRAM (prec F32 or AUTO).
 *
 * The sums over the group are the caller's: the library keeps them in one
 * fp32 "bucket" inside the workspace (every matrix's sum of squares, then
 * every p x p Gram matrix, padded; see dmuon_gram_local_bucket), and the
 * caller sums it in place over the group (e.g. an all-reduce enqueued on
 * the same stream) between the calls:
 *
 *   dmuon_gram_local_begin(...)                     bucket <- local sums
 *   for w in 0 .. windows-1:
 *     <sum the bucket over the group, in place>
 *     dmuon_gram_local_advance(..., w, ...)          w < windows-1: bucket <-
 *                                                    local sums for w+1;
 *                                                    last: out <- result
 *
 * With one rank (or no sum) the block is the whole matrix and the result is
 * dmuon_ns_orthogonalize's with the Gram backend.  The state between calls
 * lives in the workspace: keep ws, g, out and cfg the same through one
 * sequence and do not start another on the same workspace before it ends
 * (a wrong order gives wrong values, never an out-of-bounds access).
 * Momentum, the lr and weight decay stay with the caller (as on the pages).
 * out may be exactly g (it is written by the last advance only).
 */
dmuon_status_t dmuon_gram_local_workspace_size(const dmuon_batch_t* g, int32_t transposed,
                                               const dmuon_ns_cfg_t* cfg, size_t* bytes);

/* Where the bucket lies: `count` floats at byte `offset` of the workspace
 * (256-byte aligned), and the number of restart windows (sums per call
 * sequence).  Only shapes, transposed and cfg are read. */
dmuon_status_t dmuon_gram_local_bucket(const dmuon_batch_t* g, int32_t transposed,
                                       const dmuon_ns_cfg_t* cfg, size_t* offset,
                                       int64_t* count, int32_t* windows);

dmuon_status_t dmuon_gram_local_begin(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                      int32_t transposed, const dmuon_ns_cfg_t* cfg,
                                      void* ws, size_t ws_bytes, void* stream);

/* window: 0 .. windows-1, in order; anything else is DMUON_E_INVALID. */
dmuon_status_t dmuon_gram_local_advance(const dmuon_batch_t* g, const dmuon_batch_t* out,
                                        int32_t transposed, const dmuon_ns_cfg_t* cfg,
                                        int32_t window, void* ws, size_t ws_bytes,
                                        void* stream);

/*
 * Gradient-norm clipping of Muon gradients (DMuon "API Reference",
 * clip_grad_norm_: only DMuon's Muon gradients, norm_type 2.0 by default,
 * the stats of MuonGradClipStats; clip_grad_norm_buckets_: every bucket
 * keeps its own norm and coefficient).  Per bucket b:
 *   total = (sum over its gradients of |g|^p)^(1/p)   (p = +inf: max |g|;
 *           a NaN anywhere gives NaN)
 *   coef  = max_norm / (total + 1e-6)
 *   g    <- g * min(coef, 1)   (every element; bf16 rounded to nearest even;
 *           a NaN coef makes the bucket NaN, as multiplying by it does)
 *   grads       F32 or BF16 tensors (m x n, row-major), updated in place.
 *   bucket_of   host array, bucket of each gradient, values in
 *               [0, nbuckets); NULL means every gradient is in bucket 0
 *               (then nbuckets must be 1).
 *   max_norm    finite, >= 0; ignored when stats_only != 0, in which case
 *               nothing is scaled and coef is reported as 1.
 *   norm_type   p > 0, or +inf.
 *   stats       device array of nbuckets entries (8-byte aligned), written
 *               on the stream; read it after the stream has reached this
 *               point.
 *   ws          device workspace of dmuon_clip_workspace_size bytes,
 *               256-byte aligned; contents on entry are ignored.
 * Distributed reduction of the per-rank norms is outside this one-GPU call.
 * Errors: as dmuon_muon_step (nothing is enqueued when validation fails).
 */
typedef struct {
  double total_norm;    /* bucket norm before clipping */
  double clip_coef;     /* max_norm / (total_norm + 1e-6); 1 for stats only */
  int32_t clipped;      /* clip_coef < 1 */
  int32_t found_inf;    /* total_norm is not finite */
  int64_t param_count;  /* elements in the bucket */
} dmuon_clip_stats_t;

dmuon_status_t dmuon_clip_workspace_size(const dmuon_batch_t* grads,
                                         int32_t nbuckets, size_t* bytes);

dmuon_status_t dmuon_clip_grad_norm(const dmuon_batch_t* grads,
                                    const int32_t* bucket_of, int32_t nbuckets,
                                    double max_norm, int32_t stats_only,
                                    double norm_type,
                                    dmuon_clip_stats_t* stats,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * AdamW update of the parameters Muon does not own (DMuon "API Reference",
 * Muon: step runs AdamW on them; the signature's adamw_lr=1e-3,
 * adamw_betas=(0.9, 0.999), adamw_weight_decay=0.01, adamw_eps=1e-8 are
 * the Python binding's defaults).  Decoupled weight decay, t = step:
 *   p <- p * (1 - lr * weight_decay)
 *   m <- beta1 * m + (1 - beta1) * g
 *   v <- beta2 * v + (1 - beta2) * g^2
 *   p <- p - lr / (1 - beta1^t) * m / (sqrt(v) / sqrt(1 - beta2^t) + eps)
 *   params      F32 or BF16, updated in place (bf16 rounded to nearest even).
 *   grads       F32 or BF16, read only.
 *   exp_avg, exp_avg_sq   F32 moments, updated in place.
 * Same count and per-index shapes in the four batches, no overlaps; step
 * >= 1 (the count after this update); betas in [0, 1), eps > 0.  The
 * hyperparameters are doubles: 1 - beta and the bias corrections are formed
 * in double before the kernels get their fp32 factors (1 - beta from an
 * fp32 beta2 = 0.999 would be 1.3e-5 off).  No workspace.  Errors: as
 * dmuon_muon_step.
 */
dmuon_status_t dmuon_adamw_step(const dmuon_batch_t* params,
                                const dmuon_batch_t* grads,
                                const dmuon_batch_t* exp_avg,
                                const dmuon_batch_t* exp_avg_sq,
                                int64_t step, double lr, double beta1, double beta2,
                                double eps, double weight_decay, void* stream);

/* Number of launch tables built so far in this process (see the cache
 * described at the top): a caller can check that its steady state builds
 * none.  Thread-safe. */
int64_t dmuon_plan_builds(void);

/* Static string for a status code. */
const char* dmuon_status_str(dmuon_status_t status);

/* Message of the last failing call on this thread ("" if none). */
const char* dmuon_last_error(void);

/* One-line description of the compiled kernels (cf. DMuon "API Reference",
 * get_ns_backend: a one-line summary of the active NS kernel). */
const char* dmuon_backend_info(void);

/*
 * Per-kernel timing (cf. DMuon "API Reference", Muon: record_step_profile
 * records event timings of the optimizer phases).  Between
 * dmuon_profile_begin(mask) and dmuon_profile_end(), every launch of a
 * kernel kind selected by `mask` (bit k selects kind k of the list below;
 * 0 selects all) made by this thread is bracketed by HIP events on the
 * stream it is launched on.  dmuon_profile_end synchronizes those events and
 * fills up to `max` rows of `out` (one per kind that ran), returning the
 * number of rows, or -1 on error.  `flops` and `bytes` are the algorithmic
 * work of those launches: symmetric-aware flops of the NS products
 * (p(p+1)q for A = X X^T, p^2(p+1) for A A, 2p^2q for B X), and the HBM
 * bytes of each launch with every operand read once and every output
 * written once in the library's workspace layout (for the element-wise
 * kernels, the bytes the step must move at minimum).
 * Kinds: 0 momentum, 1 input, 2 norm, 3 syrk, 4 poly, 5 update_x,
 * 6 clip_norm, 7 clip_scale, 8 adamw, 9 gram_mul (a product of two commuting
 * symmetric p x p factors of Gram-space NS), 10 gram_x (Gram-space NS with
 * fp16 operands: X normalized into its fp16 form).  The last update_x launch of a
 * call also applies the parameter update (or writes the NS output), so there
 * is no separate update kind.
 */
typedef struct {
  char name[24];
  int32_t kind;
  int32_t launches;
  double ms;     /* summed event time over the launches */
  double flops;  /* summed algorithmic flops */
  double bytes;  /* summed algorithmic HBM bytes */
} dmuon_profile_row_t;

int32_t dmuon_profile_begin(uint32_t kind_mask);
int32_t dmuon_profile_end(dmuon_profile_row_t* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* DMUON_H */
