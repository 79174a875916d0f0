/*
 * muon_hip.h -- C ABI of the batched Muon optimizer step for AMD Instinct
 * MI355X (gfx950).
 *
 * The library orthogonalises batches of same-shaped 2-D updates with the
 * quintic Newton-Schulz iteration and applies the Muon parameter update.
 * Every step runs in hand-written HIP kernels on the caller's stream.
 *
 * Sources (page title and section):
 *   [CS] "Muon Custom Sizing" walkthrough of the modded-nanogpt 124M record:
 *        section 1 (Muon = SGD-momentum followed by NS orthogonalisation),
 *        section 2.3 (attn weights viewed as 4 blocks; quintic constants,
 *        5 rounds), section 3.1 (the contiguous (4, hdim, dim) view),
 *        section 4 (momentum lerp forms, decoupled weight decay, effective lr).
 *   [PG] parameter-golf train_gpt.py walkthrough, Part 1 "how the Muon
 *        optimizer works" (zeropower_via_newtonschulz5: bf16 cast, Frobenius
 *        normalisation, A = X X^T, B = bA + cA A, X = aX + BX; aspect factor
 *        max(1, m/n)^0.5).
 *   [SH] the guide to the utils module of distributed_shampoo in
 *        modded-nanogpt's optimization track, section "tensor math
 *        utilities: dimension merging, blocking and distributed allocation"
 *        (merge_small_dims: reshaping a >2-D parameter, e.g. a convolution
 *        kernel, into the 2-D matrix a Muon-style optimizer works on).
 *   [DA] the article on moving the Adam gradient reduce-scatter of
 *        modded-nanogpt's DistAdam into a backward hook (record of
 *        2025-10-31), "change two": the per-parameter AdamW body of
 *        DistAdam.step, used for the parameters Muon does not take.
 *
 * Conventions shared by every entry point
 *   - Matrices are row-major and contiguous: a batch is [batch, rows, cols].
 *   - bf16 data is passed as `void*` holding IEEE bfloat16 bit patterns.
 *   - All pointers are device pointers owned by the caller, 16-byte aligned.
 *     The library never allocates or frees device memory and keeps no device
 *     state between calls; scratch memory is the caller's `workspace` (size
 *     from the *_workspace_bytes queries, 256-byte aligned).  Its first 256
 *     bytes hold the status words of the last call that used it (see
 *     muon_workspace_status); the rest is undefined before and after a call.
 *     The only host state is a cache of persistent-loop queues per set of
 *     block shapes, kept in pinned host memory and copied into the workspace
 *     by every call that runs the loop.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every kernel and
 *     copy of a call is enqueued on it and the call returns without
 *     synchronising.  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is enqueued: on any error the
 *     call has no side effects.  batch == 0 is a valid no-op.
 *   - Non-finite inputs propagate; they are not checked.
 *   - Calls on different streams must use different workspaces.  The part of
 *     a workspace a call uses must not overlap its data buffers
 *     (MUON_ERR_INVALID_ARG).
 *   - No C++ exception crosses this boundary.
 *
 * The NS block: with view_blocks = v, each stored rows x cols matrix is read
 * as v contiguous blocks of rows x (cols / v) ([CS] sections 2.3 and 3.1:
 * block k is elements [k*rows*cols/v, (k+1)*rows*cols/v) re-read row-major).
 * A block with more rows than columns is orthogonalised in its transposed
 * (wide) orientation; the result is returned in the stored orientation.
 */
#ifndef MUON_HIP_H
#define MUON_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MUON_ABI_VERSION 7

typedef enum muon_status {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARG = 1,   /* null pointer, bad scalar, bad config field */
    MUON_ERR_SHAPE = 2,         /* rows/cols/view_blocks/batch out of range   */
    MUON_ERR_ALIGNMENT = 3,     /* pointer not 16-byte (workspace 256) aligned */
    MUON_ERR_WORKSPACE = 4,     /* workspace smaller than muon_workspace_bytes */
    MUON_ERR_HIP = 5,           /* a HIP runtime call failed                  */
    MUON_ERR_UNSUPPORTED = 6    /* current device is not gfx950               */
} muon_status;

typedef enum muon_precision {
    /* bf16 operands everywhere, fp32 MFMA accumulation, bf16 RNE stores. */
    MUON_PRECISION_FAST = 0,
    /* bf16 MFMA with split operands: B = b*A + c*A*A kept as a bf16 hi+lo
     * pair, the iterate X kept as hi+lo (about 16 significant bits), and
     * B*X formed as Bh*Xh + Bh*Xl + Bl*Xh.  About 1.6x the MFMA work. */
    MUON_PRECISION_ACCURATE = 1
} muon_precision;

/* Newton-Schulz settings ([PG] Part 1; constants from [CS] section 2.3). */
typedef struct muon_ns_config {
    int32_t ns_steps;   /* quintic iterations, 0..64 (0 returns X/(|X|_F+eps)) */
    float a, b, c;      /* X <- a X + (b A + c A A) X with A = X X^T           */
    float eps;          /* normaliser is |X|_F + eps, per NS block (>= 0)       */
    int32_t precision;  /* muon_precision                                       */
} muon_ns_config;

/* Fills cfg with ns_steps 5, (a,b,c) = (3.4445, -4.7750, 2.0315), eps 1e-7,
 * MUON_PRECISION_FAST.  No-op when cfg is NULL. */
void muon_ns_config_default(muon_ns_config* cfg);

/* Bytes of workspace that ns_orthogonalize_batched / muon_step_batched need
 * for this shape and config (cfg NULL = defaults).  Returns 0 for batch == 0
 * and (size_t)-1 for an invalid shape. */
size_t muon_workspace_bytes(int64_t batch, int64_t rows, int64_t cols,
                            int32_t view_blocks, const muon_ns_config* cfg);

/*
 * out = NS(x) for every NS block of a [batch, rows, cols] bf16 batch
 * ([PG] Part 1; [CS] section 2.3 for view_blocks = 4).
 *   x        in,  bf16 [batch, rows, cols]
 *   out      out, bf16 [batch, rows, cols]; may be x itself (exact alias),
 *            must not overlap it otherwise
 *   cfg      NULL = defaults
 * Each NS block is normalised by its own Frobenius norm s = |X|_F + eps,
 * taken as sqrt(trace(X X^T)) from the first Gram product's fp32 diagonal
 * (FAST: of the bf16 values; ACCURATE: of the hi plane; with ns_steps = 0
 * from the sum of squares of x); the first polynomial and B X apply it.
 */
muon_status ns_orthogonalize_batched(const void* x, void* out,
                                     int64_t batch, int64_t rows, int64_t cols,
                                     int32_t view_blocks, const muon_ns_config* cfg,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Largest scratch ns_orthogonalize_batched_noalloc uses (bytes): the 256-byte
 * status header plus the plan regions muon_workspace_bytes describes (without
 * the persistent loop's queue). */
#define MUON_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * ns_orthogonalize_batched for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without a workspace and the same results,
 * bit for bit.  Its scratch is one library-owned static device array per GPU
 * of MUON_NOALLOC_SCRATCH_BYTES, held until the process ends; the call makes
 * no allocation (device or host), records no timing events, and always runs
 * the per-product NS schedule.
 *   Returns MUON_ERR_WORKSPACE when the batch needs more scratch than that
 *   (muon_workspace_bytes minus the loop queue); nothing is enqueued then.
 *   Every call on one GPU shares its scratch, so calls that overlap on one
 *   GPU (different streams or host threads without ordering) race; calls on
 *   one stream are ordered and safe.
 *   The first call on a device looks up the scratch's device address
 *   (hipGetSymbolAddress); make it outside stream capture.  Later calls can
 *   be captured into a HIP graph.
 */
muon_status ns_orthogonalize_batched_noalloc(const void* x, void* out,
                                             int64_t batch, int64_t rows, int64_t cols,
                                             int32_t view_blocks, const muon_ns_config* cfg,
                                             void* stream);

/*
 * One Muon step for a [batch, rows, cols] batch of parameters ([CS] sections
 * 1 and 4, [PG] Part 1), in place:
 *   M <- M + (1 - mu)(G - M)                      (momentum buffer, fp32)
 *   U <- G + mu (M - G)   if nesterov, else U <- M
 *   O <- NS(U) per NS block                       (see ns_orthogonalize_batched)
 *   P <- P (1 - lr wd wd_mul) - lr max(1, rows/cols)^0.5 lr_mul O
 *   params     in/out fp32 [batch, rows, cols]
 *   grads      in     bf16 [batch, rows, cols]
 *   momentum_buf in/out fp32 [batch, rows, cols]
 *   update_out optional out, bf16 [batch, rows, cols]: O (before lr/aspect);
 *              NULL to skip
 *   lr, weight_decay, momentum (mu), lr_mul, wd_mul: finite floats,
 *              0 <= momentum <= 1
 * params, grads, momentum_buf and update_out must not overlap.
 */
muon_status muon_step_batched(float* params, const void* grads, float* momentum_buf,
                              int64_t batch, int64_t rows, int64_t cols,
                              int32_t view_blocks,
                              float lr, float weight_decay, float momentum,
                              int32_t nesterov, float lr_mul, float wd_mul,
                              const muon_ns_config* cfg, void* update_out,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/* One parameter matrix of a multi-matrix step, each with its own buffers
 * (row-major, contiguous).  The pages' optimizer steps every matrix with its
 * own lr_mul / wd_mul ([CS] section 4); params, grads, momentum_buf and
 * update_out are as in muon_step_batched for a batch of one. */
typedef struct muon_matrix {
    float* params;          /* in/out fp32 [rows, cols]                      */
    const void* grads;      /* in     bf16 [rows, cols]                      */
    float* momentum_buf;    /* in/out fp32 [rows, cols]                      */
    void* update_out;       /* optional out bf16 [rows, cols] (O); NULL skips */
    int64_t rows, cols;
    int32_t view_blocks;    /* as in muon_step_batched                       */
    float lr_mul, wd_mul;   /* finite                                        */
} muon_matrix;

/* Bytes of workspace muon_step_multi needs for these matrices and config
 * (cfg NULL = defaults); 0 when count is 0 or every block is small, and
 * (size_t)-1 for an invalid matrix shape or count. */
size_t muon_step_multi_workspace_bytes(const muon_matrix* mats, int32_t count,
                                       const muon_ns_config* cfg);

/*
 * One Muon step for `count` matrices of any shapes, each with its own buffers
 * (the multi-matrix form of muon_step_batched; [CS] sections 1, 2.2 and 4):
 * per matrix i, the update of muon_step_batched with its rows, cols,
 * view_blocks, lr_mul and wd_mul and the shared lr, weight_decay, momentum,
 * nesterov and cfg.  Matrices of one (rows, cols, view_blocks) shape are
 * stepped as one batch.  Batches whose NS blocks have the same padded
 * smaller side run their Newton-Schulz loops together, products of equal
 * reduction length sharing kernel launches, while their workspaces together
 * stay within 160 MB (so they stay cache-resident); the others run one after
 * the other and reuse one workspace region.  Each matrix's result is bitwise
 * the one muon_step_batched gives it.
 *   mats     host array of `count` descriptors, read during the call only
 *   No two buffers of any matrices may overlap (MUON_ERR_INVALID_ARG).
 *   Alignment: 16 bytes when a matrix's NS blocks take the matrix-core path
 *   (more than 64 rows and columns, or more than 8192 elements) and
 *   cols/view_blocks is a multiple of 8; else 4 bytes (fp32) and 2 bytes
 *   (bf16).  Blocks with at most 64 rows or columns and 8192 elements run
 *   the whole step in one fp32 workgroup each and use 16-byte accesses only
 *   where the buffers allow.
 */
muon_status muon_step_multi(const muon_matrix* mats, int32_t count,
                            float lr, float weight_decay, float momentum,
                            int32_t nesterov, const muon_ns_config* cfg,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* One tensor of an AdamW step (any shape, stored contiguously). */
typedef struct muon_adam_tensor {
    float* params;          /* in/out fp32 [numel]                                */
    const void* grads;      /* in     bf16 [numel]                                */
    float* exp_avg;         /* in/out fp32 [numel], first moment                  */
    float* exp_avg_sq;      /* in/out fp32 [numel], second moment                 */
    int64_t numel;          /* >= 0; 0 skips the tensor (pointers may be NULL)    */
    int64_t step;           /* t, the tensor's step count after this step's
                               increment (>= 1; 1 when the moments start at 0)    */
    float lr_mul, wd_mul;   /* finite                                             */
} muon_adam_tensor;

/*
 * One AdamW step ([DA] DistAdam.step, on one GPU: the whole tensor is the
 * rank's slice) for `count` tensors, in place, per element:
 *   p <- p (1 - lr lr_mul weight_decay wd_mul)     (skipped when weight_decay == 0)
 *   m <- beta1 m + (1 - beta1) g
 *   v <- beta2 v + (1 - beta2) g^2
 *   p <- p - lr lr_mul (1 - beta2^t)^0.5 / (1 - beta1^t) * m / (sqrt(v) + eps)
 * eps is added before the second-moment bias correction, as [DA] orders it
 * (torch's AdamW adds it after).  The 124M record uses lr 0.008,
 * betas (0.8, 0.95), eps 1e-8 ([CS] section 4).
 *   tensors  host array of `count` descriptors, read during the call only
 *   lr, weight_decay finite; eps finite and >= 0; 0 <= beta1, beta2 < 1
 *   Buffers: 4-byte (fp32) / 2-byte (bf16) aligned; 16-byte aligned buffers
 *   move 8 elements per access.  No two buffers of any tensors may overlap
 *   (MUON_ERR_INVALID_ARG).  count == 0 is a valid no-op.
 * All tensors run in one launch per 24 tensors; the call needs no workspace.
 */
muon_status adamw_step_multi(const muon_adam_tensor* tensors, int32_t count,
                             float lr, float beta1, float beta2, float eps,
                             float weight_decay, void* stream);

#define MUON_MAX_DIMS 16

/*
 * Merged shape of a contiguous tensor ([SH] merge_small_dims), so that a
 * parameter of any rank can be stepped as the 2-D matrix it views as
 * (e.g. a (32, 3, 64, 64) convolution kernel as 96 x 4096 at threshold 8192):
 *   - ndim == 0 gives (1); a zero extent gives (0); extents equal to 1 are
 *     dropped, and if all are 1 the result is (1);
 *   - walking from the last extent towards the first, the next extent is
 *     folded into the one being formed while their product is <= threshold
 *     and the shape still has more than target_ndim extents; an extent above
 *     the threshold is never split;
 *   - target_ndim == 0 means no target: the squeezed shape is returned.
 * Merging adjacent extents of a row-major tensor is a reinterpretation: the
 * merged tensor is a view of the same memory.
 *   shape        in, ndim extents (0 <= ndim <= MUON_MAX_DIMS), each >= 0
 *   threshold    >= 1
 *   merged       out, room for max(ndim, 1) extents
 *   merged_ndim  out
 * Host-only: needs no device.
 */
muon_status muon_merge_small_dims(const int64_t* shape, int32_t ndim, int64_t threshold,
                                  int32_t target_ndim, int64_t* merged, int32_t* merged_ndim);

/*
 * Status of the last call that used `workspace` (any entry point that needed
 * a workspace), copied into status_out[0..1] on `stream` after that call's
 * work:
 *   status_out[0]  number of NS blocks whose persistent-loop iterations did
 *                  not all complete; their outputs (NS output, update_out,
 *                  and the updated params) are NaN
 *   status_out[1]  flags: 1 a dependency wait of the loop ran out of time (or
 *                  was forced to, muon_debug_set_loop_fault), 2 blocks were
 *                  left incomplete, 4 a workgroup ran on an XCD that serves no
 *                  queue
 * Both are 0 after a call that completed.  The persistent loop bounds each
 * wait for a dependency (1 s) so that a stalled run ends; such a run never
 * returns unmarked results.  The call's first kernel clears the words.
 *   workspace   the workspace the call used (non-null, 256-byte aligned)
 *   status_out  2 uint32: device memory or pinned host memory (the copy is
 *               then asynchronous), or pageable host memory (the call then
 *               waits for the stream)
 */
muon_status muon_workspace_status(const void* workspace, uint32_t* status_out, void* stream);

/* Diagnostics for tests of the failure path (process-wide): mode 0 normal;
 * mode 1 every persistent-loop launch sets its error word at its start, so
 * every workgroup leaves at its first item; mode 2 every dependency wait that
 * is not met at once counts as timed out.  Every kernel still exits normally;
 * results are then NaN where blocks were left incomplete, as reported by
 * muon_workspace_status.  Returns MUON_ERR_INVALID_ARG for any other mode. */
muon_status muon_debug_set_loop_fault(int32_t mode);

/* Schedule of the Newton-Schulz iterations of large blocks (process-wide).
 * Two schedules give bitwise the same results:
 *   per-product: each iteration launches the Gram, polynomial and B X
 *     products in turn;
 *   persistent: all iterations of the blocks of a call (of a wave, in
 *     muon_step_multi) run in one launch of one workgroup per CU, which take
 *     runs of 256-wide tiles of the three products from a precomputed queue
 *     and wait on per-block completion counters kept in the workspace.  It
 *     needs FAST precision and both padded sides of every block batch
 *     multiples of 256; other calls use the per-product schedule.
 * mode 0 (default): automatic, per set of block shapes and counts: the first
 *   10 calls with a new set alternate the two schedules under hipEvent timing
 *   (recorded on the call's stream) and, once those events have completed,
 *   later calls use the one with the lower best time;
 * mode 1: per-product always;  mode 2: persistent wherever it applies.
 * The persistent schedule's queue for each distinct set of shapes is built on
 * the host by the first call that needs it and kept in pinned host memory
 * (hipHostMalloc) until the process ends; each call copies it into its
 * workspace on its stream.  Beyond 64 such sets (256 for the automatic
 * choice), calls with a new set use the per-product schedule.  With 8 queues
 * a workgroup serves the queue of the XCD it runs on.
 * Under stream capture (hipStreamBeginCapture on the call's stream) a call
 * allocates, times and synchronises nothing: it reuses the schedule an
 * earlier call settled for the set (and its cached queue), else runs per
 * product; captured calls replay to the eager results bit for bit.
 * Returns MUON_ERR_INVALID_ARG for any other mode. */
muon_status muon_set_ns_schedule(int32_t mode);

/* Tile width of the per-product Gram, polynomial and B X launches
 * (process-wide).  Every width accumulates each 32 x 32 output block with the
 * same MFMA sequence in the same order, so results are bitwise the same:
 *   0 (default): automatic, per launch signature (product kind, reduction
 *     length, device, every block batch's padded sides and block count),
 *     among 64-wide tiles (up to five per CU; for launches of few tiles,
 *     where the chain of dependent products is the time), 128-wide,
 *     256-wide, and 256-wide with the last partial round as 128-wide
 *     quadrants.  The plans estimated within 2x of the best estimate each
 *     run 3 launches timed with an event pair on the launch's stream; once
 *     those events have completed the plan with the lowest time is kept for
 *     the signature.  Until then, under stream capture, in
 *     ns_orthogonalize_batched_noalloc (which creates no events) and beyond
 *     1024 signatures, the best estimate is used;
 *   64, 128: that width;
 *   256: that width where both padded sides of every block batch of the
 *     launch are multiples of 256, else 128.
 * The persistent loop always uses 256-wide tiles.  Returns
 * MUON_ERR_INVALID_ARG for any other width. */
muon_status muon_set_gemm_tiling(int32_t width);

/* Kernel timing (diagnostics).  Kernel families of the library: */
typedef enum muon_kernel_kind {
    MUON_KERNEL_PREP = 0,           /* momentum + cast (+ tile norms, 0 steps) */
    MUON_KERNEL_NORM_FINALIZE = 1,  /* per-block 1/|X|_F (ns_steps = 0 only)   */
    MUON_KERNEL_GRAM = 2,           /* A = X X^T                               */
    MUON_KERNEL_POLY = 3,           /* B = b A + c A A                         */
    MUON_KERNEL_BX = 4,             /* X <- a X + B X                          */
    MUON_KERNEL_FINISH = 5,         /* NS output / parameter update            */
    MUON_KERNEL_SMALL = 6,          /* whole step for small blocks             */
    MUON_KERNEL_ADAMW = 7,          /* AdamW step (adamw_step_multi)           */
    MUON_KERNEL_NS_LOOP = 8,        /* all NS iterations in one launch         */
    MUON_KERNEL_COUNT = 9
} muon_kernel_kind;

/* While kernel_mask has bit k set, every launch of kernel family k records a
 * hipEvent before and after it on the stream it is launched on (events are
 * created on first use with hipEventDisableSystemFence, as they only measure
 * time, and reused; 0 turns recording off).  Recording adds two event packets
 * per selected launch and nothing when the mask is 0.  One launch of a family
 * is one library-level launch: the B X product of a call may run as a bulk
 * kernel plus a tail kernel, timed together. */
muon_status muon_timing_enable(uint32_t kernel_mask);

/* Waits for every recorded event, adds launch counts, elapsed milliseconds,
 * nominal and executed flops per family into launches[MUON_KERNEL_COUNT],
 * total_ms[MUON_KERNEL_COUNT], nominal_flops[MUON_KERNEL_COUNT] and
 * executed_flops[MUON_KERNEL_COUNT] (any of them may be NULL), and forgets
 * the recorded launches.  Nominal flops count the NS products a launch
 * computes on the unpadded oriented blocks m x n (m <= n): 2 m^2 n for
 * X X^T, 2 m^3 for A A, 2 m^2 n for B X, summed over the launch's blocks and,
 * for MUON_KERNEL_NS_LOOP, its iterations.  Executed flops count the matrix
 * core work of the tiles the launch ran: 2 t^2 K per t x t tile over its
 * reduction K (padding, the diagonal tiles of the symmetric products and
 * ACCURATE's three-segment B X included).  The other families report 0. */
muon_status muon_timing_collect(int64_t* launches, double* total_ms, double* nominal_flops,
                                double* executed_flops);

/* Text of the last error on the calling thread ("" if none).  Valid until
 * the next call into the library from that thread. */
const char* muon_last_error(void);

/* MUON_ABI_VERSION of the built library. */
int32_t muon_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_HIP_H */
