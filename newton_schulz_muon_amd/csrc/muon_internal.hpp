// Internal declarations of the batched Muon HIP library (gfx950).
//
// Data layout in device memory
//   Stored batches are row-major [batch][rows][cols].  With view_blocks = v the
//   NS block k of a stored matrix is its contiguous elements
//   [k*rows*cols/v, (k+1)*rows*cols/v) read as rows x (cols/v).
//   Inside the NS loop every block lives in "oriented, padded" form: an
//   mp x np bf16 tile-aligned matrix (mp, np multiples of 128) holding the
//   block (or its transpose when it is tall) in the top-left m x n corner and
//   exact zeros elsewhere.  Zero padding is invariant under the iteration
//   (zero rows of X give zero rows and columns of A and B, and B X keeps zero
//   columns of X zero), so the GEMM kernels never mask.
#pragma once

#include <hip/hip_runtime.h>
#include <vector>
#include <stdint.h>
#include <stddef.h>

#include "muon_hip.h"

namespace muon {

constexpr int kTile = 128;          // GEMM output tile edge and padding unit
constexpr int kEwTile = 64;         // element-wise kernels' tile edge
constexpr int kSmallMaxM = 64;      // small fp32 path: m <= 64 ...
constexpr int kSmallMaxElems = 8192;  // ... and m * n <= 8192
constexpr int64_t kMaxGridY = 65535;

struct Plan {
    int64_t batch = 0, R = 0, C = 0;
    int32_t v = 1;
    int64_t nb = 0;              // NS blocks = batch * v
    int64_t r = 0, c = 0;        // NS block shape as stored
    int64_t m = 0, n = 0;        // min / max side
    bool tall = false;           // r > c: oriented form is the transpose
    bool small = false;          // fp32 one-workgroup-per-block path
    int64_t mp = 0, np = 0;      // padded oriented shape
    int32_t precision = MUON_PRECISION_FAST;
    int64_t ew_tiles = 0;        // 64 x 64 tiles per padded block (norm partial slots)
    int64_t trace_stride = 0;    // floats per block of the trace partials (mp / 32 rounded up to 32)
    // workspace byte offsets
    size_t off_x[2] = {0, 0};    // iterate ping-pong, bf16 [nb][mp][np] (hi plane)
    size_t off_xlo[2] = {0, 0};  // ACCURATE: lo planes
    size_t off_a = 0;            // Gram, bf16 [nb][mp][mp]
    size_t off_b = 0;            // polynomial, bf16 [nb][mp][mp] (hi plane)
    size_t off_blo = 0;          // ACCURATE: lo plane of B
    size_t off_part = 0;         // fp32 [nb][ew_tiles] partial sums of squares
    size_t off_scale = 0;        // fp32 [nb][2]: 1/s, 1/s^2 (the zero-iteration normalisation)
    size_t off_trace = 0;        // fp32 [nb][trace_stride]: traces of X X^T's diagonal 32 x 32 blocks
    size_t off_sync = 0;         // u32 counters of the persistent NS loop (ns_loop_sync_bytes)
    size_t total = 0;
};

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------- launchers
// Per-matrix addressing of one element-wise or small-block launch.  n == 0:
// the batch is strided (each operand's base + block * r * c).  n > 0: matrix
// i of the launch (i < n <= kTabMax) has its own buffers, NS block b is
// sub-block b % v of matrix b / v, and the update scalars are per matrix.
constexpr int kTabMax = 32;
struct MatTable {
    int n = 0;
    int v = 1;
    const uint16_t* src[kTabMax];   // gradients (or x)
    float* mom[kTabMax];            // momentum buffers
    float* P[kTabMax];              // parameters
    uint16_t* out[kTabMax];         // NS output / optional O (entries may be null)
    float decay[kTabMax];           // 1 - lr wd wd_mul
    float step[kTabMax];            // lr aspect lr_mul
};

// Element-wise kernels (muon_elementwise.hip).
enum PrepMode { kPrepCast = 0, kPrepNesterov = 1, kPrepPlain = 2 };

// Reads the stored batch (bf16 x or gradients), updates the momentum buffer
// (momentum modes), writes the oriented padded iterate X0 (bf16 hi plane; lo
// plane too when x_lo != nullptr; nothing when x_hi is null, for a wide block
// read in place) and per-tile sums of squares.  When status is non-null the
// launch also clears the call's two status words.
hipError_t launch_prep(const Plan& p, PrepMode mode, const uint16_t* src, float* mom, float mu,
                       uint16_t* x_hi, uint16_t* x_lo, float* partials, uint32_t* status, hipStream_t s,
                       const MatTable* tab = nullptr);
// scales[2k] = 1/(sqrt(sum_k) + eps), scales[2k+1] = scales[2k]^2.
hipError_t launch_norm_finalize(const Plan& p, const float* partials, float* scales, float eps,
                                hipStream_t s);
// Writes the final iterate back in stored layout: NS output (out, bf16) or the
// parameter update P <- P*decay - step*O (with optional O).  `scale` (may be
// null) multiplies X first (used when ns_steps == 0).
hipError_t launch_finish(const Plan& p, const uint16_t* x_hi, const uint16_t* x_lo,
                         const float* scale, float* params, float decay, float step,
                         uint16_t* out, hipStream_t s, const MatTable* tab = nullptr);

// MFMA kernels (ns_gemm.hip).  Each launcher takes 1 to 4 products of one
// kind that share the reduction length; their tiles run in one launch (two
// when the last round is split into quadrants).
// In the first NS iteration `trace` points to the plan's norm partials (the
// Gram writes the traces of its diagonal 32 x 32 blocks there; the
// polynomial and B X derive s^-1 = 1 / (|X|_F + eps) from them); null later.
struct GramOp {
    const Plan* plan;
    const uint16_t* x;
    uint16_t* a;
    float* trace;
};
struct PolyOp {
    const Plan* plan;
    const uint16_t* a;
    uint16_t* b_hi;
    uint16_t* b_lo;
    const float* trace;
};
struct BxOp {
    const Plan* plan;
    const uint16_t* b_hi;
    const uint16_t* b_lo;
    const uint16_t* x_hi;
    const uint16_t* x_lo;
    uint16_t* out_hi;
    uint16_t* out_lo;
    const float* trace;
};
constexpr int kMaxGemmProblems = 4;
// MFMA flops the GEMM launchers below (and the persistent loop) enqueue,
// added up on the calling thread (timing diagnostics reset and read it).
double& last_exec_flops();
// status: null, or the call's two status words, which the Gram launch clears.
hipError_t launch_gram(const GramOp* ops, int n, uint32_t* status, hipStream_t s);
hipError_t launch_poly(const PolyOp* ops, int n, float ca, float cb, float cc, float eps, hipStream_t s);
hipError_t launch_bx(const BxOp* ops, int n, float eps, hipStream_t s);
// Single-product forms.  With `trace` (the first iteration), s^-1 = 1 / (sqrt(sum of the
// partials) + eps) as above.
// A = X X^T   (upper tiles computed, mirrored; with trace also the norm partials)
hipError_t launch_gram(const Plan& p, const uint16_t* x, uint16_t* a, float* trace, uint32_t* status,
                       hipStream_t s);
// B' = a I + b A + c A A, with trace a I + b s^-2 A + c s^-4 A A   (A symmetric; b_lo != nullptr
// stores the rounding residual)
hipError_t launch_poly(const Plan& p, const uint16_t* a, uint16_t* b_hi, uint16_t* b_lo,
                       float ca, float cb, float cc, const float* trace, float eps, hipStream_t s);
// X' = B' X, with trace s^-1 B' X   (a X is carried by the diagonal of B').
// ACCURATE when b_lo is given: X' = (s^-1) (Bh Xh + Bh Xl + Bl Xh), stored as hi + lo.
hipError_t launch_bx(const Plan& p, const uint16_t* b_hi, const uint16_t* b_lo, const uint16_t* x_hi,
                     const uint16_t* x_lo, uint16_t* out_hi, uint16_t* out_lo, const float* trace, float eps,
                     hipStream_t s);

// Persistent NS loop (ns_gemm.hip): every iteration of the three products
// of up to kMaxNsLoopProblems block batches in one launch of one workgroup
// per CU, which take tiles from a precomputed queue and wait on per-block
// completion counters.  Each problem brings a sync region of
// ns_loop_sync_bytes(nb) (the launch zeroes it first).  Iteration 0 reads x0,
// iteration t > 0 reads x[t % 2]; every iteration but the last writes
// x[(t + 1) % 2] and the last writes xlast; the first one writes and reads
// the norm partials `trace` as the per-product launches do.  ACCURATE adds the lo planes: iteration t
// reads xlo[t % 2] and writes xlo[(t + 1) % 2] (so x0 = x[0], xlast =
// x[ns_steps % 2] there), and B' is stored as b + blo.
struct NsLoopProblem {
    const Plan* plan;
    const uint16_t* x0;
    uint16_t* x[2];
    uint16_t* xlast;
    uint16_t* a;
    uint16_t* b;
    float* trace;           // the plan's norm partials (iteration 0)
    uint32_t* sync;
    uint16_t* xlo[2];       // ACCURATE: lo planes of the iterates (null for FAST)
    uint16_t* blo;          // ACCURATE: lo plane of B' (null for FAST)
};
constexpr int kMaxNsLoopProblems = 8;
// Queue entries the loop needs in the workspace for these block batches and
// step count: 0 when the loop does not take them (it needs one precision for
// all of them, both padded sides multiples of 256, 1 <= ns_steps <= 255, at
// most kMaxNsLoopProblems batches and at most 2^22 entries).
uint64_t ns_loop_items_cap(const Plan* const* plans, int n, int ns_steps);
bool ns_loop_eligible(const NsLoopProblem* probs, int n, int ns_steps);
// Which schedule runs the NS iterations of these problems on stream s (see
// set_ns_schedule), resolved before anything of the call is enqueued (it may
// build and cache the queues on the host); the caller launches it between
// begin and end.
struct NsChoice {
    bool persistent = false;
    int trial = -1;                            // timed trial call of the automatic choice
    const std::vector<int64_t>* key = nullptr;
    const void* sched = nullptr;               // the loop's queues (host)
    int cus = 0;                               // workgroups of the loop launch
};
NsChoice ns_schedule_begin(const NsLoopProblem* probs, int n, int ns_steps, hipStream_t s);
// Marks where the call's NS iterations start and end on stream s (the timed
// trials of the automatic choice record events there).
void ns_schedule_start(const NsChoice& c, hipStream_t s);
void ns_schedule_end(const NsChoice& c, hipStream_t s);
size_t ns_loop_sync_bytes(int64_t total_blocks);
// Enqueues the loop's setup (counters zeroed, queue copied from the pinned
// host copy into items_ws, which holds items_cap entries) and the loop.  An
// interrupted run NaN-fills the final iterates of the blocks it left
// incomplete and adds their count and its error flags to status[0], status[1].
// clear_status: the setup kernel clears the two status words first (when
// this launch is the call's first kernel).
hipError_t launch_ns_loop(const NsLoopProblem* probs, int n, int ns_steps, float ca, float cb, float cc, float eps,
                          const NsChoice& choice, uint2* items_ws, uint64_t items_cap, uint32_t* status,
                          bool clear_status, hipStream_t s);
// 0: automatic per set of shapes (default); 1: per-product launches only;
// 2: the persistent loop wherever eligible.
void set_ns_schedule(int mode);
// Diagnostics: 0 normal; 1 every loop launch sets its error word at its start;
// 2 every dependency wait of the loop that is not met at once times out.
void set_loop_fault(int mode);
// Tile width of the per-product launches: 0 by the cost model (default); 64,
// 128 or 256 where the block shapes allow it (256: padded sides multiples of
// 256; otherwise 128).
void set_gemm_tiling(int width);
// While one exists on a thread, per-product launches of that thread create,
// record and query no events for the automatic tiling choice (they use a
// settled choice or the estimate): for callers that may not allocate.
class TileTrialsOff {
public:
    TileTrialsOff();
    ~TileTrialsOff();
    TileTrialsOff(const TileTrialsOff&) = delete;
    TileTrialsOff& operator=(const TileTrialsOff&) = delete;
private:
    bool prev_;
};

// AdamW for the non-matrix parameters (adamw.hip): one launch over up to
// kAdamTab tensors.  decay = 1 - lr lr_mul wd wd_mul (exactly 1 when wd = 0),
// step = lr lr_mul (1 - beta2^t)^0.5 / (1 - beta1^t); vec: all four buffers
// 16-byte aligned.  first_chunk is filled in by the launcher.
constexpr int kAdamTab = 24;
struct AdamEntry {
    float* p;
    const uint16_t* g;
    float* m;
    float* v;
    int64_t numel;
    uint32_t first_chunk;
    int32_t vec;
    float decay, step;
};
int64_t adamw_chunks(int64_t numel);
hipError_t launch_adamw(const AdamEntry* entries, int n, float beta1, float beta2, float eps, hipStream_t s);

// Small blocks (small_ns.hip): the whole step for one block per workgroup in fp32.
struct SmallStep {
    const uint16_t* src = nullptr;   // x or gradients
    float* mom = nullptr;            // momentum buffer (step modes)
    float* params = nullptr;         // parameters (step modes)
    uint16_t* out = nullptr;         // NS output or optional O
    float mu = 0.f, decay = 1.f, step = 0.f;
    int mode = 0;                    // PrepMode
    int ns_steps = 5;
    float a = 0.f, b = 0.f, c = 0.f, eps = 0.f;
};
// With a table, src/mom/params/out/decay/step come from it (per matrix).
hipError_t launch_small(const Plan& p, const SmallStep& st, hipStream_t s, const MatTable* tab = nullptr);

}  // namespace muon
