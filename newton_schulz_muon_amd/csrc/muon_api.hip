// C ABI of the batched Muon library: argument validation, workspace plan and
// the launch sequence.  Host code only; the kernels live in the other sources.
//
// Launch sequence of one call (large blocks):
//   k_prep            momentum + cast to the oriented padded iterate + tile norms
//   k_norm_finalize   1/s and 1/s^2 per NS block
//   ns_steps x { k_gemm<kGram>, k_gemm<kPoly>, k_gemm<kBx> }   ping-pong between
//                     two iterates (kPoly forms B' = a I + b A + c A A, kBx
//                     X' = B' X);
//                     iteration 1 folds the normalisation into its epilogues
//                     (A = U U^T / s^2, X1 = B' U / s), so X0 = U / s is
//                     never materialised;
//                     or, by the NS schedule (muon_set_ns_schedule), one
//                     k_ns_loop launch running all iterations from a tile
//                     queue (after k_loop_setup zeroes its counters and copies
//                     the queue into the workspace from pinned host memory)
//   k_finish          NS output, or the parameter update (+ optional O)
// An NS-only call on wide blocks whose sides are tile multiples reads x in
// place (k_prep only sums squares) and its last iteration writes out directly
// (no k_finish).  The schedule and the queue are settled on the host before
// the first launch; the library allocates no device memory, and every launch
// and copy of a call goes to the caller's stream.
// Small blocks (m <= 64, m n <= 8192) run the whole step in one k_small launch.
// adamw_step_multi runs one k_adamw launch per 24 tensors.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "muon_internal.hpp"

namespace muon {
namespace {

thread_local std::string g_err;

muon_status fail(muon_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

muon_status hip_fail(hipError_t e, const char* what) {
    return fail(MUON_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

muon_ns_config default_config() {
    muon_ns_config c;
    c.ns_steps = 5;
    c.a = 3.4445f;
    c.b = -4.7750f;
    c.c = 2.0315f;
    c.eps = 1e-7f;
    c.precision = MUON_PRECISION_FAST;
    return c;
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

muon_status validate_config(const muon_ns_config& c) {
    if (c.ns_steps < 0 || c.ns_steps > 64)
        return fail(MUON_ERR_INVALID_ARG, "ns_steps %d outside [0, 64]", c.ns_steps);
    if (!std::isfinite(c.a) || !std::isfinite(c.b) || !std::isfinite(c.c))
        return fail(MUON_ERR_INVALID_ARG, "NS coefficients must be finite");
    if (!std::isfinite(c.eps) || c.eps < 0.f)
        return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (c.precision != MUON_PRECISION_FAST && c.precision != MUON_PRECISION_ACCURATE)
        return fail(MUON_ERR_INVALID_ARG, "unknown precision %d", c.precision);
    return MUON_OK;
}

muon_status make_plan(int64_t batch, int64_t rows, int64_t cols, int32_t v,
                      const muon_ns_config& cfg, Plan& p) {
    constexpr int64_t kMaxSide = int64_t(1) << 24;
    constexpr int64_t kMaxMinSide = 16384;
    if (batch < 0) return fail(MUON_ERR_SHAPE, "batch %lld < 0", (long long)batch);
    if (rows < 1 || cols < 1 || rows > kMaxSide || cols > kMaxSide)
        return fail(MUON_ERR_SHAPE, "rows %lld / cols %lld out of range", (long long)rows, (long long)cols);
    if (v < 1 || cols % v != 0)
        return fail(MUON_ERR_SHAPE, "view_blocks %d must be >= 1 and divide cols %lld", v, (long long)cols);
    p = Plan();
    p.batch = batch;
    p.R = rows;
    p.C = cols;
    p.v = v;
    p.nb = batch * v;
    if (p.nb > 0x7fffffffLL) return fail(MUON_ERR_SHAPE, "too many NS blocks");
    p.r = rows;
    p.c = cols / v;
    p.m = p.r < p.c ? p.r : p.c;
    p.n = p.r < p.c ? p.c : p.r;
    p.tall = p.r > p.c;
    if (p.r * p.c > 0x7fffffffLL) return fail(MUON_ERR_SHAPE, "NS block larger than 2^31 elements");
    p.precision = cfg.precision;
    p.small = p.m <= kSmallMaxM && p.m * p.n <= kSmallMaxElems;
    if (p.small) return MUON_OK;
    if (p.m > kMaxMinSide)
        return fail(MUON_ERR_SHAPE, "smaller side %lld exceeds %lld", (long long)p.m, (long long)kMaxMinSide);
    p.mp = round_up(p.m, kTile);
    p.np = round_up(p.n, kTile);
    if (p.mp * p.np > 0x7fffffffLL) return fail(MUON_ERR_SHAPE, "padded NS block larger than 2^31 elements");
    p.ew_tiles = (p.mp / kEwTile) * (p.np / kEwTile);
    const bool split = cfg.precision == MUON_PRECISION_ACCURATE;
    const double xb = double(p.nb) * double(p.mp) * double(p.np) * 2.0;
    const double ab = double(p.nb) * double(p.mp) * double(p.mp) * 2.0;
    if (xb * 4 + ab * 3 > 1e15) return fail(MUON_ERR_SHAPE, "workspace would exceed 1 PB");
    size_t off = 0;
    const size_t xbytes = size_t(p.nb) * size_t(p.mp) * size_t(p.np) * 2;
    const size_t abytes = size_t(p.nb) * size_t(p.mp) * size_t(p.mp) * 2;
    for (int i = 0; i < 2; ++i) { p.off_x[i] = off; off = align256(off + xbytes); }
    if (split)
        for (int i = 0; i < 2; ++i) { p.off_xlo[i] = off; off = align256(off + xbytes); }
    p.off_a = off; off = align256(off + abytes);
    p.off_b = off; off = align256(off + abytes);
    if (split) { p.off_blo = off; off = align256(off + abytes); }
    p.off_part = off; off = align256(off + size_t(p.nb) * size_t(p.ew_tiles) * 4);
    p.off_scale = off; off = align256(off + size_t(p.nb) * 2 * 4);
    p.trace_stride = round_up(p.mp / 32, 32);
    p.off_trace = off; off = align256(off + size_t(p.nb) * size_t(p.trace_stride) * 4);
    p.off_sync = off; off += ns_loop_sync_bytes(p.nb);
    p.total = off;
    return MUON_OK;
}

muon_status check_device() {
    static std::atomic<int> cache[64];
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int state = (dev >= 0 && dev < 64) ? cache[dev].load() : 0;
    if (state == 0) {
        hipDeviceProp_t prop;
        const hipError_t e2 = hipGetDeviceProperties(&prop, dev);
        if (e2 != hipSuccess) return hip_fail(e2, "hipGetDeviceProperties");
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (dev >= 0 && dev < 64) cache[dev].store(state);
        if (state == 2)
            return fail(MUON_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (state == 2) return fail(MUON_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return MUON_OK;
}

// ---------------------------------------------------------------- kernel timing
struct TimingState {
    std::mutex mu;
    std::atomic<uint32_t> mask{0};
    std::map<int, std::vector<hipEvent_t>> pool;   // per device
    struct Rec { int kind; int dev; hipEvent_t a, b; double flops, exec; };
    std::vector<Rec> recs;
};

TimingState& timing() {
    static TimingState* t = new TimingState();   // never destroyed: events outlive static teardown
    return *t;
}

hipEvent_t pool_get(TimingState& ts, int dev) {
    auto& v = ts.pool[dev];
    if (!v.empty()) {
        hipEvent_t e = v.back();
        v.pop_back();
        return e;
    }
    // Timing only: without the system-scope fence a record does not write back
    // and invalidate caches, which would otherwise slow the bracketed launch.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Records an event pair around one launch when its kernel family is selected,
// with the nominal flops of the products the launch computes.
// Set for the duration of a call that must not create timing events (the
// no-allocation entry point).
thread_local bool g_timing_off = false;

class LaunchTimer {
  public:
    LaunchTimer(int kind, hipStream_t s, double flops) : kind_(kind), s_(s), flops_(flops) {
        last_exec_flops() = 0.0;
        TimingState& ts = timing();
        if (g_timing_off || !(ts.mask.load() & (1u << kind))) return;
        std::lock_guard<std::mutex> lk(ts.mu);
        if (hipGetDevice(&dev_) != hipSuccess) return;
        a_ = pool_get(ts, dev_);
        b_ = pool_get(ts, dev_);
        if (a_ && b_ && hipEventRecord(a_, s_) == hipSuccess) on_ = true;
    }
    void stop() {
        if (!on_) return;
        on_ = false;
        TimingState& ts = timing();
        std::lock_guard<std::mutex> lk(ts.mu);
        if (hipEventRecord(b_, s_) == hipSuccess) ts.recs.push_back({kind_, dev_, a_, b_, flops_, last_exec_flops()});
    }
    ~LaunchTimer() { stop(); }

  private:
    int kind_;
    hipStream_t s_;
    double flops_;
    int dev_ = 0;
    hipEvent_t a_ = nullptr, b_ = nullptr;
    bool on_ = false;
};

template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& f, double flops = 0.0) {
    LaunchTimer t(kind, s, flops);
    const hipError_t e = f();
    t.stop();
    return e;
}

// Nominal flops of one NS product over a plan's blocks, on the unpadded
// oriented block m x n (m <= n): X X^T 2 m^2 n, A A 2 m^3, B X 2 m^2 n.
// The polynomial's b A and a X terms and the symmetric products' skipped
// tiles are not counted, nor the extra products of the hi/lo precision.
double product_flops(const Plan& p, int kind) {
    const double m = double(p.m), n = double(p.n), nb = double(p.nb);
    switch (kind) {
        case MUON_KERNEL_GRAM: return nb * 2.0 * m * m * n;
        case MUON_KERNEL_POLY: return nb * 2.0 * m * m * m;
        case MUON_KERNEL_BX: return nb * 2.0 * m * m * n;
        default: return 0.0;
    }
}
double ns_flops(const Plan& p, int steps) {
    return double(steps) * (product_flops(p, MUON_KERNEL_GRAM) + product_flops(p, MUON_KERNEL_POLY) +
                            product_flops(p, MUON_KERNEL_BX));
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bn && b0 < a0 + an;
}

// Every workspace starts with a 256-byte header: word 0 counts the NS blocks
// whose persistent-loop iteration did not complete in the last call that used
// the workspace (their outputs are NaN), word 1 holds that call's error flags.
// The call's first kernel clears both.  The plan regions follow the header.
constexpr size_t kHeaderBytes = 256;

struct Buffers {
    uint16_t* xh[2];
    uint16_t* xl[2];
    uint16_t* a;
    uint16_t* bh;
    uint16_t* bl;
    float* part;
    float* scale;
    float* trace;
    uint32_t* sync;
};

Buffers carve(const Plan& p, void* ws) {
    char* base = static_cast<char*>(ws);
    const bool split = p.precision == MUON_PRECISION_ACCURATE;
    Buffers b;
    for (int i = 0; i < 2; ++i) {
        b.xh[i] = reinterpret_cast<uint16_t*>(base + p.off_x[i]);
        b.xl[i] = split ? reinterpret_cast<uint16_t*>(base + p.off_xlo[i]) : nullptr;
    }
    b.a = reinterpret_cast<uint16_t*>(base + p.off_a);
    b.bh = reinterpret_cast<uint16_t*>(base + p.off_b);
    b.bl = split ? reinterpret_cast<uint16_t*>(base + p.off_blo) : nullptr;
    b.part = reinterpret_cast<float*>(base + p.off_part);
    b.scale = reinterpret_cast<float*>(base + p.off_scale);
    b.trace = reinterpret_cast<float*>(base + p.off_trace);
    b.sync = reinterpret_cast<uint32_t*>(base + p.off_sync);
    return b;
}

// Queue region of the persistent loop for these block batches: bytes (0 when
// the loop does not take them) and entries.
size_t loop_items_bytes(const Plan* const* plans, int n, int ns_steps, uint64_t* cap = nullptr) {
    const uint64_t c = ns_loop_items_cap(plans, n, ns_steps);
    if (cap) *cap = c;
    return align256(size_t(c) * 8);
}

// Layout of a single-batch call's workspace: header, plan regions, queue.
struct BatchedLayout {
    size_t items_off = 0;
    uint64_t items_cap = 0;
    size_t total = 0;
};
BatchedLayout batched_layout(const Plan& p, int ns_steps) {
    BatchedLayout l;
    if (p.small || p.nb == 0) return l;
    const Plan* pp = &p;
    const size_t ib = loop_items_bytes(&pp, 1, ns_steps, &l.items_cap);
    l.items_off = kHeaderBytes + p.total;
    l.total = kHeaderBytes + p.total + ib;
    return l;
}

// The iterate a call starts from and the buffer its last iteration writes.
// A wide block whose sides are already multiples of the tile (r = mp,
// c / v = np) is laid out in the caller's bf16 buffer exactly as the
// oriented padded iterate, so NS-only calls in FAST precision read x in
// place (the prep pass then only sums squares) and the last iteration writes
// the caller's output directly (no write-back pass).  With one iteration and
// out == x the output would overwrite operands still being read, so that
// case writes the workspace and copies back.
struct NsEnds {
    const uint16_t* x0;
    uint16_t* xlast;
    bool direct_in = false, direct_out = false;
};
NsEnds ns_ends(const Plan& p, const muon_ns_config& cfg, const Buffers& b, const void* x, void* out) {
    NsEnds e;
    e.x0 = b.xh[0];
    e.xlast = b.xh[cfg.ns_steps & 1];
    const bool exact = !p.small && !p.tall && p.precision == MUON_PRECISION_FAST && p.r == p.mp && p.c == p.np;
    if (x != nullptr && exact && cfg.ns_steps >= 1) {
        e.direct_in = true;
        e.x0 = static_cast<const uint16_t*>(x);
        if (out != nullptr && (cfg.ns_steps >= 2 || out != x)) {
            e.direct_out = true;
            e.xlast = static_cast<uint16_t*>(out);
        }
    }
    return e;
}

// Runs the NS iterations on an iterate already prepared by k_prep (e.x0: in
// xh[0] and xl[0], or the caller's x in place) with the schedule resolved
// before the call enqueued anything.  The first iteration's Gram also yields
// the norm |X|_F^2 = trace(X X^T) (partials in b.trace); with no iteration
// the prep's sums of squares are finalized instead (for k_finish).
// clear_status: the first kernel enqueued here clears the call's status
// words (no prep did).  Returns the buffer index of the result (when it is
// not e.xlast outside the workspace).
muon_status run_ns(const Plan& p, const muon_ns_config& cfg, const Buffers& b, const NsEnds& ends,
                   const NsChoice& ch, uint2* items, uint64_t items_cap, uint32_t* status, bool clear_status,
                   hipStream_t s, int* final_idx) {
    hipError_t e = hipSuccess;
    *final_idx = cfg.ns_steps & 1;
    if (cfg.ns_steps == 0) {
        e = timed(MUON_KERNEL_NORM_FINALIZE, s, [&] { return launch_norm_finalize(p, b.part, b.scale, cfg.eps, s); });
        return e == hipSuccess ? MUON_OK : hip_fail(e, "k_norm_finalize launch");
    }
    ns_schedule_start(ch, s);
    if (ch.persistent) {
        const NsLoopProblem lp{&p, ends.x0, {b.xh[0], b.xh[1]}, ends.xlast, b.a, b.bh, b.trace, b.sync, {b.xl[0], b.xl[1]}, b.bl};
        e = timed(MUON_KERNEL_NS_LOOP, s, [&] {
            return launch_ns_loop(&lp, 1, cfg.ns_steps, cfg.a, cfg.b, cfg.c, cfg.eps, ch, items, items_cap, status,
                                  clear_status, s);
        }, ns_flops(p, cfg.ns_steps));
        if (e != hipSuccess) return hip_fail(e, "k_ns_loop launch");
        ns_schedule_end(ch, s);
        return MUON_OK;
    }
    for (int it = 0; it < cfg.ns_steps; ++it) {
        const int cur = it & 1;
        float* tr = it == 0 ? b.trace : nullptr;
        const uint16_t* xin = it == 0 ? ends.x0 : b.xh[cur];
        uint16_t* xout = it + 1 == cfg.ns_steps ? ends.xlast : b.xh[cur ^ 1];
        uint32_t* clr = it == 0 && clear_status ? status : nullptr;
        e = timed(MUON_KERNEL_GRAM, s, [&] { return launch_gram(p, xin, b.a, tr, clr, s); },
                  product_flops(p, MUON_KERNEL_GRAM));
        if (e != hipSuccess) return hip_fail(e, "k_gemm<gram> launch");
        e = timed(MUON_KERNEL_POLY, s, [&] {
            return launch_poly(p, b.a, b.bh, b.bl, cfg.a, cfg.b, cfg.c, tr, cfg.eps, s);
        }, product_flops(p, MUON_KERNEL_POLY));
        if (e != hipSuccess) return hip_fail(e, "k_gemm<poly> launch");
        e = timed(MUON_KERNEL_BX, s, [&] {
            return launch_bx(p, b.bh, b.bl, xin, b.xl[cur], xout, b.xl[cur ^ 1], tr, cfg.eps, s);
        }, product_flops(p, MUON_KERNEL_BX));
        if (e != hipSuccess) return hip_fail(e, "k_gemm<bx> launch");
    }
    ns_schedule_end(ch, s);
    return MUON_OK;
}

muon_status common_checks(size_t need, void* ws, size_t ws_bytes) {
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return fail(MUON_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? ws_bytes : 0, need);
        if (!aligned(ws, 256)) return fail(MUON_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
    }
    return MUON_OK;
}


// ---------------------------------------------------------------- multi-matrix step
// Matrices of one (rows, cols, view_blocks) shape, stepped as one batch.
struct ShapeGroup {
    int64_t R = 0, C = 0;
    int32_t v = 1;
    std::vector<int32_t> mats;   // indices into the caller's array
    Plan plan;
    int wave = 0;          // groups of one wave run their NS loops together
    size_t ws_off = 0;     // offset of its workspace within the (shared) wave region
};

// Working-set budget of one wave: the NS workspaces of the groups that share
// launches stay resident in the 256 MB Infinity Cache only if together they
// fit well inside it (interleaving two groups of 141 MB and 234 MB measured
// slower than running them one after the other).
constexpr size_t kWaveBudget = size_t(160) << 20;

// One wave of a multi-matrix call: its groups' plan regions follow the
// workspace header, then the persistent loop's queue for all of them.
struct WavePlan {
    int64_t mp = 0;
    size_t bytes = 0;        // plan regions
    int n = 0;               // groups
    size_t items_off = 0;    // queue region (from the workspace start)
    uint64_t items_cap = 0;  // its entries (0: the loop does not take this wave)
};

muon_status plan_multi(const muon_matrix* mats, int32_t count, const muon_ns_config& cfg,
                       std::vector<ShapeGroup>& groups, std::vector<WavePlan>& waves, size_t& total) {
    groups.clear();
    waves.clear();
    total = 0;
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count %d < 0", count);
    if (count > 0 && mats == nullptr) return fail(MUON_ERR_INVALID_ARG, "matrices must be non-null");
    std::map<std::tuple<int64_t, int64_t, int32_t>, size_t> index;
    for (int32_t i = 0; i < count; ++i) {
        const muon_matrix& m = mats[i];
        Plan probe;
        const muon_status st = make_plan(1, m.rows, m.cols, m.view_blocks, cfg, probe);
        if (st != MUON_OK) return fail(st, "matrix %d: %s", i, g_err.c_str());
        const auto key = std::make_tuple(m.rows, m.cols, m.view_blocks);
        auto it = index.find(key);
        if (it == index.end()) {
            it = index.emplace(key, groups.size()).first;
            ShapeGroup g;
            g.R = m.rows;
            g.C = m.cols;
            g.v = m.view_blocks;
            groups.push_back(g);
        }
        groups[it->second].mats.push_back(i);
    }
    for (ShapeGroup& g : groups) {
        const muon_status st = make_plan(int64_t(g.mats.size()), g.R, g.C, g.v, cfg, g.plan);
        if (st != MUON_OK) return st;
    }
    // Waves: a large group joins the first wave of its padded side m (the
    // products share launches by m) whose workspace stays within the budget
    // and which has room for it; else it opens a new wave.  Waves run one
    // after the other and reuse one workspace region.
    for (ShapeGroup& g : groups) {
        if (g.plan.small) continue;
        const size_t need = align256(g.plan.total);
        int w = -1;
        for (size_t k = 0; k < waves.size() && w < 0; ++k)
            if (waves[k].mp == g.plan.mp && waves[k].n < kMaxGemmProblems && waves[k].bytes + need <= kWaveBudget)
                w = int(k);
        if (w < 0) {
            w = int(waves.size());
            waves.push_back(WavePlan());
            waves.back().mp = g.plan.mp;
        }
        g.wave = w;
        g.ws_off = kHeaderBytes + waves[w].bytes;
        waves[w].bytes += need;
        waves[w].n += 1;
    }
    for (size_t w = 0; w < waves.size(); ++w) {
        const Plan* plans[kMaxGemmProblems];
        int n = 0;
        for (const ShapeGroup& g : groups)
            if (!g.plan.small && g.wave == int(w)) plans[n++] = &g.plan;
        WavePlan& wp = waves[w];
        const size_t ib = loop_items_bytes(plans, n, cfg.ns_steps, &wp.items_cap);
        wp.items_off = kHeaderBytes + wp.bytes;
        total = std::max(total, kHeaderBytes + wp.bytes + ib);
    }
    return MUON_OK;
}

// Vector-path blocks (not small, block width a multiple of 8) are read and
// written in 16-byte pieces; the others element by element.
muon_status check_multi_buffers(const muon_matrix* mats, int32_t count, const std::vector<ShapeGroup>& groups,
                                const void* workspace, size_t ws_bytes) {
    struct Range { uintptr_t a, b; int32_t mat; };
    std::vector<Range> ranges;
    ranges.reserve(size_t(count) * 4);
    std::vector<char> vec16(size_t(count), 0);
    for (const ShapeGroup& g : groups)
        for (int32_t i : g.mats) vec16[i] = !g.plan.small && g.plan.c % 8 == 0;
    for (int32_t i = 0; i < count; ++i) {
        const muon_matrix& m = mats[i];
        if (!m.params || !m.grads || !m.momentum_buf)
            return fail(MUON_ERR_INVALID_ARG, "matrix %d: params, grads and momentum_buf must be non-null", i);
        const uintptr_t a32 = vec16[i] ? 16 : 4, a16 = vec16[i] ? 16 : 2;
        if (!aligned(m.params, a32) || !aligned(m.grads, a16) || !aligned(m.momentum_buf, a32) ||
            (m.update_out && !aligned(m.update_out, a16)))
            return fail(MUON_ERR_ALIGNMENT, "matrix %d: data pointers must be %s aligned", i,
                        vec16[i] ? "16-byte" : "element-");
        if (!std::isfinite(m.lr_mul) || !std::isfinite(m.wd_mul))
            return fail(MUON_ERR_INVALID_ARG, "matrix %d: lr_mul and wd_mul must be finite", i);
        const size_t n = size_t(m.rows) * size_t(m.cols);
        auto add = [&](const void* p, size_t bytes) {
            const uintptr_t a = reinterpret_cast<uintptr_t>(p);
            ranges.push_back({a, a + bytes, i});
        };
        add(m.params, 4 * n);
        add(m.grads, 2 * n);
        add(m.momentum_buf, 4 * n);
        if (m.update_out) add(m.update_out, 2 * n);
    }
    if (workspace != nullptr && ws_bytes > 0) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(workspace);
        ranges.push_back({a, a + ws_bytes, -1});
    }
    std::sort(ranges.begin(), ranges.end(), [](const Range& x, const Range& y) { return x.a < y.a; });
    for (size_t k = 1; k < ranges.size(); ++k)
        if (ranges[k].a < ranges[k - 1].b)
            return (ranges[k - 1].mat < 0 || ranges[k].mat < 0)
                       ? fail(MUON_ERR_INVALID_ARG, "the workspace overlaps buffers of matrix %d",
                              ranges[k - 1].mat < 0 ? ranges[k].mat : ranges[k - 1].mat)
                       : fail(MUON_ERR_INVALID_ARG, "buffers of matrices %d and %d overlap", ranges[k - 1].mat,
                              ranges[k].mat);
    return MUON_OK;
}

// Offsets a group's buffers to the blocks of matrices [m0, m0 + cnt).
Buffers chunk_buffers(const Plan& p, const Buffers& b, int64_t m0) {
    Buffers c = b;
    const int64_t blk0 = m0 * p.v;
    const size_t xe = size_t(p.mp) * size_t(p.np);
    for (int i = 0; i < 2; ++i) {
        c.xh[i] = b.xh[i] + blk0 * xe;
        c.xl[i] = b.xl[i] ? b.xl[i] + blk0 * xe : nullptr;
    }
    c.part = b.part + blk0 * p.ew_tiles;
    c.scale = b.scale + 2 * blk0;
    c.trace = b.trace + blk0 * p.trace_stride;
    return c;
}

Plan chunk_plan(const Plan& p, int64_t cnt) {
    Plan c = p;
    c.batch = cnt;
    c.nb = cnt * p.v;
    return c;
}

MatTable make_table(const muon_matrix* mats, const ShapeGroup& g, size_t m0, size_t cnt, float lr, float wd,
                    double aspect) {
    MatTable t;
    t.n = static_cast<int>(cnt);
    t.v = g.v;
    for (size_t k = 0; k < cnt; ++k) {
        const muon_matrix& m = mats[g.mats[m0 + k]];
        t.src[k] = static_cast<const uint16_t*>(m.grads);
        t.mom[k] = m.momentum_buf;
        t.P[k] = m.params;
        t.out[k] = static_cast<uint16_t*>(m.update_out);
        t.decay[k] = static_cast<float>(1.0 - double(lr) * double(wd) * double(m.wd_mul));
        t.step[k] = static_cast<float>(double(lr) * aspect * double(m.lr_mul));
    }
    return t;
}

// ---------------------------------------------------------------- no-allocation scratch
// Scratch memory of ns_orthogonalize_batched_noalloc, for callers that cannot
// allocate (code under graph capture, tight serving loops): one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory; the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = size_t(MUON_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

muon_status scratch_of_current_device(void** out) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MUON_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        const hipError_t e2 = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e2 != hipSuccess) return hip_fail(e2, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr || !aligned(ptr, 256)) return fail(MUON_ERR_HIP, "scratch symbol has no usable address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MUON_OK;
}

// ns_orthogonalize_batched; with per_product_only the persistent loop (whose
// queue lives in pinned host memory the first call allocates) is not used.
muon_status ns_batched_impl(const void* x, void* out, int64_t batch, int64_t rows, int64_t cols, int32_t view_blocks,
                            const muon_ns_config* cfg_in, void* workspace, size_t workspace_bytes, void* stream,
                            bool per_product_only) {
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    muon_status st = validate_config(cfg);
    if (st != MUON_OK) return st;
    Plan p;
    st = make_plan(batch, rows, cols, view_blocks, cfg, p);
    if (st != MUON_OK) return st;
    if (batch == 0) return MUON_OK;
    if (!x || !out) return fail(MUON_ERR_INVALID_ARG, "x and out must be non-null");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(MUON_ERR_ALIGNMENT, "x and out must be 16-byte aligned");
    const size_t bytes = size_t(batch) * size_t(rows) * size_t(cols) * 2;
    if (x != out && overlaps(x, bytes, out, bytes))
        return fail(MUON_ERR_INVALID_ARG, "out overlaps x without being x");
    BatchedLayout lay = batched_layout(p, cfg.ns_steps);
    if (per_product_only && lay.total > 0) {
        lay.total = kHeaderBytes + p.total;
        lay.items_cap = 0;
    }
    st = common_checks(lay.total, workspace, workspace_bytes);
    if (st != MUON_OK) return st;
    if (lay.total > 0 && (overlaps(workspace, lay.total, x, bytes) || overlaps(workspace, lay.total, out, bytes)))
        return fail(MUON_ERR_INVALID_ARG, "workspace overlaps x or out");
    st = check_device();
    if (st != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);

    if (p.small) {
        SmallStep ss;
        ss.src = static_cast<const uint16_t*>(x);
        ss.out = static_cast<uint16_t*>(out);
        ss.mode = kPrepCast;
        ss.ns_steps = cfg.ns_steps;
        ss.a = cfg.a;
        ss.b = cfg.b;
        ss.c = cfg.c;
        ss.eps = cfg.eps;
        const hipError_t e = timed(MUON_KERNEL_SMALL, s, [&] { return launch_small(p, ss, s); });
        return e == hipSuccess ? MUON_OK : hip_fail(e, "k_small launch");
    }
    char* ws = static_cast<char*>(workspace);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws);
    const Buffers b = carve(p, ws + kHeaderBytes);
    const NsEnds ends = ns_ends(p, cfg, b, x, out);
    // The schedule (and on first use its queue) is settled before anything is enqueued.
    const NsLoopProblem lp{&p, ends.x0, {b.xh[0], b.xh[1]}, ends.xlast, b.a, b.bh, b.trace, b.sync, {b.xl[0], b.xl[1]}, b.bl};
    const NsChoice ch = per_product_only ? NsChoice() : ns_schedule_begin(&lp, 1, cfg.ns_steps, s);
    hipError_t e = hipSuccess;
    // With x read in place there is nothing to prepare: the first Gram also
    // yields the norm.
    if (!ends.direct_in) {
        e = timed(MUON_KERNEL_PREP, s, [&] {
            return launch_prep(p, kPrepCast, static_cast<const uint16_t*>(x), nullptr, 0.f, b.xh[0], b.xl[0],
                               cfg.ns_steps == 0 ? b.part : nullptr, status, s);
        });
        if (e != hipSuccess) return hip_fail(e, "k_prep launch");
    }
    int fin = 0;
    st = run_ns(p, cfg, b, ends, ch, reinterpret_cast<uint2*>(ws + lay.items_off), lay.items_cap, status,
                ends.direct_in, s, &fin);
    if (st != MUON_OK) return st;
    if (ends.direct_out) return MUON_OK;
    e = timed(MUON_KERNEL_FINISH, s, [&] {
        return launch_finish(p, b.xh[fin], b.xl[fin], cfg.ns_steps == 0 ? b.scale : nullptr, nullptr, 1.f, 0.f,
                             static_cast<uint16_t*>(out), s);
    });
    return e == hipSuccess ? MUON_OK : hip_fail(e, "k_finish launch");
}

}  // namespace
}  // namespace muon

using namespace muon;

extern "C" {

void muon_ns_config_default(muon_ns_config* cfg) {
    if (cfg) *cfg = default_config();
}

size_t muon_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t view_blocks,
                            const muon_ns_config* cfg_in) {
    g_err.clear();
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    if (validate_config(cfg) != MUON_OK) return size_t(-1);
    Plan p;
    if (make_plan(batch, rows, cols, view_blocks, cfg, p) != MUON_OK) return size_t(-1);
    if (batch == 0) return 0;
    return batched_layout(p, cfg.ns_steps).total;
}

muon_status ns_orthogonalize_batched(const void* x, void* out, int64_t batch, int64_t rows,
                                     int64_t cols, int32_t view_blocks, const muon_ns_config* cfg_in,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    return ns_batched_impl(x, out, batch, rows, cols, view_blocks, cfg_in, workspace, workspace_bytes, stream,
                           false);
}

muon_status ns_orthogonalize_batched_noalloc(const void* x, void* out, int64_t batch, int64_t rows, int64_t cols,
                                             int32_t view_blocks, const muon_ns_config* cfg_in, void* stream) {
    g_err.clear();
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    muon_status st = validate_config(cfg);
    if (st != MUON_OK) return st;
    Plan p;
    st = make_plan(batch, rows, cols, view_blocks, cfg, p);
    if (st != MUON_OK) return st;
    if (batch == 0) return MUON_OK;
    // This entry point runs the per-product schedule only, which needs no
    // queue region.
    const size_t need = p.small ? 0 : kHeaderBytes + p.total;
    if (need > kScratchBytes)
        return fail(MUON_ERR_WORKSPACE,
                    "this batch needs %zu bytes of scratch; the no-allocation entry point has %zu (use "
                    "ns_orthogonalize_batched with a workspace)", need, kScratchBytes);
    st = check_device();
    if (st != MUON_OK) return st;
    void* ws = nullptr;
    if (need > 0) {
        st = scratch_of_current_device(&ws);
        if (st != MUON_OK) return st;
    }
    struct TimingOff {
        TimingOff() { g_timing_off = true; }
        ~TimingOff() { g_timing_off = false; }
    } no_events;
    const TileTrialsOff no_tile_events;
    return ns_batched_impl(x, out, batch, rows, cols, view_blocks, cfg_in, ws, need, stream, true);
}

muon_status muon_step_batched(float* params, const void* grads, float* momentum_buf, int64_t batch,
                              int64_t rows, int64_t cols, int32_t view_blocks, float lr,
                              float weight_decay, float momentum, int32_t nesterov, float lr_mul,
                              float wd_mul, const muon_ns_config* cfg_in, void* update_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    muon_status st = validate_config(cfg);
    if (st != MUON_OK) return st;
    Plan p;
    st = make_plan(batch, rows, cols, view_blocks, cfg, p);
    if (st != MUON_OK) return st;
    if (!std::isfinite(lr) || !std::isfinite(weight_decay) || !std::isfinite(lr_mul) || !std::isfinite(wd_mul))
        return fail(MUON_ERR_INVALID_ARG, "lr, weight_decay, lr_mul and wd_mul must be finite");
    if (!(momentum >= 0.f && momentum <= 1.f)) return fail(MUON_ERR_INVALID_ARG, "momentum must be in [0, 1]");
    if (batch == 0) return MUON_OK;
    if (!params || !grads || !momentum_buf)
        return fail(MUON_ERR_INVALID_ARG, "params, grads and momentum_buf must be non-null");
    if (!aligned(params, 16) || !aligned(grads, 16) || !aligned(momentum_buf, 16) ||
        (update_out && !aligned(update_out, 16)))
        return fail(MUON_ERR_ALIGNMENT, "data pointers must be 16-byte aligned");
    const size_t n = size_t(batch) * size_t(rows) * size_t(cols);
    if (overlaps(params, 4 * n, grads, 2 * n) || overlaps(params, 4 * n, momentum_buf, 4 * n) ||
        overlaps(grads, 2 * n, momentum_buf, 4 * n) || overlaps(update_out, 2 * n, params, 4 * n) ||
        overlaps(update_out, 2 * n, grads, 2 * n) || overlaps(update_out, 2 * n, momentum_buf, 4 * n))
        return fail(MUON_ERR_INVALID_ARG, "params, grads, momentum_buf and update_out must not overlap");
    const BatchedLayout lay = batched_layout(p, cfg.ns_steps);
    st = common_checks(lay.total, workspace, workspace_bytes);
    if (st != MUON_OK) return st;
    if (lay.total > 0 &&
        (overlaps(workspace, lay.total, params, 4 * n) || overlaps(workspace, lay.total, grads, 2 * n) ||
         overlaps(workspace, lay.total, momentum_buf, 4 * n) || overlaps(workspace, lay.total, update_out, 2 * n)))
        return fail(MUON_ERR_INVALID_ARG, "workspace overlaps a data buffer");
    st = check_device();
    if (st != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);

    const double aspect = std::sqrt(std::fmax(1.0, double(rows) / double(cols)));
    const float decay = static_cast<float>(1.0 - double(lr) * double(weight_decay) * double(wd_mul));
    const float step = static_cast<float>(double(lr) * aspect * double(lr_mul));
    const PrepMode mode = nesterov ? kPrepNesterov : kPrepPlain;

    if (p.small) {
        SmallStep ss;
        ss.src = static_cast<const uint16_t*>(grads);
        ss.mom = momentum_buf;
        ss.params = params;
        ss.out = static_cast<uint16_t*>(update_out);
        ss.mu = momentum;
        ss.decay = decay;
        ss.step = step;
        ss.mode = mode;
        ss.ns_steps = cfg.ns_steps;
        ss.a = cfg.a;
        ss.b = cfg.b;
        ss.c = cfg.c;
        ss.eps = cfg.eps;
        const hipError_t e = timed(MUON_KERNEL_SMALL, s, [&] { return launch_small(p, ss, s); });
        return e == hipSuccess ? MUON_OK : hip_fail(e, "k_small launch");
    }
    char* ws = static_cast<char*>(workspace);
    uint32_t* status = reinterpret_cast<uint32_t*>(ws);
    const Buffers b = carve(p, ws + kHeaderBytes);
    const NsEnds ends = ns_ends(p, cfg, b, nullptr, nullptr);
    const NsLoopProblem lp{&p, ends.x0, {b.xh[0], b.xh[1]}, ends.xlast, b.a, b.bh, b.trace, b.sync, {b.xl[0], b.xl[1]}, b.bl};
    const NsChoice ch = ns_schedule_begin(&lp, 1, cfg.ns_steps, s);
    hipError_t e = timed(MUON_KERNEL_PREP, s, [&] {
        return launch_prep(p, mode, static_cast<const uint16_t*>(grads), momentum_buf, momentum, b.xh[0], b.xl[0],
                           cfg.ns_steps == 0 ? b.part : nullptr, status, s);
    });
    if (e != hipSuccess) return hip_fail(e, "k_prep launch");
    int fin = 0;
    st = run_ns(p, cfg, b, ends, ch, reinterpret_cast<uint2*>(ws + lay.items_off), lay.items_cap, status, false, s,
                &fin);
    if (st != MUON_OK) return st;
    e = timed(MUON_KERNEL_FINISH, s, [&] {
        return launch_finish(p, b.xh[fin], b.xl[fin], cfg.ns_steps == 0 ? b.scale : nullptr, params, decay, step,
                             static_cast<uint16_t*>(update_out), s);
    });
    return e == hipSuccess ? MUON_OK : hip_fail(e, "k_finish launch");
}

size_t muon_step_multi_workspace_bytes(const muon_matrix* mats, int32_t count, const muon_ns_config* cfg_in) {
    g_err.clear();
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    if (validate_config(cfg) != MUON_OK) return size_t(-1);
    std::vector<ShapeGroup> groups;
    std::vector<WavePlan> waves;
    size_t total = 0;
    if (plan_multi(mats, count, cfg, groups, waves, total) != MUON_OK) return size_t(-1);
    return total;
}

muon_status muon_step_multi(const muon_matrix* mats, int32_t count, float lr, float weight_decay, float momentum,
                            int32_t nesterov, const muon_ns_config* cfg_in, void* workspace, size_t workspace_bytes,
                            void* stream) {
    g_err.clear();
    const muon_ns_config cfg = cfg_in ? *cfg_in : default_config();
    muon_status st = validate_config(cfg);
    if (st != MUON_OK) return st;
    if (!std::isfinite(lr) || !std::isfinite(weight_decay))
        return fail(MUON_ERR_INVALID_ARG, "lr and weight_decay must be finite");
    if (!(momentum >= 0.f && momentum <= 1.f)) return fail(MUON_ERR_INVALID_ARG, "momentum must be in [0, 1]");
    std::vector<ShapeGroup> groups;
    std::vector<WavePlan> waves;
    size_t total = 0;
    st = plan_multi(mats, count, cfg, groups, waves, total);
    if (st != MUON_OK) return st;
    if (count == 0) return MUON_OK;
    st = check_multi_buffers(mats, count, groups, total > 0 ? workspace : nullptr, total);
    if (st != MUON_OK) return st;
    st = common_checks(total, workspace, workspace_bytes);
    if (st != MUON_OK) return st;
    st = check_device();
    if (st != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const PrepMode mode = nesterov ? kPrepNesterov : kPrepPlain;
    char* ws = static_cast<char*>(workspace);
    uint32_t* status = total > 0 ? reinterpret_cast<uint32_t*>(ws) : nullptr;

    // Every wave's buffers and NS schedule, settled before anything is enqueued.
    const int nwaves = int(waves.size());
    std::vector<Buffers> bufs(groups.size());
    std::vector<std::vector<size_t>> wave_groups(nwaves);
    std::vector<std::vector<NsLoopProblem>> wave_lps(nwaves);
    std::vector<NsChoice> choices(nwaves);
    for (size_t gi = 0; gi < groups.size(); ++gi) {
        const ShapeGroup& g = groups[gi];
        if (g.plan.small) continue;
        bufs[gi] = carve(g.plan, ws + g.ws_off);
        const Buffers& bb = bufs[gi];
        wave_groups[g.wave].push_back(gi);
        wave_lps[g.wave].push_back(
            NsLoopProblem{&g.plan, bb.xh[0], {bb.xh[0], bb.xh[1]}, bb.xh[cfg.ns_steps & 1], bb.a, bb.bh, bb.trace, bb.sync,
                          {bb.xl[0], bb.xl[1]}, bb.bl});
    }
    for (int w = 0; w < nwaves; ++w)
        choices[w] = ns_schedule_begin(wave_lps[w].data(), int(wave_lps[w].size()), cfg.ns_steps, s);

    // Small groups: the whole step in one launch per pointer table.
    for (const ShapeGroup& g : groups) {
        if (!g.plan.small) continue;
        const double aspect = std::sqrt(std::fmax(1.0, double(g.R) / double(g.C)));
        for (size_t m0 = 0; m0 < g.mats.size(); m0 += kTabMax) {
            const size_t cnt = std::min<size_t>(kTabMax, g.mats.size() - m0);
            const MatTable tab = make_table(mats, g, m0, cnt, lr, weight_decay, aspect);
            const Plan pc = chunk_plan(g.plan, int64_t(cnt));
            SmallStep ss;
            ss.mu = momentum;
            ss.mode = mode;
            ss.ns_steps = cfg.ns_steps;
            ss.a = cfg.a;
            ss.b = cfg.b;
            ss.c = cfg.c;
            ss.eps = cfg.eps;
            const hipError_t e = timed(MUON_KERNEL_SMALL, s, [&] { return launch_small(pc, ss, s, &tab); });
            if (e != hipSuccess) return hip_fail(e, "k_small launch");
        }
    }

    // Large groups, one wave after the other.
    bool first_prep = true;
    const int fin = cfg.ns_steps & 1;
    for (int w = 0; w < nwaves; ++w) {
        const std::vector<size_t>& wave = wave_groups[w];

        // Momentum + cast to the iterate, per group in chunks of pointer tables.
        for (size_t gi : wave) {
            const ShapeGroup& g = groups[gi];
            const Plan& p = g.plan;
            const double aspect = std::sqrt(std::fmax(1.0, double(g.R) / double(g.C)));
            for (size_t m0 = 0; m0 < g.mats.size(); m0 += kTabMax) {
                const size_t cnt = std::min<size_t>(kTabMax, g.mats.size() - m0);
                const MatTable tab = make_table(mats, g, m0, cnt, lr, weight_decay, aspect);
                const Plan pc = chunk_plan(p, int64_t(cnt));
                const Buffers bc = chunk_buffers(p, bufs[gi], int64_t(m0));
                uint32_t* reset = first_prep ? status : nullptr;
                first_prep = false;
                const hipError_t e = timed(MUON_KERNEL_PREP, s, [&] {
                    return launch_prep(pc, mode, nullptr, nullptr, momentum, bc.xh[0], bc.xl[0],
                                       cfg.ns_steps == 0 ? bc.part : nullptr, reset, s, &tab);
                });
                if (e != hipSuccess) return hip_fail(e, "k_prep launch");
            }
            // With NS iterations the first Gram yields the norm; without, the
            // prep's sums of squares give it.
            if (cfg.ns_steps == 0) {
                const hipError_t e = timed(MUON_KERNEL_NORM_FINALIZE, s, [&] {
                    return launch_norm_finalize(p, bufs[gi].part, bufs[gi].scale, cfg.eps, s);
                });
                if (e != hipSuccess) return hip_fail(e, "k_norm_finalize launch");
            }
        }

        // NS iterations: products of equal reduction length share launches.
        auto buckets = [&](auto key) {
            std::vector<std::vector<size_t>> out;
            std::map<int64_t, size_t> at;
            for (size_t gi : wave) {
                const int64_t k = key(groups[gi].plan);
                auto it = at.find(k);
                if (it == at.end() || out[it->second].size() == size_t(kMaxGemmProblems)) {
                    at[k] = out.size();
                    out.emplace_back();
                    it = at.find(k);
                }
                out[it->second].push_back(gi);
            }
            return out;
        };
        const auto by_np = buckets([](const Plan& p) { return p.np; });
        const auto by_mp = buckets([](const Plan& p) { return p.mp; });
        const NsChoice& ch = choices[w];
        ns_schedule_start(ch, s);
        if (ch.persistent) {
            double fl = 0.0;
            for (size_t gi : wave) fl += ns_flops(groups[gi].plan, cfg.ns_steps);
            const std::vector<NsLoopProblem>& lps = wave_lps[w];
            const hipError_t e = timed(MUON_KERNEL_NS_LOOP, s, [&] {
                return launch_ns_loop(lps.data(), int(lps.size()), cfg.ns_steps, cfg.a, cfg.b, cfg.c, cfg.eps, ch,
                                      reinterpret_cast<uint2*>(ws + waves[w].items_off), waves[w].items_cap, status,
                                      false, s);
            }, fl);
            if (e != hipSuccess) return hip_fail(e, "k_ns_loop launch");
        }
        for (int it = 0; it < (ch.persistent ? 0 : cfg.ns_steps); ++it) {
            const int cur = it & 1;
            for (const auto& bk : by_np) {
                GramOp ops[kMaxGemmProblems];
                double fl = 0.0;
                for (size_t k = 0; k < bk.size(); ++k) {
                    const Buffers& b = bufs[bk[k]];
                    ops[k] = GramOp{&groups[bk[k]].plan, b.xh[cur], b.a, it == 0 ? b.trace : nullptr};
                    fl += product_flops(groups[bk[k]].plan, MUON_KERNEL_GRAM);
                }
                const hipError_t e =
                    timed(MUON_KERNEL_GRAM, s, [&] { return launch_gram(ops, int(bk.size()), nullptr, s); }, fl);
                if (e != hipSuccess) return hip_fail(e, "k_gemm<gram> launch");
            }
            for (const auto& bk : by_mp) {
                PolyOp ops[kMaxGemmProblems];
                double fl = 0.0;
                for (size_t k = 0; k < bk.size(); ++k) {
                    const Buffers& b = bufs[bk[k]];
                    ops[k] = PolyOp{&groups[bk[k]].plan, b.a, b.bh, b.bl, it == 0 ? b.trace : nullptr};
                    fl += product_flops(groups[bk[k]].plan, MUON_KERNEL_POLY);
                }
                const hipError_t e = timed(MUON_KERNEL_POLY, s, [&] {
                    return launch_poly(ops, int(bk.size()), cfg.a, cfg.b, cfg.c, cfg.eps, s);
                }, fl);
                if (e != hipSuccess) return hip_fail(e, "k_gemm<poly> launch");
            }
            for (const auto& bk : by_mp) {
                BxOp ops[kMaxGemmProblems];
                double fl = 0.0;
                for (size_t k = 0; k < bk.size(); ++k) {
                    const Buffers& b = bufs[bk[k]];
                    ops[k] = BxOp{&groups[bk[k]].plan, b.bh, b.bl, b.xh[cur], b.xl[cur], b.xh[cur ^ 1],
                                  b.xl[cur ^ 1], it == 0 ? b.trace : nullptr};
                    fl += product_flops(groups[bk[k]].plan, MUON_KERNEL_BX);
                }
                const hipError_t e =
                    timed(MUON_KERNEL_BX, s, [&] { return launch_bx(ops, int(bk.size()), cfg.eps, s); }, fl);
                if (e != hipSuccess) return hip_fail(e, "k_gemm<bx> launch");
            }
        }
        ns_schedule_end(ch, s);

        // Update, per group in chunks.
        for (size_t gi : wave) {
            const ShapeGroup& g = groups[gi];
            const Plan& p = g.plan;
            const double aspect = std::sqrt(std::fmax(1.0, double(g.R) / double(g.C)));
            for (size_t m0 = 0; m0 < g.mats.size(); m0 += kTabMax) {
                const size_t cnt = std::min<size_t>(kTabMax, g.mats.size() - m0);
                const MatTable tab = make_table(mats, g, m0, cnt, lr, weight_decay, aspect);
                const Plan pc = chunk_plan(p, int64_t(cnt));
                const Buffers bc = chunk_buffers(p, bufs[gi], int64_t(m0));
                const hipError_t e = timed(MUON_KERNEL_FINISH, s, [&] {
                    return launch_finish(pc, bc.xh[fin], bc.xl[fin], cfg.ns_steps == 0 ? bc.scale : nullptr, nullptr,
                                         1.f, 0.f, nullptr, s, &tab);
                });
                if (e != hipSuccess) return hip_fail(e, "k_finish launch");
            }
        }
    }
    return MUON_OK;
}

muon_status adamw_step_multi(const muon_adam_tensor* tensors, int32_t count, float lr, float beta1, float beta2,
                             float eps, float weight_decay, void* stream) {
    g_err.clear();
    if (count < 0) return fail(MUON_ERR_SHAPE, "count must be >= 0");
    if (count == 0) return MUON_OK;
    if (tensors == nullptr) return fail(MUON_ERR_INVALID_ARG, "tensors must be non-null");
    if (!std::isfinite(lr) || !std::isfinite(weight_decay))
        return fail(MUON_ERR_INVALID_ARG, "lr and weight_decay must be finite");
    if (!std::isfinite(eps) || eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
        return fail(MUON_ERR_INVALID_ARG, "betas must be in [0, 1)");
    struct Range { uintptr_t a, b; int32_t t; };
    std::vector<Range> ranges;
    std::vector<AdamEntry> entries;
    for (int32_t i = 0; i < count; ++i) {
        const muon_adam_tensor& x = tensors[i];
        if (x.numel < 0) return fail(MUON_ERR_SHAPE, "tensor %d: numel must be >= 0", i);
        if (x.numel == 0) continue;
        if (!x.params || !x.grads || !x.exp_avg || !x.exp_avg_sq)
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: params, grads, exp_avg and exp_avg_sq must be non-null", i);
        if (!aligned(x.params, 4) || !aligned(x.exp_avg, 4) || !aligned(x.exp_avg_sq, 4) || !aligned(x.grads, 2))
            return fail(MUON_ERR_ALIGNMENT, "tensor %d: buffers must be element-aligned", i);
        if (x.step < 1) return fail(MUON_ERR_INVALID_ARG, "tensor %d: step must be >= 1", i);
        if (!std::isfinite(x.lr_mul) || !std::isfinite(x.wd_mul))
            return fail(MUON_ERR_INVALID_ARG, "tensor %d: lr_mul and wd_mul must be finite", i);
        const size_t n = size_t(x.numel);
        if (n > (size_t(1) << 46)) return fail(MUON_ERR_SHAPE, "tensor %d: numel too large", i);
        auto add = [&](const void* p, size_t bytes) {
            const uintptr_t a = reinterpret_cast<uintptr_t>(p);
            ranges.push_back({a, a + bytes, i});
        };
        add(x.params, 4 * n);
        add(x.grads, 2 * n);
        add(x.exp_avg, 4 * n);
        add(x.exp_avg_sq, 4 * n);
        AdamEntry e{};
        e.p = x.params;
        e.g = static_cast<const uint16_t*>(x.grads);
        e.m = x.exp_avg;
        e.v = x.exp_avg_sq;
        e.numel = x.numel;
        e.vec = aligned(x.params, 16) && aligned(x.grads, 16) && aligned(x.exp_avg, 16) && aligned(x.exp_avg_sq, 16);
        // Per-tensor constants in double ([DA]): decay first, bias corrections in the step size.
        const double lr_eff = double(lr) * double(x.lr_mul);
        e.decay = weight_decay != 0.f ? float(1.0 - lr_eff * double(weight_decay) * double(x.wd_mul)) : 1.0f;
        const double t = double(x.step);
        const double bias1 = 1.0 - std::pow(double(beta1), t), bias2 = 1.0 - std::pow(double(beta2), t);
        e.step = float(lr_eff * std::sqrt(bias2) / bias1);
        entries.push_back(e);
    }
    std::sort(ranges.begin(), ranges.end(), [](const Range& x, const Range& y) { return x.a < y.a; });
    for (size_t k = 1; k < ranges.size(); ++k)
        if (ranges[k].a < ranges[k - 1].b)
            return fail(MUON_ERR_INVALID_ARG, "buffers of tensors %d and %d overlap", ranges[k - 1].t, ranges[k].t);
    if (entries.empty()) return MUON_OK;
    muon_status st = check_device();
    if (st != MUON_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (size_t i0 = 0; i0 < entries.size(); i0 += kAdamTab) {
        const int n = int(std::min<size_t>(kAdamTab, entries.size() - i0));
        const hipError_t e =
            timed(MUON_KERNEL_ADAMW, s, [&] { return launch_adamw(entries.data() + i0, n, beta1, beta2, eps, s); });
        if (e != hipSuccess) return hip_fail(e, "k_adamw launch");
    }
    return MUON_OK;
}

muon_status muon_merge_small_dims(const int64_t* shape, int32_t ndim, int64_t threshold, int32_t target_ndim,
                                  int64_t* merged, int32_t* merged_ndim) {
    g_err.clear();
    if (ndim < 0 || ndim > MUON_MAX_DIMS) return fail(MUON_ERR_SHAPE, "ndim must be in [0, %d]", MUON_MAX_DIMS);
    if ((ndim > 0 && shape == nullptr) || merged == nullptr || merged_ndim == nullptr)
        return fail(MUON_ERR_INVALID_ARG, "shape, merged and merged_ndim must be non-null");
    if (threshold < 1) return fail(MUON_ERR_INVALID_ARG, "threshold must be >= 1");
    if (target_ndim < 0) return fail(MUON_ERR_INVALID_ARG, "target_ndim must be >= 1, or 0 for no target");
    for (int32_t i = 0; i < ndim; ++i)
        if (shape[i] < 0) return fail(MUON_ERR_SHAPE, "extent %d is negative", i);
    auto put1 = [&](int64_t v) {
        merged[0] = v;
        *merged_ndim = 1;
        return MUON_OK;
    };
    if (ndim == 0) return put1(1);                       // a 0-D tensor is 1-D
    for (int32_t i = 0; i < ndim; ++i)
        if (shape[i] == 0) return put1(0);               // empty
    int64_t sq[MUON_MAX_DIMS];
    int32_t ns = 0;
    for (int32_t i = 0; i < ndim; ++i)
        if (shape[i] != 1) sq[ns++] = shape[i];          // size-1 extents squeezed out
    if (ns == 0) return put1(1);
    if (target_ndim == 0) {                              // no target: no merging
        for (int32_t i = 0; i < ns; ++i) merged[i] = sq[i];
        *merged_ndim = ns;
        return MUON_OK;
    }
    // Walk from the last extent to the first.  `cur` is the extent being
    // formed; out[] collects finished extents right to left.  The next extent
    // folds into `cur` while the shape still has more than target_ndim
    // extents and the product stays within the threshold.
    int64_t out[MUON_MAX_DIMS];
    int32_t nout = 0;
    int64_t cur = sq[ns - 1];
    for (int32_t i = ns - 2; i >= 0; --i) {
        const int64_t count = int64_t(i) + 2 + nout;
        const bool fits = sq[i] <= threshold / cur;     // sq[i] * cur <= threshold, without overflow
        if (count > target_ndim && fits) {
            cur *= sq[i];
        } else {
            out[nout++] = cur;
            cur = sq[i];
        }
    }
    out[nout++] = cur;
    for (int32_t i = 0; i < nout; ++i) merged[i] = out[nout - 1 - i];
    *merged_ndim = nout;
    return MUON_OK;
}

muon_status muon_set_ns_schedule(int32_t mode) {
    g_err.clear();
    if (mode < 0 || mode > 2) return fail(MUON_ERR_INVALID_ARG, "schedule mode %d is not 0, 1 or 2", mode);
    set_ns_schedule(mode);
    return MUON_OK;
}

muon_status muon_timing_enable(uint32_t kernel_mask) {
    g_err.clear();
    if (kernel_mask >> MUON_KERNEL_COUNT) return fail(MUON_ERR_INVALID_ARG, "unknown kernel bits in mask 0x%x", kernel_mask);
    timing().mask.store(kernel_mask);
    return MUON_OK;
}

muon_status muon_timing_collect(int64_t* launches, double* total_ms, double* nominal_flops,
                                double* executed_flops) {
    g_err.clear();
    TimingState& ts = timing();
    std::lock_guard<std::mutex> lk(ts.mu);
    muon_status st = MUON_OK;
    for (const auto& r : ts.recs) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) {
            st = hip_fail(e, "muon_timing_collect");
        } else {
            if (launches) launches[r.kind] += 1;
            if (total_ms) total_ms[r.kind] += ms;
            if (nominal_flops) nominal_flops[r.kind] += r.flops;
            if (executed_flops) executed_flops[r.kind] += r.exec;
        }
        ts.pool[r.dev].push_back(r.a);
        ts.pool[r.dev].push_back(r.b);
    }
    ts.recs.clear();
    return st;
}

muon_status muon_workspace_status(const void* workspace, uint32_t* status_out, void* stream) {
    g_err.clear();
    if (status_out == nullptr || workspace == nullptr)
        return fail(MUON_ERR_INVALID_ARG, "workspace and status_out must be non-null");
    if (!aligned(workspace, 256)) return fail(MUON_ERR_ALIGNMENT, "workspace must be 256-byte aligned");
    if (!aligned(status_out, 4)) return fail(MUON_ERR_ALIGNMENT, "status_out must be 4-byte aligned");
    const hipError_t e = hipMemcpyAsync(status_out, workspace, 2 * sizeof(uint32_t), hipMemcpyDefault,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MUON_OK : hip_fail(e, "muon_workspace_status copy");
}

muon_status muon_set_gemm_tiling(int32_t width) {
    g_err.clear();
    if (width != 0 && width != 64 && width != 128 && width != 256)
        return fail(MUON_ERR_INVALID_ARG, "tile width %d is not 0, 64, 128 or 256", width);
    set_gemm_tiling(width);
    return MUON_OK;
}

muon_status muon_debug_set_loop_fault(int32_t mode) {
    g_err.clear();
    if (mode < 0 || mode > 2) return fail(MUON_ERR_INVALID_ARG, "loop fault mode %d is not 0, 1 or 2", mode);
    set_loop_fault(mode);
    return MUON_OK;
}

const char* muon_last_error(void) { return g_err.c_str(); }

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

}  // extern "C"
