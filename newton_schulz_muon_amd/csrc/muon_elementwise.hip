// HBM-bound kernels of the batched Muon step (gfx950).
//
//   k_prep      momentum update ("Muon Custom Sizing" walkthrough, section 4:
//               buffer lerp towards the gradient, Nesterov look-ahead from the
//               updated buffer) fused with the cast to the oriented, padded bf16
//               iterate and with the per-tile sums of squares that give the
//               Frobenius norm (parameter-golf walkthrough, Part 1: the input is
//               divided by its norm once).  Tall blocks are transposed through LDS
//               on the way, so orientation costs no extra pass.
//   k_norm_finalize   per NS block: 1/(sqrt(sum) + eps) and its square, summed in
//               a fixed order so results are run-to-run deterministic.
//   k_finish    reads the final iterate back into stored layout and either writes
//               the NS output or applies the decoupled-decay update
//               P <- P (1 - lr wd wd_mul) - lr max(1, R/C)^0.5 lr_mul O
//               ("Muon Custom Sizing" walkthrough, section 4; aspect factor from
//               the parameter-golf walkthrough, Part 1).
//
// Every kernel works on 64 x 64 tiles of the oriented block with 256 threads;
// each thread owns two rows of 8 consecutive elements, so stored rows are read
// and written as 16-byte (bf16) or 2 x 16-byte (fp32) vectors when the stored
// column count is a multiple of 8, and element by element otherwise.
#include "muon_internal.hpp"

namespace muon {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int T = kEwTile;

struct PrepArgs {
    MatTable tab;          // per-matrix buffers (tab.n > 0) or strided (src, mom)
    int64_t b0;            // first NS block of this launch (launches are split at kMaxGridY blocks)
    uint32_t* status;      // when non-null: the call's status words, cleared by workgroup (0, 0)
    const uint16_t* src;   // stored bf16 (gradients or x), this launch's first block
    float* mom;            // stored fp32 momentum buffer
    uint16_t* dh;          // padded copy in stored orientation [rp][cp] (hi, lo)
    uint16_t* dl;
    uint16_t* th;          // padded transposed copy [cp][rp] (hi, lo)
    uint16_t* tl;
    float* part;           // [nb][ew_tiles] sums of squares, or null (not needed)
    int64_t r, c;          // stored block shape
    int64_t rp, cp;        // padded stored-orientation shape
    int64_t be;            // r * c
    int64_t ew_tiles;
    int tiles_j;           // cp / TC (tiles per padded row)
    float mu, omm;
};

__device__ __forceinline__ float block_sum_256(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
    if (threadIdx.x == 0) s = ((red[0] + red[1]) + red[2]) + red[3];
    return s;
}

template <int MODE>
__device__ __forceinline__ float momentum_update(float g, float* mptr, float mu, float omm) {
    if constexpr (MODE == kPrepCast) {
        return g;
    } else {
        const float m = *mptr;
        const float mn = fmaf(omm, g - m, m);
        *mptr = mn;
        if constexpr (MODE == kPrepNesterov) return fmaf(mu, mn - g, g);
        else return mn;
    }
}

// 8 stored elements (bi, bj0 .. bj0 + 7) of one block as read from HBM.
struct Raw8 {
    u32x4 g;        // bf16 gradient / x
    f32x4 m0, m1;   // fp32 momentum buffer
    bool valid;
};

// Vector path: both loads of a row piece are 16-byte.
template <int MODE>
__device__ __forceinline__ Raw8 load8(const PrepArgs& a, const uint16_t* src, const float* mom, int64_t bi,
                                      int64_t bj0) {
    Raw8 r;
    r.valid = (bi < a.r) && (bj0 < a.c);
    r.g = u32x4{0u, 0u, 0u, 0u};
    r.m0 = r.m1 = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!r.valid) return r;
    const int64_t off = bi * a.c + bj0;
    r.g = *reinterpret_cast<const u32x4*>(src + off);
    if constexpr (MODE != kPrepCast) {
        r.m0 = *reinterpret_cast<const f32x4*>(mom + off);
        r.m1 = *(reinterpret_cast<const f32x4*>(mom + off) + 1);
    }
    return r;
}

// Applies the momentum update to loaded elements, stores the buffer and
// returns the update direction in u[].
template <int MODE>
__device__ __forceinline__ void update8(const PrepArgs& a, const Raw8& r, float* mom, int64_t bi, int64_t bj0,
                                        float (&u)[8], bool (&ok)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) { ok[e] = r.valid; u[e] = 0.f; }
    if (!r.valid) return;
    float g[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        g[2 * q] = bf16_to_f32(static_cast<uint16_t>(r.g[q] & 0xffffu));
        g[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(r.g[q] >> 16));
    }
    if constexpr (MODE == kPrepCast) {
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = g[e];
    } else {
        float m[8] = {r.m0[0], r.m0[1], r.m0[2], r.m0[3], r.m1[0], r.m1[1], r.m1[2], r.m1[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = momentum_update<MODE>(g[e], &m[e], a.mu, a.omm);
        f32x4* mp4 = reinterpret_cast<f32x4*>(mom + bi * a.c + bj0);
        *mp4 = f32x4{m[0], m[1], m[2], m[3]};
        mp4[1] = f32x4{m[4], m[5], m[6], m[7]};
    }
}

// Scalar path (stored column count not a multiple of 8).
template <int MODE>
__device__ __forceinline__ void load_update8_scalar(const PrepArgs& a, const uint16_t* src, float* mom,
                                                    int64_t bi, int64_t bj0, float (&u)[8], bool (&ok)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        ok[e] = (bi < a.r) && (bj0 + e < a.c);
        u[e] = 0.f;
        if (ok[e]) {
            const int64_t off = bi * a.c + bj0 + e;
            const float g = bf16_to_f32(src[off]);
            u[e] = momentum_update<MODE>(g, mom ? mom + off : nullptr, a.mu, a.omm);
        }
    }
}

// One tile of 4096 elements of the padded stored-orientation block per
// workgroup: TR x TC with TC = T for tall blocks (64 x 64, transposed through
// LDS) and the scalar path, and row strips up to 4 x 1024 for wide blocks,
// whose longer row pieces stream from HBM faster (measured with a probe of
// this access pattern: 5.1 TB/s as 64 x 64 tiles, 5.6 as 16 x 256, 5.7 as
// 4 x 1024).  The oriented iterate X is that block for wide blocks (written
// through dh/dl) and its transpose for tall ones (TALL: written through
// th/tl, via LDS).  Both passes' loads are issued before any store, so a
// thread has its whole share of HBM reads in flight at once.
template <int MODE, bool VEC, bool SPLIT, bool TALL, int TC = T>
__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
    static_assert(TC == T || (!TALL && VEC), "row strips only on the wide vector path");
    constexpr int TR = T * T / TC;    // tile rows
    constexpr int TPR = TC / 8;       // threads per tile row (8 elements each)
    constexpr int RPP = 256 / TPR;    // rows per pass; two passes
    static_assert(2 * RPP == TR, "a tile is two passes of the workgroup");
    __shared__ uint16_t lds_hi[TALL ? T : 1][T + 2];
    __shared__ uint16_t lds_lo[(TALL && SPLIT) ? T : 1][T + 2];
    __shared__ float red[4];

    const int t = threadIdx.x;
    const int64_t blk = blockIdx.y;
    const int tile = blockIdx.x;
    const int si = tile / a.tiles_j, sj = tile % a.tiles_j;
    if (a.status != nullptr && blk == 0 && tile == 0 && t < 2) a.status[t] = 0u;
    const uint16_t* src;
    float* mom = nullptr;
    if (a.tab.n > 0) {
        const int64_t tb = a.b0 + blk;      // block index within the table
        const int64_t mi = tb / a.tab.v, sub = tb % a.tab.v;
        src = a.tab.src[mi] + sub * a.be;
        if constexpr (MODE != kPrepCast) mom = a.tab.mom[mi] + sub * a.be;
    } else {
        src = a.src + blk * a.be;
        if constexpr (MODE != kPrepCast) mom = a.mom + blk * a.be;
    }
    const int64_t pad = a.rp * a.cp;
    uint16_t* dh = (TALL || a.dh == nullptr) ? nullptr : a.dh + blk * pad;
    uint16_t* dl = (!TALL && SPLIT) ? a.dl + blk * pad : nullptr;
    uint16_t* th = TALL ? a.th + blk * pad : nullptr;
    uint16_t* tl = (TALL && SPLIT) ? a.tl + blk * pad : nullptr;
    const int rl = t / TPR;
    const int cl = (t % TPR) * 8;
    float ss = 0.f;

    Raw8 raw[2];
    if constexpr (VEC) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            raw[h] = load8<MODE>(a, src, mom, (int64_t)si * TR + rl + RPP * h, (int64_t)sj * TC + cl);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = rl + RPP * h;
        const int64_t bi = (int64_t)si * TR + row;
        const int64_t bj0 = (int64_t)sj * TC + cl;
        float u[8];
        bool ok[8];
        if constexpr (VEC) update8<MODE>(a, raw[h], mom, bi, bj0, u, ok);
        else load_update8_scalar<MODE>(a, src, mom, bi, bj0, u, ok);
        uint16_t hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            hi[e] = ok[e] ? f32_to_bf16(u[e]) : uint16_t(0);
            const float hv = bf16_to_f32(hi[e]);
            if constexpr (SPLIT) {
                lo[e] = ok[e] ? f32_to_bf16(u[e] - hv) : uint16_t(0);
                ss = fmaf(u[e], u[e], ss);
            } else {
                ss = fmaf(hv, hv, ss);
            }
        }
        if constexpr (!TALL) {
            if (dh == nullptr) continue;         // sums of squares only: X0 is the caller's buffer
            const int64_t o = bi * a.cp + bj0;   // inside the padded block
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = uint32_t(hi[2 * q]) | (uint32_t(hi[2 * q + 1]) << 16);
            *reinterpret_cast<u32x4*>(dh + o) = w;
            if constexpr (SPLIT) {
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = uint32_t(lo[2 * q]) | (uint32_t(lo[2 * q + 1]) << 16);
                *reinterpret_cast<u32x4*>(dl + o) = w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                lds_hi[row][cl + e] = hi[e];
                if constexpr (SPLIT) lds_lo[row][cl + e] = lo[e];
            }
        }
    }

    if constexpr (TALL) {
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = rl + 32 * h;   // transposed local row = stored local column
            const int64_t o = ((int64_t)sj * T + row) * a.rp + (int64_t)si * T + cl;
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = uint32_t(lds_hi[cl + 2 * q][row]) | (uint32_t(lds_hi[cl + 2 * q + 1][row]) << 16);
            *reinterpret_cast<u32x4*>(th + o) = w;
            if constexpr (SPLIT) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = uint32_t(lds_lo[cl + 2 * q][row]) | (uint32_t(lds_lo[cl + 2 * q + 1][row]) << 16);
                *reinterpret_cast<u32x4*>(tl + o) = w;
            }
        }
    }

    if (a.part != nullptr) {   // uniform: the sums of squares only where the norm is taken here
        const float tot = block_sum_256(ss, red);
        if (t == 0) a.part[blk * a.ew_tiles + tile] = tot;
    }
}

__global__ __launch_bounds__(256) void k_norm_finalize(const float* part, float* scales,
                                                       int64_t ew_tiles, float eps) {
    __shared__ float red[4];
    const int64_t blk = blockIdx.x;
    const float* p = part + blk * ew_tiles;
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < ew_tiles; i += 256) s += p[i];
    const float tot = block_sum_256(s, red);
    if (threadIdx.x == 0) {
        const float inv = 1.0f / (sqrtf(tot) + eps);
        scales[2 * blk] = inv;
        scales[2 * blk + 1] = inv * inv;
    }
}

struct FinArgs {
    MatTable tab;          // per-matrix buffers and scalars (tab.n > 0) or strided (P, out)
    int64_t b0;            // first NS block of this launch (launches are split at kMaxGridY blocks)
    const uint16_t* xhi;   // oriented padded final iterate
    const uint16_t* xlo;
    const float* scale;    // [nb][2] or null
    float* P;              // stored fp32 parameters (update mode)
    uint16_t* out;         // stored bf16 output (NS output, or optional O)
    int64_t r, c, mp, np, be;
    int tiles_j;           // ceil(n / TC)
    float decay, step;
};

// Parameters of 8 stored elements (bi, bj0 .. bj0 + 7), vector path.
struct P8 {
    f32x4 p0, p1;
};

template <bool UPDATE, bool VEC>
__device__ __forceinline__ P8 load_p8(const FinArgs& a, const float* P, int64_t bi, int64_t bj0) {
    P8 r{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (UPDATE && VEC) {
        if (bi < a.r && bj0 < a.c) {
            const f32x4* p4 = reinterpret_cast<const f32x4*>(P + bi * a.c + bj0);
            r.p0 = *p4;
            r.p1 = *(p4 + 1);
        }
    }
    return r;
}

template <bool UPDATE, bool VEC>
__device__ __forceinline__ void finish_store8(const FinArgs& a, float* P, uint16_t* out, int64_t bi, int64_t bj0,
                                              const P8& pv, const float (&o)[8], const uint16_t (&bits)[8],
                                              bool exact_bits, float decay, float step) {
    if (bi >= a.r) return;
    if constexpr (VEC) {
        if (bj0 >= a.c) return;
        const int64_t off = bi * a.c + bj0;
        if constexpr (UPDATE) {
            f32x4 p0 = pv.p0, p1 = pv.p1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p0[e] = fmaf(-step, o[e], p0[e] * decay);
                p1[e] = fmaf(-step, o[e + 4], p1[e] * decay);
            }
            f32x4* p4 = reinterpret_cast<f32x4*>(P + off);
            p4[0] = p0;
            p4[1] = p1;
        }
        if (out != nullptr) {
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint16_t l = exact_bits ? bits[2 * q] : f32_to_bf16(o[2 * q]);
                const uint16_t h = exact_bits ? bits[2 * q + 1] : f32_to_bf16(o[2 * q + 1]);
                w[q] = uint32_t(l) | (uint32_t(h) << 16);
            }
            *reinterpret_cast<u32x4*>(out + off) = w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (bj0 + e >= a.c) break;
            const int64_t off = bi * a.c + bj0 + e;
            if constexpr (UPDATE) P[off] = fmaf(-step, o[e], P[off] * decay);
            if (out != nullptr) out[off] = exact_bits ? bits[e] : f32_to_bf16(o[e]);
        }
    }
}

// One tile of 4096 elements of the oriented block per workgroup (TR x TC as
// in k_prep: 64 x 64 for tall blocks and the scalar path, row strips for
// wide blocks); both passes' loads (the final iterate, and for the update
// the parameters) are issued before any store.  (Non-temporal loads and
// stores here measured slower: 5.0-5.3 TB/s against 5.6, and again 4.8-4.9
// against 5.3-5.4 with the momentum kernel's also non-temporal.)
template <bool UPDATE, bool TALL, bool VEC, bool SPLIT, int TC = T>
__global__ __launch_bounds__(256) void k_finish(FinArgs a) {
    static_assert(TC == T || (!TALL && VEC), "row strips only on the wide vector path");
    constexpr int TR = T * T / TC;    // tile rows
    constexpr int TPR = TC / 8;       // threads per tile row (8 elements each)
    constexpr int RPP = 256 / TPR;    // rows per pass; two passes
    static_assert(2 * RPP == TR, "a tile is two passes of the workgroup");
    __shared__ float lds[TALL ? T : 1][T + 1];
    __shared__ uint16_t ldsb[TALL ? T : 1][T + 2];
    const int t = threadIdx.x;
    const int64_t blk = blockIdx.y;
    const int tile = blockIdx.x;
    const int ti = tile / a.tiles_j, tj = tile % a.tiles_j;
    const uint16_t* xhi = a.xhi + blk * a.mp * a.np;
    const uint16_t* xlo = SPLIT ? a.xlo + blk * a.mp * a.np : nullptr;
    float* P = nullptr;
    uint16_t* out = nullptr;
    float decay = a.decay, step = a.step;
    if (a.tab.n > 0) {
        const int64_t tb = a.b0 + blk;      // block index within the table
        const int64_t mi = tb / a.tab.v, sub = tb % a.tab.v;
        if constexpr (UPDATE) P = a.tab.P[mi] + sub * a.be;
        out = a.tab.out[mi] ? a.tab.out[mi] + sub * a.be : nullptr;
        decay = a.tab.decay[mi];
        step = a.tab.step[mi];
    } else {
        if constexpr (UPDATE) P = a.P + blk * a.be;
        out = a.out ? a.out + blk * a.be : nullptr;
    }
    const float sc = a.scale ? a.scale[2 * blk] : 1.0f;
    const bool exact_bits = !SPLIT && a.scale == nullptr;
    const int rl = t / TPR;
    const int cl = (t % TPR) * 8;

    u32x4 vh[2], vl[2];
    P8 pv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t o = ((int64_t)ti * TR + rl + RPP * h) * a.np + (int64_t)tj * TC + cl;   // inside the padded buffer
        vh[h] = *reinterpret_cast<const u32x4*>(xhi + o);
        vl[h] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (SPLIT) vl[h] = *reinterpret_cast<const u32x4*>(xlo + o);
        if constexpr (!TALL)
            pv[h] = load_p8<UPDATE, VEC>(a, P, (int64_t)ti * TR + rl + RPP * h, (int64_t)tj * TC + cl);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = rl + RPP * h;
        const int64_t oi = (int64_t)ti * TR + row;
        const int64_t oj = (int64_t)tj * TC + cl;
        float v[8];
        uint16_t bits[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            bits[2 * q] = static_cast<uint16_t>(vh[h][q] & 0xffffu);
            bits[2 * q + 1] = static_cast<uint16_t>(vh[h][q] >> 16);
            v[2 * q] = bf16_to_f32(bits[2 * q]);
            v[2 * q + 1] = bf16_to_f32(bits[2 * q + 1]);
            if constexpr (SPLIT) {
                v[2 * q] += bf16_to_f32(static_cast<uint16_t>(vl[h][q] & 0xffffu));
                v[2 * q + 1] += bf16_to_f32(static_cast<uint16_t>(vl[h][q] >> 16));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= sc;
        if constexpr (!TALL) {
            finish_store8<UPDATE, VEC>(a, P, out, oi, oj, pv[h], v, bits, exact_bits, decay, step);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                lds[row][cl + e] = v[e];
                ldsb[row][cl + e] = bits[e];
            }
        }
    }

    if constexpr (TALL) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            pv[h] = load_p8<UPDATE, VEC>(a, P, (int64_t)tj * T + rl + 32 * h, (int64_t)ti * T + cl);
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = rl + 32 * h;    // stored local row = oriented local column
            const int64_t bi = (int64_t)tj * T + row;
            const int64_t bj0 = (int64_t)ti * T + cl;
            float v[8];
            uint16_t bits[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[e] = lds[cl + e][row];
                bits[e] = ldsb[cl + e][row];
            }
            finish_store8<UPDATE, VEC>(a, P, out, bi, bj0, pv[h], v, bits, exact_bits, decay, step);
        }
    }
}

template <typename F>
hipError_t for_block_chunks(int64_t nb, F&& f) {
    for (int64_t b0 = 0; b0 < nb; b0 += kMaxGridY) {
        const int64_t cnt = (nb - b0) < kMaxGridY ? (nb - b0) : kMaxGridY;
        f(b0, static_cast<unsigned>(cnt));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Widest row strip (columns, up to 1024) whose width divides the padded
// columns `cols` (a multiple of 128): every tile then lies inside the padded
// block.
inline int strip_cols(int64_t cols) {
    return cols % 1024 == 0 ? 1024 : cols % 512 == 0 ? 512 : cols % 256 == 0 ? 256 : 128;
}

template <int MODE, bool VEC, bool SPLIT, bool TALL, int TC = T>
hipError_t run_prep(const Plan& p, const PrepArgs& a, hipStream_t s) {
    const int64_t be = p.r * p.c;
    const int64_t pad = p.mp * p.np;
    // the padded block's rows (a multiple of 128) and columns (of TC) tile exactly
    if (a.rp % (T * T / TC) != 0 || a.cp % TC != 0 || (a.rp / (T * T / TC)) * (a.cp / TC) != p.ew_tiles)
        return hipErrorInvalidValue;
    return for_block_chunks(p.nb, [&](int64_t b0, unsigned cnt) {
        PrepArgs c = a;
        c.tiles_j = static_cast<int>(a.cp / TC);
        c.b0 = b0;
        c.status = b0 == 0 ? a.status : nullptr;
        c.src = a.src ? a.src + b0 * be : nullptr;
        c.mom = a.mom ? a.mom + b0 * be : nullptr;
        c.dh = a.dh ? a.dh + b0 * pad : nullptr;
        c.dl = a.dl ? a.dl + b0 * pad : nullptr;
        c.th = a.th ? a.th + b0 * pad : nullptr;
        c.tl = a.tl ? a.tl + b0 * pad : nullptr;
        c.part = a.part ? a.part + b0 * p.ew_tiles : nullptr;
        k_prep<MODE, VEC, SPLIT, TALL, TC><<<dim3(static_cast<unsigned>(p.ew_tiles), cnt), dim3(256), 0, s>>>(c);
    });
}

template <int MODE, bool SPLIT>
hipError_t prep_strips(const Plan& p, const PrepArgs& a, hipStream_t s) {
    switch (strip_cols(a.cp)) {
        case 1024: return run_prep<MODE, true, SPLIT, false, 1024>(p, a, s);
        case 512: return run_prep<MODE, true, SPLIT, false, 512>(p, a, s);
        case 256: return run_prep<MODE, true, SPLIT, false, 256>(p, a, s);
        default: return run_prep<MODE, true, SPLIT, false, 128>(p, a, s);
    }
}

template <int MODE, bool TALL>
hipError_t prep_orient(const Plan& p, const PrepArgs& a, hipStream_t s) {
    const bool vec = (p.c % 8) == 0;
    const bool split = a.dl != nullptr || a.tl != nullptr;
    if (vec && !TALL) return split ? prep_strips<MODE, true>(p, a, s) : prep_strips<MODE, false>(p, a, s);
    if (vec) return split ? run_prep<MODE, true, true, TALL>(p, a, s) : run_prep<MODE, true, false, TALL>(p, a, s);
    return split ? run_prep<MODE, false, true, TALL>(p, a, s) : run_prep<MODE, false, false, TALL>(p, a, s);
}

template <int MODE>
hipError_t prep_mode(const Plan& p, const PrepArgs& a, hipStream_t s) {
    return p.tall ? prep_orient<MODE, true>(p, a, s) : prep_orient<MODE, false>(p, a, s);
}

template <bool UPDATE, bool TALL, bool VEC, bool SPLIT, int TC = T>
hipError_t run_finish(const Plan& p, const FinArgs& a, hipStream_t s) {
    const int64_t be = p.r * p.c;
    const int64_t pad = p.mp * p.np;
    constexpr int TR = T * T / TC;
    // the tiles cover rows up to ceil(m / TR) TR <= mp and columns up to
    // ceil(n / TC) TC <= np (mp is a multiple of 128, np of TC)
    if (p.mp % TR != 0 || p.np % TC != 0) return hipErrorInvalidValue;
    const int64_t ti = (p.m + TR - 1) / TR;
    const int tiles_j = static_cast<int>((p.n + TC - 1) / TC);
    const int64_t tiles = ti * tiles_j;
    return for_block_chunks(p.nb, [&](int64_t b0, unsigned cnt) {
        FinArgs c = a;
        c.tiles_j = tiles_j;
        c.b0 = b0;
        c.xhi = a.xhi + b0 * pad;
        c.xlo = a.xlo ? a.xlo + b0 * pad : nullptr;
        c.scale = a.scale ? a.scale + 2 * b0 : nullptr;
        c.P = a.P ? a.P + b0 * be : nullptr;
        c.out = a.out ? a.out + b0 * be : nullptr;
        k_finish<UPDATE, TALL, VEC, SPLIT, TC><<<dim3(static_cast<unsigned>(tiles), cnt), dim3(256), 0, s>>>(c);
    });
}

template <bool UPDATE>
hipError_t finish_mode(const Plan& p, const FinArgs& a, hipStream_t s) {
    const bool vec = (p.c % 8) == 0;
    const bool split = a.xlo != nullptr;
    if (p.tall) {
        if (vec) return split ? run_finish<UPDATE, true, true, true>(p, a, s) : run_finish<UPDATE, true, true, false>(p, a, s);
        return split ? run_finish<UPDATE, true, false, true>(p, a, s) : run_finish<UPDATE, true, false, false>(p, a, s);
    }
    if (vec) {
        switch (strip_cols(p.np)) {
            case 1024: return split ? run_finish<UPDATE, false, true, true, 1024>(p, a, s)
                                    : run_finish<UPDATE, false, true, false, 1024>(p, a, s);
            case 512: return split ? run_finish<UPDATE, false, true, true, 512>(p, a, s)
                                   : run_finish<UPDATE, false, true, false, 512>(p, a, s);
            case 256: return split ? run_finish<UPDATE, false, true, true, 256>(p, a, s)
                                   : run_finish<UPDATE, false, true, false, 256>(p, a, s);
            default: return split ? run_finish<UPDATE, false, true, true, 128>(p, a, s)
                                  : run_finish<UPDATE, false, true, false, 128>(p, a, s);
        }
    }
    return split ? run_finish<UPDATE, false, false, true>(p, a, s) : run_finish<UPDATE, false, false, false>(p, a, s);
}

}  // namespace

hipError_t launch_prep(const Plan& p, PrepMode mode, const uint16_t* src, float* mom, float mu,
                       uint16_t* x_hi, uint16_t* x_lo, float* partials, uint32_t* status, hipStream_t s,
                       const MatTable* tab) {
    if (x_hi == nullptr && (p.tall || x_lo != nullptr)) return hipErrorInvalidValue;
    PrepArgs a;
    a.b0 = 0;
    a.status = status;
    if (tab != nullptr) {
        if (tab->n < 1 || tab->n > kTabMax || tab->v != p.v || p.nb != int64_t(tab->n) * tab->v)
            return hipErrorInvalidValue;
        a.tab = *tab;
    }
    a.src = src;
    a.mom = mom;
    // wide block: X is the stored orientation; tall block: X is its transpose
    a.dh = p.tall ? nullptr : x_hi;
    a.dl = p.tall ? nullptr : x_lo;
    a.th = p.tall ? x_hi : nullptr;
    a.tl = p.tall ? x_lo : nullptr;
    a.part = partials;
    a.r = p.r;
    a.c = p.c;
    a.rp = p.tall ? p.np : p.mp;
    a.cp = p.tall ? p.mp : p.np;
    a.be = p.r * p.c;
    a.ew_tiles = p.ew_tiles;
    a.tiles_j = static_cast<int>(a.cp / T);
    a.mu = mu;
    a.omm = 1.0f - mu;
    switch (mode) {
        case kPrepCast: return prep_mode<kPrepCast>(p, a, s);
        case kPrepNesterov: return prep_mode<kPrepNesterov>(p, a, s);
        case kPrepPlain: return prep_mode<kPrepPlain>(p, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_norm_finalize(const Plan& p, const float* partials, float* scales, float eps,
                                hipStream_t s) {
    if (p.nb > 0x7fffffff) return hipErrorInvalidValue;
    k_norm_finalize<<<dim3(static_cast<unsigned>(p.nb)), dim3(256), 0, s>>>(partials, scales, p.ew_tiles, eps);
    return hipGetLastError();
}

hipError_t launch_finish(const Plan& p, const uint16_t* x_hi, const uint16_t* x_lo,
                         const float* scale, float* params, float decay, float step,
                         uint16_t* out, hipStream_t s, const MatTable* tab) {
    FinArgs a;
    a.b0 = 0;
    if (tab != nullptr) {
        if (tab->n < 1 || tab->n > kTabMax || tab->v != p.v || p.nb != int64_t(tab->n) * tab->v)
            return hipErrorInvalidValue;
        a.tab = *tab;
    }
    a.xhi = x_hi;
    a.xlo = x_lo;
    a.scale = scale;
    a.P = params;
    a.out = out;
    a.r = p.r;
    a.c = p.c;
    a.mp = p.mp;
    a.np = p.np;
    a.be = p.r * p.c;
    a.tiles_j = static_cast<int>((p.n + T - 1) / T);
    a.decay = decay;
    a.step = step;
    const bool update = params != nullptr || (a.tab.n > 0 && a.tab.P[0] != nullptr);
    return update ? finish_mode<true>(p, a, s) : finish_mode<false>(p, a, s);
}

}  // namespace muon
