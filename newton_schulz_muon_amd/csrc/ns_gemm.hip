// MFMA kernels of the quintic Newton-Schulz iteration (gfx950, bf16 in, fp32
// accumulate): parameter-golf walkthrough Part 1 (A = X X^T, B = b A + c A A,
// X = a X + B X) with the coefficients of the "Muon Custom Sizing"
// walkthrough, section 2.3, which also names a symmetric kernel for X X^T.
//
//   k_sym<GRAM>  A  = scale * X X^T             K = np, both operands rows of X
//   k_sym<POLY>  B' = a I + b A + c A A^T       K = mp, A symmetric so A A = A A^T
//   k_bx         X' = scale * B' X              K = mp, X read k-major
//
// The a X term of the update is carried by the diagonal of B' (exact in the
// algebra: a X + B X = (a I + B) X), so k_bx has no read-modify epilogue and
// the bf16 rounding of B' happens after the cancellation between a and the
// diagonal of b A + c A^2 rather than before it.
//
// A and B' are symmetric, so k_sym computes only the tiles (ti <= tj) of the
// upper triangle and also stores each off-diagonal tile transposed.
//
// Tiling: a 256-thread workgroup (2 x 2 waves) computes a BM x BN output tile
// (256 x 256 or 128 x 128); each wave owns (BM/2) x (BN/2) as a grid of
// v_mfma_f32_32x32x16_bf16 accumulators.  K steps by 64 through two LDS
// stages: while the waves multiply stage s, the next K slice is fetched into
// stage s^1 (rows of a k-contiguous operand by buffer_load ... lds DMA, the
// k-major X of k_bx through registers), with one barrier per step.  Operand
// tiles sit in LDS as rows x 64 bf16 (8 chunks of 16 bytes per row) with the
// chunk index XOR-swizzled by the row, so 16-byte fragment reads are
// conflict-free.  X in k_bx is k-major in memory: each thread loads 4 k-rows x
// 8 columns and writes them transposed (8-byte LDS stores).
//
// MFMA 32x32x16 lane layout: lane l supplies row (l % 32) of its operand and
// 8 consecutive k values starting at 8 (l / 32); result element (r, c) of a
// 32 x 32 block sits in lane 32 ((r / 4) % 2) + c, register 4 (r / 8) + r % 4.
// The kernels pass the column operand first, so each lane ends up holding 4
// consecutive output columns of one output row (8-byte stores).
#include "muon_internal.hpp"

namespace muon {
namespace {

constexpr int BK = 64;
constexpr int NTHR = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return (row << 7) + ((chunk ^ swz(row)) << 4);
}

template <int BM, int BN>
struct TileCfg {
    static constexpr int TM = BM / 2, TN = BN / 2;   // wave tile
    static constexpr int FM = TM / 32, FN = TN / 32; // 32x32 blocks per wave
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
};

// Buffer resource over one matrix (raw addressing, byte offsets): loads are
// range-checked by the hardware against `bytes`, and each lane keeps a 32-bit
// offset instead of a 64-bit pointer.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// R rows x 64 k of a k-contiguous matrix: R * 8 16-byte vectors, R / 32 per
// thread (vector v = thread + 256 q covers row v / 8, k chunk v % 8).
template <int R>
struct RowTile {
    u32x4 v[R / 32];
    uint32_t voff[R / 32];

    __device__ __forceinline__ void init(int64_t ld, int row0) {
#pragma unroll
        for (int q = 0; q < R / 32; ++q) {
            const int v = threadIdx.x + NTHR * q;
            voff[q] = static_cast<uint32_t>(((int64_t)(row0 + (v >> 3)) * ld + (v & 7) * 8) * 2);
        }
    }
    // k0: first k column of the slice
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int k0) {
#pragma unroll
        for (int q = 0; q < R / 32; ++q) v[q] = buf_load16(r, voff[q], static_cast<uint32_t>(k0 * 2));
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int q = 0; q < R / 32; ++q) {
            const int vi = threadIdx.x + NTHR * q;
            *reinterpret_cast<u32x4*>(lds + lds_off(vi >> 3, vi & 7)) = v[q];
        }
    }
};

// The same R x 64 tile fetched straight into LDS (buffer_load_dwordx4 ... lds):
// an instruction of one wave fills 1 KB of LDS, lane L writing bytes
// [16 L, 16 L + 16) of it, i.e. 8 rows x 8 chunks.  The swizzle is applied on
// the global side: the lane whose LDS slot is (row, physical chunk p) fetches
// logical chunk p ^ swz(row).  No registers stage the data.
template <int R>
struct RowDma {
    static constexpr int PER_WAVE = R / 32;   // 1 KB windows per wave
    uint32_t voff[PER_WAVE];

    __device__ __forceinline__ void init(int64_t ld, int row0) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int row = 8 * (w * PER_WAVE + q) + (l >> 3);
            const int chunk = (l & 7) ^ swz(row);
            voff[q] = static_cast<uint32_t>(((int64_t)(row0 + row) * ld + chunk * 8) * 2);
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, char* lds, int k0) const {
        const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)(lds + (w * PER_WAVE + q) * 1024), 16, voff[q],
                static_cast<uint32_t>(k0 * 2), 0, 0);
    }
};

// 64 k x C columns of a column-contiguous matrix: 2C sub-blocks of 4 k x 8
// columns, C / 128 per thread.  Sub-block sb covers columns 8 (sb % (C/8)) ..
// and k rows 4 (sb / (C/8)) ..; it is written transposed (LDS row = column).
template <int C>
struct ColTile {
    u32x4 v[C / 32];
    uint32_t voff[C / 32];
    uint32_t ldb;   // row pitch in bytes

    __device__ __forceinline__ void init(int64_t ld, int col0) {
        ldb = static_cast<uint32_t>(ld * 2);
#pragma unroll
        for (int s = 0; s < C / 128; ++s) {
            const int sb = threadIdx.x + NTHR * s;
            const int jg = sb % (C / 8), kg = sb / (C / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                voff[4 * s + r] = static_cast<uint32_t>(((int64_t)(kg * 4 + r) * ld + col0 + jg * 8) * 2);
        }
    }
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int k0) {
#pragma unroll
        for (int q = 0; q < C / 32; ++q) v[q] = buf_load16(r, voff[q], static_cast<uint32_t>(k0) * ldb);
    }
    __device__ __forceinline__ void store(char* lds) const {
#pragma unroll
        for (int s = 0; s < C / 128; ++s) {
            const int sb = threadIdx.x + NTHR * s;
            const int jg = sb % (C / 8), kg = sb / (C / 8);
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int p = cc >> 1;
                const uint32_t a0 = v[4 * s][p], a1 = v[4 * s + 1][p];
                const uint32_t a2 = v[4 * s + 2][p], a3 = v[4 * s + 3][p];
                u32x2 w;
                if (cc & 1) {
                    w[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                    w[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                } else {
                    w[0] = (a0 & 0xffffu) | (a1 << 16);
                    w[1] = (a2 & 0xffffu) | (a3 << 16);
                }
                *reinterpret_cast<u32x2*>(lds + lds_off(jg * 8 + cc, kg >> 1) + ((kg & 1) << 3)) = w;
            }
        }
    }
};

// Work attached to a K step (see kstep): global prefetch of the next stage and
// the transposing LDS write of k_bx.  Plain functors rather than lambdas.
struct NoWork {
    __device__ __forceinline__ void operator()() const {}
};

template <int R>
struct PrefetchRows2 {   // two row tiles by DMA (k_sym)
    const RowDma<R>& ra;
    const RowDma<R>& rb;
    __amdgpu_buffer_rsrc_t rs;
    char* lds_a;
    char* lds_b;
    int k0;
    bool on;
    __device__ __forceinline__ void operator()() const {
        if (on) {
            ra.load(rs, lds_a, k0);
            rb.load(rs, lds_b, k0);
        }
    }
};

template <int R, int C>
struct PrefetchRowCol {   // B' rows by DMA, X columns into registers (k_bx)
    const RowDma<R>& rb;
    ColTile<C>& cx;
    __amdgpu_buffer_rsrc_t rbs, rxs;
    char* lds_b;
    int k0;
    bool on;
    __device__ __forceinline__ void operator()() const {
        if (on) {
            rb.load(rbs, lds_b, k0);
            cx.load(rxs, k0);
        }
    }
};

template <int C>
struct StoreCols {
    const ColTile<C>& cx;
    char* lds;
    bool on;
    __device__ __forceinline__ void operator()() const {
        if (on) cx.store(lds);
    }
};

template <typename F, typename G>
struct Both {
    const F& f;
    const G& g;
    __device__ __forceinline__ void operator()() const {
        f();
        g();
    }
};

// Workgroups of one launch are handed to the 8 XCDs round-robin (w -> XCD
// w % 8).  Renumbering them so that each XCD gets one contiguous range of
// logical tiles keeps the operand panels of a matrix in a single XCD's L2.
__device__ __forceinline__ uint32_t xcd_logical(uint32_t w, uint32_t total) {
    const uint32_t q = total >> 3, r = total & 7, x = w & 7;
    return x * q + (x < r ? x : r) + (w >> 3);
}

template <int FM, int FN>
__device__ __forceinline__ void load_frags(const char* As, const char* Bs, int wr0, int wc0, int ks,
                                           bf16x8 (&a)[FM], bf16x8 (&b)[FN]) {
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(As + lds_off(wr0 + i * 32 + lr, ch));
#pragma unroll
    for (int j = 0; j < FN; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wc0 + j * 32 + lr, ch));
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_block(const bf16x8 (&a)[FM], const bf16x8 (&b)[FN],
                                           f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
}

// Scheduling pattern for one 16-deep sub-slice region: the FM + FN fragment
// reads of the next sub-slice spread evenly between the FM * FN MFMAs.
template <int FM, int FN>
__device__ __forceinline__ void interleave_reads() {
#pragma unroll
    for (int t = 0; t < FM + FN; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, FM * FN / (FM + FN), 0);  // MFMA
    }
}

// One 64-deep K step of a wave: acc += A(rows) B(cols)^T over stage `st`.
// `prefetch` issues the global loads of the next stage right after the first
// fragment reads; `late` runs in the last sub-slice region (k_bx writes the
// transposed X there).  Each 16-deep sub-slice is its own scheduling region
// (sched_barrier), so the LDS reads placed between its MFMAs are the next
// sub-slice's fragments and their latency hides behind the current MFMAs.
template <int FM, int FN, typename Prefetch, typename Late>
__device__ __forceinline__ void kstep(const char* As, const char* Bs, int wr0, int wc0,
                                      f32x16 (&acc)[FM][FN], const Prefetch& prefetch, const Late& late) {
    constexpr int KS = BK / 16;
    bf16x8 a[2][FM], b[2][FN];
    load_frags<FM, FN>(As, Bs, wr0, wc0, 0, a[0], b[0]);
    prefetch();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int cur = ks & 1;
        if (ks + 1 < KS) load_frags<FM, FN>(As, Bs, wr0, wc0, ks + 1, a[cur ^ 1], b[cur ^ 1]);
        mfma_block<FM, FN>(a[cur], b[cur], acc);
        if (ks + 1 < KS) {
            interleave_reads<FM, FN>();
        } else {
            late();
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[FM][FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int s = 0; s < 16; ++s) acc[i][j][s] = 0.f;
}

__device__ __forceinline__ u32x2 pack4(const uint16_t (&h)[4]) {
    u32x2 w;
    w[0] = uint32_t(h[0]) | (uint32_t(h[1]) << 16);
    w[1] = uint32_t(h[2]) | (uint32_t(h[3]) << 16);
    return w;
}

enum SymKind { kGram = 0, kPoly = 1, kPolySplit = 2 };

struct SymArgs {
    const uint16_t* src;     // X (Gram) or A (poly), this launch's first block
    uint16_t* out;           // A (Gram) or B' hi (poly)
    uint16_t* out_lo;        // B' lo (poly split)
    const float* scale;      // [nb][2] (Gram, iteration 1) or null
    int64_t src_stride, out_stride;
    int64_t ld;              // row pitch of src = K
    int64_t ldo;             // row pitch of out = mp
    int T;                   // tiles per side
    uint32_t tiles;          // tiles per block = T (T + 1) / 2
    uint32_t total;          // tiles * blocks in this launch
    uint32_t src_bytes;      // bytes of one source matrix
    float ca, cb, cc;
};

template <int KIND, int BT>
__global__ __launch_bounds__(NTHR) void k_sym(SymArgs a) {
    using Cfg = TileCfg<BT, BT>;
    constexpr int FM = Cfg::FM, FN = Cfg::FN;
    __shared__ __attribute__((aligned(16))) char lds[2 * Cfg::STAGE];

    const uint32_t L = xcd_logical(blockIdx.x, a.total);
    const int64_t blk = L / a.tiles;
    int id = static_cast<int>(L % a.tiles), ti = 0, len = a.T;
    while (id >= len) { id -= len; ++ti; --len; }
    const int tj = ti + id;
    const uint16_t* src = a.src + blk * a.src_stride;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, a.src_bytes);
    const int row0 = ti * BT, col0 = tj * BT;
    const int wave = threadIdx.x >> 6;
    const int wr0 = (wave >> 1) * Cfg::TM, wc0 = (wave & 1) * Cfg::TN;

    f32x16 acc[FM][FN];
    zero_acc(acc);

    RowDma<BT> ra, rb;
    ra.init(a.ld, row0);
    rb.init(a.ld, col0);
    ra.load(rs, lds, 0);
    rb.load(rs, lds + Cfg::A_BYTES, 0);
    __syncthreads();
    const int nk = static_cast<int>(a.ld / BK);
    for (int kt = 0; kt < nk; ++kt) {
        char* cur = lds + (kt & 1) * Cfg::STAGE;
        char* nxt = lds + ((kt & 1) ^ 1) * Cfg::STAGE;
        const bool more = kt + 1 < nk;
        const PrefetchRows2<BT> pf{ra, rb, rs, nxt, nxt + Cfg::A_BYTES, (kt + 1) * BK, more};
        kstep<FM, FN>(cur, cur + Cfg::A_BYTES, wr0, wc0, acc, pf, NoWork{});
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lk = lane >> 5;
    uint16_t* out = a.out + blk * a.out_stride;
    uint16_t* out_lo = (KIND == kPolySplit) ? a.out_lo + blk * a.out_stride : nullptr;
    const uint16_t* amat = src;   // poly: the b A term reads A itself (pitch ld == ldo)
    const float sc = (KIND == kGram && a.scale) ? a.scale[2 * blk + 1] : 1.0f;
    const bool mirror = ti != tj;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = row0 + wr0 + i * 32 + lr;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            __builtin_amdgcn_sched_barrier(0);   // keep the epilogue one 32 x 32 block at a time
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = col0 + wc0 + j * 32 + g * 8 + lk * 4;
                const int64_t o = (int64_t)r * a.ldo + c0;
                uint16_t hb[4], lb[4];
                if constexpr (KIND == kGram) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) hb[q] = f32_to_bf16(acc[i][j][g * 4 + q] * sc);
                } else {
                    const u32x2 av = *reinterpret_cast<const u32x2*>(amat + o);
                    const float am[4] = {bf16_to_f32(uint16_t(av[0] & 0xffffu)), bf16_to_f32(uint16_t(av[0] >> 16)),
                                         bf16_to_f32(uint16_t(av[1] & 0xffffu)), bf16_to_f32(uint16_t(av[1] >> 16))};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = fmaf(a.cc, acc[i][j][g * 4 + q], a.cb * am[q]);
                        if (r == c0 + q) v += a.ca;
                        hb[q] = f32_to_bf16(v);
                        if constexpr (KIND == kPolySplit) lb[q] = f32_to_bf16(v - bf16_to_f32(hb[q]));
                    }
                }
                *reinterpret_cast<u32x2*>(out + o) = pack4(hb);
                if constexpr (KIND == kPolySplit) *reinterpret_cast<u32x2*>(out_lo + o) = pack4(lb);
                if (mirror) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        out[(int64_t)(c0 + q) * a.ldo + r] = hb[q];
                        if constexpr (KIND == kPolySplit) out_lo[(int64_t)(c0 + q) * a.ldo + r] = lb[q];
                    }
                }
            }
        }
    }
}

struct BxArgs {
    const uint16_t* bh;      // B' hi [mp][mp]
    const uint16_t* bl;      // B' lo (split)
    const uint16_t* xh;      // X hi [mp][np]
    const uint16_t* xl;      // X lo (split)
    uint16_t* oh;            // X' hi
    uint16_t* ol;            // X' lo (split)
    const float* scale;      // [nb][2] (iteration 1) or null
    int64_t bstride, xstride;
    int64_t mp, np;
    uint32_t tiles_i;        // row tiles per block (ti varies fastest)
    uint32_t tiles;          // tiles per block
    uint32_t total;          // tiles * blocks in this launch
    uint32_t bbytes, xbytes; // bytes of one B' / X matrix
};

template <bool SPLIT, int BM, int BN>
__global__ __launch_bounds__(NTHR) void k_bx(BxArgs a) {
    using Cfg = TileCfg<BM, BN>;
    constexpr int FM = Cfg::FM, FN = Cfg::FN;
    constexpr int NOPS = SPLIT ? 2 : 1;            // hi (and lo) planes of each operand
    constexpr int STAGE = NOPS * Cfg::STAGE;
    __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

    const uint32_t L = xcd_logical(blockIdx.x, a.total);
    const int64_t blk = L / a.tiles;
    const uint32_t tile = L % a.tiles;
    const int ti = static_cast<int>(tile % a.tiles_i), tj = static_cast<int>(tile / a.tiles_i);
    const __amdgpu_buffer_rsrc_t rbh_s = make_rsrc(a.bh + blk * a.bstride, a.bbytes);
    const __amdgpu_buffer_rsrc_t rxh_s = make_rsrc(a.xh + blk * a.xstride, a.xbytes);
    __amdgpu_buffer_rsrc_t rbl_s = rbh_s, rxl_s = rxh_s;
    if constexpr (SPLIT) {
        rbl_s = make_rsrc(a.bl + blk * a.bstride, a.bbytes);
        rxl_s = make_rsrc(a.xl + blk * a.xstride, a.xbytes);
    }
    const int row0 = ti * BM, col0 = tj * BN;
    const int wave = threadIdx.x >> 6;
    const int wr0 = (wave >> 1) * Cfg::TM, wc0 = (wave & 1) * Cfg::TN;

    f32x16 acc[FM][FN];
    zero_acc(acc);

    // stage layout: [Bh | Xh | Bl | Xl]; B' arrives by DMA, X through registers
    RowDma<BM> rbh, rbl;
    ColTile<BN> cxh, cxl;
    rbh.init(a.mp, row0);
    cxh.init(a.np, col0);
    rbh.load(rbh_s, lds, 0);
    cxh.load(rxh_s, 0);
    if constexpr (SPLIT) {
        rbl.init(a.mp, row0);
        cxl.init(a.np, col0);
        rbl.load(rbl_s, lds + Cfg::STAGE, 0);
        cxl.load(rxl_s, 0);
    }
    cxh.store(lds + Cfg::A_BYTES);
    if constexpr (SPLIT) cxl.store(lds + Cfg::STAGE + Cfg::A_BYTES);
    __syncthreads();
    const int nk = static_cast<int>(a.mp / BK);
    for (int kt = 0; kt < nk; ++kt) {
        char* cur = lds + (kt & 1) * STAGE;
        char* nxt = lds + ((kt & 1) ^ 1) * STAGE;
        const bool more = kt + 1 < nk;
        const int k1 = (kt + 1) * BK;
        const PrefetchRowCol<BM, BN> pfh{rbh, cxh, rbh_s, rxh_s, nxt, k1, more};
        const StoreCols<BN> sth{cxh, nxt + Cfg::A_BYTES, more};
        if constexpr (!SPLIT) {
            kstep<FM, FN>(cur, cur + Cfg::A_BYTES, wr0, wc0, acc, pfh, sth);
        } else {
            const PrefetchRowCol<BM, BN> pfl{rbl, cxl, rbl_s, rxl_s, nxt + Cfg::STAGE, k1, more};
            const StoreCols<BN> stl{cxl, nxt + Cfg::STAGE + Cfg::A_BYTES, more};
            kstep<FM, FN>(cur, cur + Cfg::A_BYTES, wr0, wc0, acc, Both<decltype(pfh), decltype(pfl)>{pfh, pfl},
                          NoWork{});
            kstep<FM, FN>(cur, cur + Cfg::STAGE + Cfg::A_BYTES, wr0, wc0, acc, NoWork{}, NoWork{});  // Bh Xl
            kstep<FM, FN>(cur + Cfg::STAGE, cur + Cfg::A_BYTES, wr0, wc0, acc, NoWork{},             // Bl Xh
                          Both<decltype(sth), decltype(stl)>{sth, stl});
        }
        __syncthreads();
    }

    const int lane = threadIdx.x & 63;
    const int lr = lane & 31, lk = lane >> 5;
    const float sc = a.scale ? a.scale[2 * blk] : 1.0f;
    uint16_t* oh = a.oh + blk * a.xstride;
    uint16_t* ol = SPLIT ? a.ol + blk * a.xstride : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int r = row0 + wr0 + i * 32 + lr;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            __builtin_amdgcn_sched_barrier(0);   // keep the epilogue one 32 x 32 block at a time
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = col0 + wc0 + j * 32 + g * 8 + lk * 4;
                const int64_t o = (int64_t)r * a.np + c0;
                uint16_t hb[4], lb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float v = sc * acc[i][j][g * 4 + q];
                    hb[q] = f32_to_bf16(v);
                    if constexpr (SPLIT) lb[q] = f32_to_bf16(v - bf16_to_f32(hb[q]));
                }
                *reinterpret_cast<u32x2*>(oh + o) = pack4(hb);
                if constexpr (SPLIT) *reinterpret_cast<u32x2*>(ol + o) = pack4(lb);
            }
        }
    }
}

// Every kernel instantiation is named explicitly: with implicit instantiation
// from the launchers below, hipcc emitted host launch stubs for only some of
// them, leaving undefined symbols in the shared library.
template __global__ void k_sym<kGram, 128>(SymArgs);
template __global__ void k_sym<kGram, 256>(SymArgs);
template __global__ void k_sym<kPoly, 128>(SymArgs);
template __global__ void k_sym<kPoly, 256>(SymArgs);
template __global__ void k_sym<kPolySplit, 128>(SymArgs);
template __global__ void k_bx<false, 128, 128>(BxArgs);
template __global__ void k_bx<false, 256, 256>(BxArgs);
template __global__ void k_bx<true, 128, 128>(BxArgs);

constexpr int64_t kCUs = 256;

// 256-wide symmetric tiles when the side divides and they give at least one
// full wave of workgroups; 128 otherwise.
bool use_big_sym(const Plan& p) {
    if (p.mp % 256 != 0) return false;
    const int64_t T = p.mp / 256;
    return p.nb * T * (T + 1) / 2 >= kCUs;
}

bool use_big_bx(const Plan& p) {
    if (p.mp % 256 != 0 || p.np % 256 != 0) return false;
    return p.nb * (p.mp / 256) * (p.np / 256) >= kCUs;
}

template <int KIND, int BT>
hipError_t run_sym(const Plan& p, SymArgs a, hipStream_t s) {
    a.T = static_cast<int>(p.mp / BT);
    a.tiles = static_cast<uint32_t>(a.T * (a.T + 1) / 2);
    const int64_t total = int64_t(a.tiles) * p.nb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    a.total = static_cast<uint32_t>(total);
    k_sym<KIND, BT><<<dim3(a.total), dim3(NTHR), 0, s>>>(a);
    return hipGetLastError();
}

template <bool SPLIT, int BM, int BN>
hipError_t run_bx(const Plan& p, BxArgs a, hipStream_t s) {
    a.tiles_i = static_cast<uint32_t>(p.mp / BM);
    a.tiles = a.tiles_i * static_cast<uint32_t>(p.np / BN);
    const int64_t total = int64_t(a.tiles) * p.nb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    a.total = static_cast<uint32_t>(total);
    k_bx<SPLIT, BM, BN><<<dim3(a.total), dim3(NTHR), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gram(const Plan& p, const uint16_t* x, uint16_t* a_out, const float* scale2,
                       hipStream_t s) {
    SymArgs a{};
    a.src = x;
    a.out = a_out;
    a.scale = scale2;
    a.src_stride = p.mp * p.np;
    a.out_stride = p.mp * p.mp;
    a.ld = p.np;
    a.ldo = p.mp;
    a.src_bytes = static_cast<uint32_t>(p.mp * p.np * 2);
    return use_big_sym(p) ? run_sym<kGram, 256>(p, a, s) : run_sym<kGram, 128>(p, a, s);
}

hipError_t launch_poly(const Plan& p, const uint16_t* a_in, uint16_t* b_hi, uint16_t* b_lo,
                       float ca, float cb, float cc, hipStream_t s) {
    SymArgs a{};
    a.src = a_in;
    a.out = b_hi;
    a.out_lo = b_lo;
    a.src_stride = p.mp * p.mp;
    a.out_stride = p.mp * p.mp;
    a.ld = p.mp;
    a.ldo = p.mp;
    a.ca = ca;
    a.cb = cb;
    a.cc = cc;
    a.src_bytes = static_cast<uint32_t>(p.mp * p.mp * 2);
    if (b_lo) return run_sym<kPolySplit, 128>(p, a, s);
    return use_big_sym(p) ? run_sym<kPoly, 256>(p, a, s) : run_sym<kPoly, 128>(p, a, s);
}

hipError_t launch_bx(const Plan& p, const uint16_t* b_hi, const uint16_t* b_lo,
                     const uint16_t* x_hi, const uint16_t* x_lo, uint16_t* out_hi,
                     uint16_t* out_lo, const float* scale1, hipStream_t s) {
    BxArgs a{};
    a.bh = b_hi;
    a.bl = b_lo;
    a.xh = x_hi;
    a.xl = x_lo;
    a.oh = out_hi;
    a.ol = out_lo;
    a.scale = scale1;
    a.bstride = p.mp * p.mp;
    a.xstride = p.mp * p.np;
    a.mp = p.mp;
    a.np = p.np;
    a.bbytes = static_cast<uint32_t>(p.mp * p.mp * 2);
    a.xbytes = static_cast<uint32_t>(p.mp * p.np * 2);
    if (b_lo) return run_bx<true, 128, 128>(p, a, s);
    return use_big_bx(p) ? run_bx<false, 256, 256>(p, a, s) : run_bx<false, 128, 128>(p, a, s);
}

}  // namespace muon
