// MFMA kernels of the quintic Newton-Schulz iteration (gfx950, bf16 in, fp32
// accumulate), parameter-golf walkthrough Part 1 (A = X X^T, B = b A + c A A,
// X = a X + B X) with the coefficients of the "Muon Custom Sizing"
// walkthrough, section 2.3, which also names a symmetric kernel for X X^T.
//
//   k_sym<GRAM>  A = scale * X X^T     K = np, both operands rows of X
//   k_sym<POLY>  B = b A + c A A^T     K = mp, A symmetric so A A = A A^T
//   k_bx         X' = scale * (a X + B X)   K = mp, X read k-major
//
// A and B are symmetric, so k_sym computes only the tiles (ti <= tj) of the
// upper triangle and writes each off-diagonal tile twice (C and C^T).
//
// Tiling: a 256-thread workgroup computes a 128 x 128 output tile; each of
// its 4 waves owns 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators.
// The K loop steps by 64.  Operand tiles are staged in LDS as 128 rows x 64
// bf16 (8 chunks of 16 bytes per row) with the chunk index XOR-swizzled by the
// row, so 16-byte fragment reads and the transposing 8-byte writes of k_bx
// hit distinct banks.  The next K slice is fetched into registers while the
// current one is multiplied.
//
// MFMA 32x32x16 operand layout used here: lane l supplies row (l % 32) of its
// operand and 8 consecutive k values starting at 8 * (l / 32); the result
// element (i, j) sits in lane 32 * ((i / 4) % 2) + j, register 4 * (i / 8) + i % 4.
// Any k permutation shared by both operands gives the same sum.
#include "muon_internal.hpp"

namespace muon {
namespace {

constexpr int BM = 128;
constexpr int BK = 64;
constexpr int NTHR = 256;
constexpr int TILE_BYTES = BM * BK * 2;   // 16 KB per operand tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return (row << 7) + ((chunk ^ swz(row)) << 4);
}

// 128 rows x 64 k of a k-contiguous matrix.
struct RowTile { u32x4 v[4]; };

__device__ __forceinline__ void load_rows(RowTile& t, const uint16_t* __restrict__ src, int64_t ld,
                                          int row0, int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int v = threadIdx.x + NTHR * q;
        const int row = v >> 3, ch = v & 7;
        t.v[q] = *reinterpret_cast<const u32x4*>(src + (int64_t)(row0 + row) * ld + k0 + ch * 8);
    }
}

__device__ __forceinline__ void store_rows(const RowTile& t, char* lds) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int v = threadIdx.x + NTHR * q;
        const int row = v >> 3, ch = v & 7;
        *reinterpret_cast<u32x4*>(lds + lds_off(row, ch)) = t.v[q];
    }
}

// 64 k x 128 columns of a column-contiguous matrix (X in B X).  Thread
// (jg = t % 16, kg = t / 16) loads rows 4kg..4kg+3 at columns 8jg..8jg+7 and
// writes them transposed: LDS row = column, 4 k values per 8-byte store.
struct ColTile { u32x4 v[4]; };

__device__ __forceinline__ void load_cols(ColTile& t, const uint16_t* __restrict__ src, int64_t ld,
                                          int k0, int col0) {
    const int jg = threadIdx.x & 15, kg = threadIdx.x >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        t.v[r] = *reinterpret_cast<const u32x4*>(src + (int64_t)(k0 + kg * 4 + r) * ld + col0 + jg * 8);
}

__device__ __forceinline__ void store_cols(const ColTile& t, char* lds) {
    const int jg = threadIdx.x & 15, kg = threadIdx.x >> 4;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        const int p = cc >> 1;
        const uint32_t a0 = t.v[0][p], a1 = t.v[1][p], a2 = t.v[2][p], a3 = t.v[3][p];
        u32x2 w;
        if (cc & 1) {
            w[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            w[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
            w[0] = (a0 & 0xffffu) | (a1 << 16);
            w[1] = (a2 & 0xffffu) | (a3 << 16);
        }
        const int row = jg * 8 + cc;
        *reinterpret_cast<u32x2*>(lds + lds_off(row, kg >> 1) + ((kg & 1) << 3)) = w;
    }
}

__device__ __forceinline__ void mfma_slice(const char* As, const char* Bs, f32x16 (&acc)[2][2]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + lk;
        bf16x8 a[2], b[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            a[mt] = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 64 + mt * 32 + lr, ch));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            b[nt] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wn * 64 + nt * 32 + lr, ch));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b[nt], acc[mt][nt], 0, 0, 0);
    }
}

enum SymKind { kGram = 0, kPoly = 1, kPolySplit = 2 };

struct SymArgs {
    const uint16_t* src;     // X (Gram) or A (poly), this launch's first block
    uint16_t* out;           // A (Gram) or B hi (poly)
    uint16_t* out_lo;        // B lo (poly split)
    const float* scale;      // [nb][2] (Gram, iteration 1) or null
    int64_t src_stride, out_stride;
    int64_t ld;              // row pitch of src = K
    int64_t ldo;             // row pitch of out = mp
    int T;                   // tiles per side
    float cb, cc;
};

template <int KIND>
__global__ __launch_bounds__(NTHR) void k_sym(SymArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[2 * TILE_BYTES];
    char* As = lds;
    char* Bs = lds + TILE_BYTES;

    int id = blockIdx.x, ti = 0, len = a.T;
    while (id >= len) { id -= len; ++ti; --len; }
    const int tj = ti + id;
    const int64_t blk = blockIdx.y;
    const uint16_t* src = a.src + blk * a.src_stride;
    const int row0 = ti * BM, col0 = tj * BM;

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int s = 0; s < 16; ++s) acc[mt][nt][s] = 0.f;

    RowTile ra, rb;
    load_rows(ra, src, a.ld, row0, 0);
    load_rows(rb, src, a.ld, col0, 0);
    const int nk = static_cast<int>(a.ld / BK);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        store_rows(ra, As);
        store_rows(rb, Bs);
        __syncthreads();
        if (kt + 1 < nk) {
            load_rows(ra, src, a.ld, row0, (kt + 1) * BK);
            load_rows(rb, src, a.ld, col0, (kt + 1) * BK);
        }
        mfma_slice(As, Bs, acc);
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lk = lane >> 5;
    uint16_t* out = a.out + blk * a.out_stride;
    uint16_t* out_lo = (KIND == kPolySplit) ? a.out_lo + blk * a.out_stride : nullptr;
    const uint16_t* amat = src;   // poly: the b A term reads A itself (pitch ld == ldo)
    const float sc = (KIND == kGram && a.scale) ? a.scale[2 * blk + 1] : 1.0f;
    const bool mirror = ti != tj;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int j = col0 + wn * 64 + nt * 32 + lr;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int i0 = row0 + wm * 64 + mt * 32 + g * 8 + lk * 4;
                uint16_t hb[4], lb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x = acc[mt][nt][g * 4 + q];
                    float v;
                    if constexpr (KIND == kGram) {
                        v = x * sc;
                    } else {
                        v = fmaf(a.cc, x, a.cb * bf16_to_f32(amat[(int64_t)(i0 + q) * a.ldo + j]));
                    }
                    hb[q] = f32_to_bf16(v);
                    if constexpr (KIND == kPolySplit) lb[q] = f32_to_bf16(v - bf16_to_f32(hb[q]));
                    out[(int64_t)(i0 + q) * a.ldo + j] = hb[q];
                    if constexpr (KIND == kPolySplit) out_lo[(int64_t)(i0 + q) * a.ldo + j] = lb[q];
                }
                if (mirror) {
                    u32x2 w;
                    w[0] = uint32_t(hb[0]) | (uint32_t(hb[1]) << 16);
                    w[1] = uint32_t(hb[2]) | (uint32_t(hb[3]) << 16);
                    *reinterpret_cast<u32x2*>(out + (int64_t)j * a.ldo + i0) = w;
                    if constexpr (KIND == kPolySplit) {
                        w[0] = uint32_t(lb[0]) | (uint32_t(lb[1]) << 16);
                        w[1] = uint32_t(lb[2]) | (uint32_t(lb[3]) << 16);
                        *reinterpret_cast<u32x2*>(out_lo + (int64_t)j * a.ldo + i0) = w;
                    }
                }
            }
        }
    }
}

struct BxArgs {
    const uint16_t* bh;      // B hi [mp][mp]
    const uint16_t* bl;      // B lo (split)
    const uint16_t* xh;      // X hi [mp][np]
    const uint16_t* xl;      // X lo (split)
    uint16_t* oh;            // X' hi
    uint16_t* ol;            // X' lo (split)
    const float* scale;      // [nb][2] (iteration 1) or null
    int64_t bstride, xstride;
    int64_t mp, np;
    int tiles_j;
    float ca;
};

template <bool SPLIT>
__global__ __launch_bounds__(NTHR) void k_bx(BxArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[(SPLIT ? 4 : 2) * TILE_BYTES];
    char* Bh = lds;
    char* Xh = lds + TILE_BYTES;
    char* Bl = lds + 2 * TILE_BYTES;
    char* Xl = lds + 3 * TILE_BYTES;

    const int ti = blockIdx.x / a.tiles_j, tj = blockIdx.x % a.tiles_j;
    const int64_t blk = blockIdx.y;
    const uint16_t* bh = a.bh + blk * a.bstride;
    const uint16_t* bl = SPLIT ? a.bl + blk * a.bstride : nullptr;
    const uint16_t* xh = a.xh + blk * a.xstride;
    const uint16_t* xl = SPLIT ? a.xl + blk * a.xstride : nullptr;
    const int row0 = ti * BM, col0 = tj * BM;

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int s = 0; s < 16; ++s) acc[mt][nt][s] = 0.f;

    RowTile rbh, rbl;
    ColTile cxh, cxl;
    load_rows(rbh, bh, a.mp, row0, 0);
    load_cols(cxh, xh, a.np, 0, col0);
    if constexpr (SPLIT) {
        load_rows(rbl, bl, a.mp, row0, 0);
        load_cols(cxl, xl, a.np, 0, col0);
    }
    const int nk = static_cast<int>(a.mp / BK);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
        store_rows(rbh, Bh);
        store_cols(cxh, Xh);
        if constexpr (SPLIT) {
            store_rows(rbl, Bl);
            store_cols(cxl, Xl);
        }
        __syncthreads();
        if (kt + 1 < nk) {
            const int k1 = (kt + 1) * BK;
            load_rows(rbh, bh, a.mp, row0, k1);
            load_cols(cxh, xh, a.np, k1, col0);
            if constexpr (SPLIT) {
                load_rows(rbl, bl, a.mp, row0, k1);
                load_cols(cxl, xl, a.np, k1, col0);
            }
        }
        mfma_slice(Bh, Xh, acc);
        if constexpr (SPLIT) {
            mfma_slice(Bh, Xl, acc);
            mfma_slice(Bl, Xh, acc);
        }
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, lk = lane >> 5;
    const float sc = a.scale ? a.scale[2 * blk] : 1.0f;
    uint16_t* oh = a.oh + blk * a.xstride;
    uint16_t* ol = SPLIT ? a.ol + blk * a.xstride : nullptr;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int j = col0 + wn * 64 + nt * 32 + lr;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int i = row0 + wm * 64 + mt * 32 + (s >> 2) * 8 + lk * 4 + (s & 3);
                const int64_t o = (int64_t)i * a.np + j;
                float x = bf16_to_f32(xh[o]);
                if constexpr (SPLIT) x += bf16_to_f32(xl[o]);
                const float v = sc * fmaf(a.ca, x, acc[mt][nt][s]);
                const uint16_t h = f32_to_bf16(v);
                oh[o] = h;
                if constexpr (SPLIT) ol[o] = f32_to_bf16(v - bf16_to_f32(h));
            }
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

}  // namespace

hipError_t launch_gram(const Plan& p, const uint16_t* x, uint16_t* a_out, const float* scale2,
                       hipStream_t s) {
    const int T = static_cast<int>(p.mp / BM);
    const unsigned tiles = static_cast<unsigned>(T * (T + 1) / 2);
    SymArgs a{};
    a.src_stride = p.mp * p.np;
    a.out_stride = p.mp * p.mp;
    a.ld = p.np;
    a.ldo = p.mp;
    a.T = T;
    return for_block_chunks(p.nb, [&](int64_t b0, unsigned cnt) {
        SymArgs c = a;
        c.src = x + b0 * a.src_stride;
        c.out = a_out + b0 * a.out_stride;
        c.scale = scale2 ? scale2 + 2 * b0 : nullptr;
        k_sym<kGram><<<dim3(tiles, cnt), dim3(NTHR), 0, s>>>(c);
    });
}

hipError_t launch_poly(const Plan& p, const uint16_t* a_in, uint16_t* b_hi, uint16_t* b_lo,
                       float cb, float cc, hipStream_t s) {
    const int T = static_cast<int>(p.mp / BM);
    const unsigned tiles = static_cast<unsigned>(T * (T + 1) / 2);
    SymArgs a{};
    a.src_stride = p.mp * p.mp;
    a.out_stride = p.mp * p.mp;
    a.ld = p.mp;
    a.ldo = p.mp;
    a.T = T;
    a.cb = cb;
    a.cc = cc;
    return for_block_chunks(p.nb, [&](int64_t b0, unsigned cnt) {
        SymArgs c = a;
        c.src = a_in + b0 * a.src_stride;
        c.out = b_hi + b0 * a.out_stride;
        c.out_lo = b_lo ? b_lo + b0 * a.out_stride : nullptr;
        if (b_lo)
            k_sym<kPolySplit><<<dim3(tiles, cnt), dim3(NTHR), 0, s>>>(c);
        else
            k_sym<kPoly><<<dim3(tiles, cnt), dim3(NTHR), 0, s>>>(c);
    });
}

hipError_t launch_bx(const Plan& p, const uint16_t* b_hi, const uint16_t* b_lo,
                     const uint16_t* x_hi, const uint16_t* x_lo, uint16_t* out_hi,
                     uint16_t* out_lo, float ca, const float* scale1, hipStream_t s) {
    const int tm = static_cast<int>(p.mp / BM), tn = static_cast<int>(p.np / BM);
    const unsigned tiles = static_cast<unsigned>(tm * tn);
    const bool split = b_lo != nullptr;
    BxArgs a{};
    a.bstride = p.mp * p.mp;
    a.xstride = p.mp * p.np;
    a.mp = p.mp;
    a.np = p.np;
    a.tiles_j = tn;
    a.ca = ca;
    return for_block_chunks(p.nb, [&](int64_t b0, unsigned cnt) {
        BxArgs c = a;
        c.bh = b_hi + b0 * a.bstride;
        c.bl = split ? b_lo + b0 * a.bstride : nullptr;
        c.xh = x_hi + b0 * a.xstride;
        c.xl = split ? x_lo + b0 * a.xstride : nullptr;
        c.oh = out_hi + b0 * a.xstride;
        c.ol = split ? out_lo + b0 * a.xstride : nullptr;
        c.scale = scale1 ? scale1 + 2 * b0 : nullptr;
        if (split)
            k_bx<true><<<dim3(tiles, cnt), dim3(NTHR), 0, s>>>(c);
        else
            k_bx<false><<<dim3(tiles, cnt), dim3(NTHR), 0, s>>>(c);
    });
}

}  // namespace muon
