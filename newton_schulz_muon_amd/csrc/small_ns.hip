// Whole Muon step for small NS blocks (m <= 64, m * n <= 8192), one 256-thread
// workgroup per block, everything in LDS and fp32: one launch for the whole
// step instead of the ~17 of the MFMA path, whose tiles such blocks cannot
// fill.  The three products run on fp32 matrix cores (exact fp32 products,
// fp32 accumulation) for m > 4, with the 16-row tile count T = ceil(m / 16)
// a template parameter so that every per-wave split is fixed at compile time,
// and as vector FMAs with the reduction split over all 256 threads for m <= 4.
//
// The 124M custom-sizing model sends its small gate parameters through Muon
// ahead of the large groups ("Muon Custom Sizing" walkthrough, sections 1 and
// 2.1).  Such blocks are far too small for matrix cores and, for a 1 x n block,
// bf16 rounding of B is amplified by the cancellation in p(1) = a + b + c, so
// this path keeps the iterate, A and B in fp32 and fuses momentum, norm, the
// NS loop and the update into one launch.  The arithmetic is the same as the
// large path: momentum lerp and Nesterov look-ahead (section 4 of that page),
// X = U / (|U|_F + eps), then X <- a X + (b A + c A A) X with A = X X^T
// (parameter-golf walkthrough, Part 1), then the decoupled-decay update.
#include "muon_internal.hpp"

namespace muon {
namespace {

struct SmallArgs {
    MatTable tab;     // per-matrix buffers and scalars (tab.n > 0) or strided
    const uint16_t* src;
    float* mom;
    float* P;
    uint16_t* out;
    int64_t be;       // r * c
    int r, c, m, n;
    bool tall;
    int mode;         // PrepMode
    int steps;
    float mu, omm, decay, step;
    float a, b, cc, eps;
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// LDS layout.  The iterate is m rows of ldx floats (ldx = n rounded up to 64,
// zero beyond n); A and B are 64 x 64.  Every row starts on bank 0 and its
// 16-byte chunks are XOR-permuted inside each 64-float segment by
// s(r) = 4 (r mod 4) + (r / 4 mod 4), so that both read patterns below touch
// 64 distinct banks: 16 consecutive rows at one chunk (Gram-type operands)
// and 4 consecutive rows x 16 consecutive columns (B X operands).
__device__ __forceinline__ int row_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int sw(int r, int k, int ld) {
    return r * ld + (((k >> 2) ^ row_swz(r)) << 2) + (k & 3);
}
__device__ __forceinline__ f32x4 ld_chunk(const float* M, int r, int c, int ld) {
    return *reinterpret_cast<const f32x4*>(M + r * ld + ((c ^ row_swz(r)) << 2));
}
__device__ __forceinline__ void st_chunk(float* M, int r, int c, int ld, f32x4 v) {
    *reinterpret_cast<f32x4*>(M + r * ld + ((c ^ row_swz(r)) << 2)) = v;
}

constexpr int kLdA = 64;
constexpr int kXMax = kSmallMaxElems + 64 * kSmallMaxM;   // m * ldx <= m n + 63 m
constexpr int kPerThread = kSmallMaxElems / 256;          // elements per thread (one pass)
static_assert(kPerThread * 256 >= kSmallMaxElems && kPerThread % 8 == 0, "a block is loaded in one pass");
constexpr int kMaxGramSlots = 5;                          // upper 16 x 16 tiles per wave group
// Gram partial tiles, indexed (writer wave * kMaxGramSlots + slot).
constexpr int kPartMax = 3 * kMaxGramSlots * 256;
static_assert(kSmallMaxM <= 64, "A and B are 64 x 64 in LDS");

// Wave index as a scalar, so per-wave work splits branch on scalar registers.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Upper-triangle 16 x 16 tile u (row-major over ti <= tj) of a T x T tiling.
__device__ __forceinline__ void upper_tile(int u, int T, int& ti, int& tj) {
    ti = 0;
    for (int len = T; len > 0 && u >= len; --len) {
        u -= len;
        ++ti;
    }
    tj = ti + u;
}

// Writes D (one 16 x 16 tile in the MFMA output layout: lane (g, jj) holds
// rows 4 g + e, e < 4, of column jj) and its mirror image; entries below the
// diagonal come from the mirror only, so the stored matrix is exactly
// symmetric.
__device__ __forceinline__ void store_sym_tile(float* M, int ti, int tj, f32x4 v) {
    const int lane = threadIdx.x & 63, g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * ti + 4 * g + e, j = 16 * tj + jj;
        if (i <= j) {
            M[sw(i, j, kLdA)] = v[e];
            M[sw(j, i, kLdA)] = v[e];
        }
    }
}

// ---- matrix-core products (m > 4): fp32 MFMA 16x16x4, exact fp32 products.
// Lane (g, ii) of an MFMA supplies row ii, k-slot g of the left operand and
// column ii, k-slot g of the right one.  Rows of X at or beyond m are read
// from row m - 1 (in bounds, no branch) and their contributions are dropped:
// the Gram tile stores zeros there, so A and B vanish beyond m, and B X
// multiplies those rows of X by zeros of B.

// How the 4 waves share the T (T + 1) / 2 upper Gram tiles: 4 / KS groups of
// KS waves, each group owning NSL tiles and its KS waves splitting the
// reduction over n.
template <int T>
struct GramSplit {
    static constexpr int U = T * (T + 1) / 2;
    static constexpr int KS = T <= 2 ? 4 : 2;
    static constexpr int G = 4 / KS;
    static constexpr int NSL = U / G;
    static_assert(U % G == 0 && NSL <= kMaxGramSlots, "groups own equal tile counts");
    static_assert(G * (KS - 1) <= 3, "partial buffer holds at most 3 writer waves");
};

// A = X X^T (upper tiles + mirror).  The first wave of each group adds the
// others' partial tiles in a fixed order, so results are reproducible.
template <int T>
__device__ void gram_mfma(const float* X, int ldx, int m, int n, float* A, float* part) {
    using S = GramSplit<T>;
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, ii = lane & 15;
    const int gi = w / S::KS, kp = w % S::KS;
    const int nks = (n + 15) >> 4;
    const int k0 = kp * nks / S::KS, k1 = (kp + 1) * nks / S::KS;
    int ti[S::NSL], tj[S::NSL], oa[S::NSL], ob[S::NSL], sa[S::NSL], sb[S::NSL];
    f32x4 acc[S::NSL];
#pragma unroll
    for (int sl = 0; sl < S::NSL; ++sl) {
        upper_tile(gi + S::G * sl, T, ti[sl], tj[sl]);
        const int ra = min(16 * ti[sl] + ii, m - 1), rb = min(16 * tj[sl] + ii, m - 1);
        oa[sl] = ra * ldx;
        ob[sl] = rb * ldx;
        sa[sl] = row_swz(ra);
        sb[sl] = row_swz(rb);
        acc[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int ks = k0; ks < k1; ++ks) {
        const int c = 4 * ks + g;
        f32x4 pa[S::NSL], pb[S::NSL];
#pragma unroll
        for (int sl = 0; sl < S::NSL; ++sl) {
            pa[sl] = *reinterpret_cast<const f32x4*>(X + oa[sl] + ((c ^ sa[sl]) << 2));
            pb[sl] = *reinterpret_cast<const f32x4*>(X + ob[sl] + ((c ^ sb[sl]) << 2));
        }
#pragma unroll
        for (int sl = 0; sl < S::NSL; ++sl)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[sl] = mfma4(pa[sl][q], pb[sl][q], acc[sl]);
    }
    if (kp > 0) {
#pragma unroll
        for (int sl = 0; sl < S::NSL; ++sl)
            reinterpret_cast<f32x4*>(part)[((gi * (S::KS - 1) + kp - 1) * kMaxGramSlots + sl) * 64 + lane] = acc[sl];
    }
    __syncthreads();
    if (kp == 0) {
#pragma unroll
        for (int sl = 0; sl < S::NSL; ++sl) {
            f32x4 d = acc[sl];
#pragma unroll
            for (int o = 1; o < S::KS; ++o)
                d += reinterpret_cast<const f32x4*>(part)[((gi * (S::KS - 1) + o - 1) * kMaxGramSlots + sl) * 64 + lane];
            if (16 * tj[sl] + ii >= m) d = f32x4{0.f, 0.f, 0.f, 0.f};   // column >= m (then i <= j >= m too)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (16 * ti[sl] + 4 * g + e >= m) d[e] = 0.f;
            store_sym_tile(A, ti[sl], tj[sl], d);
        }
    }
}

// B' = a I + b A + c A A (A symmetric, so A A = A A^T): upper tiles u = w + 4 s.
// The a X term of the iteration rides on the diagonal of B' (rows < m only).
template <int T>
__device__ void poly_mfma(const float* A, int m, float ca, float cb, float cc, float* B) {
    constexpr int U = T * (T + 1) / 2;
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, ii = lane & 15;
    for (int u = w; u < U; u += 4) {
        int ti, tj;
        upper_tile(u, T, ti, tj);
        f32x4 pa[T], pb[T], av;
#pragma unroll
        for (int ks = 0; ks < T; ++ks) {
            pa[ks] = ld_chunk(A, 16 * ti + ii, 4 * ks + g, kLdA);
            pb[ks] = ld_chunk(A, 16 * tj + ii, 4 * ks + g, kLdA);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = A[sw(16 * ti + 4 * g + e, 16 * tj + ii, kLdA)];
        f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = mfma4(pa[ks][q], pb[ks][q], acc);
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * ti + 4 * g + e, j = 16 * tj + ii;
            v[e] = fmaf(cc, acc[e], cb * av[e]) + ((i == j && i < m) ? ca : 0.f);
        }
        store_sym_tile(B, ti, tj, v);
    }
}

// Y = B' X.  Jobs are 16 x 64 strips (4 output tiles sharing the left
// operand); k slot g of MFMA q is row 16 ks + 4 q + g, and the left operand
// B'(i, k) is read as B'(k, i) (B' is symmetric) so that both operands are
// read as 4 consecutive rows x 16 consecutive columns.  All operand reads of
// a strip are issued before its MFMAs.
template <int T>
__device__ void bx_mfma(const float* B, const float* X, float* Y, int ldx, int m) {
    const int w = wave_id(), lane = threadIdx.x & 63, g = lane >> 4, ii = lane & 15;
    const int NG = ldx >> 6;
    for (int job = w; job < T * NG; job += 4) {
        const int ti = job / NG, j0 = 64 * (job - ti * NG);
        float pa[T][4], pb[T][4][4];
#pragma unroll
        for (int ks = 0; ks < T; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = 16 * ks + 4 * q + g, kc = min(k, m - 1);
                pa[ks][q] = B[sw(k, 16 * ti + ii, kLdA)];
#pragma unroll
                for (int tc = 0; tc < 4; ++tc) pb[ks][q][tc] = X[sw(kc, j0 + 16 * tc + ii, ldx)];
            }
        f32x4 acc[4];
#pragma unroll
        for (int tc = 0; tc < 4; ++tc) acc[tc] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < T; ++ks)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int tc = 0; tc < 4; ++tc) acc[tc] = mfma4(pa[ks][q], pb[ks][q][tc], acc[tc]);
#pragma unroll
        for (int tc = 0; tc < 4; ++tc)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ti + 4 * g + e;
                if (i < m) Y[sw(i, j0 + 16 * tc + ii, ldx)] = acc[tc][e];
            }
    }
}

// ---- vector products for m <= 4 (gates, 1 x n blocks): all 256 threads
// split the length-n reductions; partial sums are combined in a fixed order.
__device__ void ns_iter_tiny(const float* X, float* Y, int ldx, int m, float* A, float* B, float* part,
                             float ca, float cb, float cc) {
    const int t = threadIdx.x, w = wave_id();
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    const int nc = ldx >> 2;
    for (int c = t; c < nc; c += 256) {
        f32x4 xr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[i] = i < m ? ld_chunk(X, i, c, ldx) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = i; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j] = fmaf(xr[i][e], xr[j][e], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = i; j < 4; ++j) {
            if (j >= m) break;
            const float s = wave_sum(acc[i][j]);
            if ((t & 63) == 0) part[w * 16 + 4 * i + j] = s;
        }
    __syncthreads();
    if (t < 16) {
        const int i = t >> 2, j = t & 3;
        if (i < m && j < m) {
            const int p = i <= j ? 4 * i + j : 4 * j + i;
            A[sw(i, j, kLdA)] = ((part[p] + part[16 + p]) + part[32 + p]) + part[48 + p];
        }
    }
    __syncthreads();
    if (t < 16) {
        const int i = t >> 2, j = t & 3;
        if (i < m && j < m) {
            float s = 0.f;
            for (int k = 0; k < m; ++k) s = fmaf(A[sw(i, k, kLdA)], A[sw(k, j, kLdA)], s);
            B[sw(i, j, kLdA)] = fmaf(cc, s, cb * A[sw(i, j, kLdA)]);
        }
    }
    __syncthreads();
    for (int c = t; c < nc; c += 256) {
        f32x4 xr[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) xr[k] = k < m ? ld_chunk(X, k, c, ldx) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= m) break;
            f32x4 y = ca * xr[i];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (k >= m) break;
                const float bik = B[sw(i, k, kLdA)];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = fmaf(bik, xr[k][e], y[e]);
            }
            st_chunk(Y, i, c, ldx, y);
        }
    }
}

// ---- global memory phases.  A thread's elements (at most kPerThread) stay
// in registers across the norm reduction.  Indices past the block are clamped
// to its last element (loaded, unused), so the loads need no branches and are
// in flight together.  VEC: 8 consecutive elements per 16-byte load (the host
// checks be % 8 == 0, c % 8 == 0 and 16-byte aligned buffers), which keeps
// this run-once code short.
// Momentum (step modes) and the sum of squares; v holds the NS input U.
template <bool VEC>
__device__ __forceinline__ float load_block(const SmallArgs& a, const uint16_t* src, float* mom, int be, float* v) {
    const int t = threadIdx.x;
    float ss = 0.f;
    const bool momentum = a.mode != kPrepCast;
    const bool nesterov = a.mode == kPrepNesterov;
    if constexpr (VEC) {
        const int ng = be >> 3, nj = (ng + 255) >> 8;
        u16x8 graw[kPerThread / 8];
        f32x4 mo[kPerThread / 4];
#pragma unroll
        for (int j = 0; j < kPerThread / 8; ++j) {
            if (j >= nj) break;
            const int q = min(t + 256 * j, ng - 1);
            graw[j] = *reinterpret_cast<const u16x8*>(src + 8 * q);
            if (momentum) {
                mo[2 * j] = *reinterpret_cast<const f32x4*>(mom + 8 * q);
                mo[2 * j + 1] = *reinterpret_cast<const f32x4*>(mom + 8 * q + 4);
            }
        }
#pragma unroll
        for (int j = 0; j < kPerThread / 8; ++j) {
            if (j >= nj) break;
            const int q = t + 256 * j;
            f32x4 mn[2];
#pragma unroll
            for (int w8 = 0; w8 < 8; ++w8) {
                const float gr = bf16_to_f32(graw[j][w8]);
                float u = gr;
                if (momentum) {
                    const float mo_ = mo[2 * j + (w8 >> 2)][w8 & 3];
                    const float m1 = fmaf(a.omm, gr - mo_, mo_);
                    mn[w8 >> 2][w8 & 3] = m1;
                    u = nesterov ? fmaf(a.mu, m1 - gr, gr) : m1;
                }
                v[8 * j + w8] = u;
                if (q < ng) ss = fmaf(u, u, ss);
            }
            if (momentum && q < ng) {
                *reinterpret_cast<f32x4*>(mom + 8 * q) = mn[0];
                *reinterpret_cast<f32x4*>(mom + 8 * q + 4) = mn[1];
            }
        }
    } else {
        const int nu = (be + 255) >> 8;
        uint16_t graw[kPerThread];
        float mo[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u >= nu) break;
            const int e = min(t + 256 * u, be - 1);
            graw[u] = src[e];
            if (momentum) mo[u] = mom[e];
        }
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u >= nu) break;
            const int e = t + 256 * u;
            const float gr = bf16_to_f32(graw[u]);
            v[u] = gr;
            if (momentum) {
                const float m1 = fmaf(a.omm, gr - mo[u], mo[u]);
                if (e < be) mom[e] = m1;
                v[u] = nesterov ? fmaf(a.mu, m1 - gr, gr) : m1;
            }
            if (e < be) ss = fmaf(v[u], v[u], ss);
        }
    }
    return ss;
}

// X (oriented) = v * inv.
template <bool VEC>
__device__ __forceinline__ void write_iterate(const SmallArgs& a, int be, int ldx, const float* v, float inv,
                                              float* X) {
    const int t = threadIdx.x, c = a.c;
    if constexpr (VEC) {
        const int ng = be >> 3, nj = (ng + 255) >> 8;
#pragma unroll
        for (int j = 0; j < kPerThread / 8; ++j) {
            if (j >= nj) break;
            const int q = t + 256 * j;
            if (q < ng) {
                const int bi = (8 * q) / c, bj = 8 * q - bi * c;
                if (a.tall) {
#pragma unroll
                    for (int w8 = 0; w8 < 8; ++w8) X[sw(bj + w8, bi, ldx)] = v[8 * j + w8] * inv;
                } else {
                    st_chunk(X, bi, bj >> 2, ldx, f32x4{v[8 * j], v[8 * j + 1], v[8 * j + 2], v[8 * j + 3]} * inv);
                    st_chunk(X, bi, (bj >> 2) + 1, ldx,
                             f32x4{v[8 * j + 4], v[8 * j + 5], v[8 * j + 6], v[8 * j + 7]} * inv);
                }
            }
        }
    } else {
        const int nu = (be + 255) >> 8;
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u >= nu) break;
            const int e = t + 256 * u;
            if (e < be) {
                const int bi = e / c, bj = e - bi * c;
                const int oi = a.tall ? bj : bi, oj = a.tall ? bi : bj;
                X[sw(oi, oj, ldx)] = v[u] * inv;
            }
        }
    }
}

// Stored-layout write-back: NS output (cast mode) or P <- P decay - step O.
template <bool VEC>
__device__ __forceinline__ void store_block(const SmallArgs& a, int be, int ldx, const float* X, float* P,
                                            uint16_t* out, float decay, float step) {
    const int t = threadIdx.x, c = a.c;
    const bool update = a.mode != kPrepCast;
    if constexpr (VEC) {
        const int ng = be >> 3, nj = (ng + 255) >> 8;
        f32x4 pv[kPerThread / 4], o[kPerThread / 4];
#pragma unroll
        for (int j = 0; j < kPerThread / 8; ++j) {
            if (j >= nj) break;
            const int q = min(t + 256 * j, ng - 1);
            if (update) {
                pv[2 * j] = *reinterpret_cast<const f32x4*>(P + 8 * q);
                pv[2 * j + 1] = *reinterpret_cast<const f32x4*>(P + 8 * q + 4);
            }
            const int bi = (8 * q) / c, bj = 8 * q - bi * c;
            if (a.tall) {
#pragma unroll
                for (int w8 = 0; w8 < 8; ++w8) o[2 * j + (w8 >> 2)][w8 & 3] = X[sw(bj + w8, bi, ldx)];
            } else {
                o[2 * j] = ld_chunk(X, bi, bj >> 2, ldx);
                o[2 * j + 1] = ld_chunk(X, bi, (bj >> 2) + 1, ldx);
            }
        }
#pragma unroll
        for (int j = 0; j < kPerThread / 8; ++j) {
            if (j >= nj) break;
            const int q = t + 256 * j;
            if (q >= ng) continue;
            if (update) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = fmaf(-step, o[2 * j + h][e], pv[2 * j + h][e] * decay);
                    *reinterpret_cast<f32x4*>(P + 8 * q + 4 * h) = r;
                }
            }
            if (out) {
                u16x8 ob;
#pragma unroll
                for (int w8 = 0; w8 < 8; ++w8) ob[w8] = f32_to_bf16(o[2 * j + (w8 >> 2)][w8 & 3]);
                *reinterpret_cast<u16x8*>(out + 8 * q) = ob;
            }
        }
    } else {
        const int nu = (be + 255) >> 8;
        float pv[kPerThread], o[kPerThread];
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u >= nu) break;
            const int e = min(t + 256 * u, be - 1);
            if (update) pv[u] = P[e];
            const int bi = e / c, bj = e - bi * c;
            const int oi = a.tall ? bj : bi, oj = a.tall ? bi : bj;
            o[u] = X[sw(oi, oj, ldx)];
        }
#pragma unroll
        for (int u = 0; u < kPerThread; ++u) {
            if (u >= nu) break;
            const int e = t + 256 * u;
            if (e < be) {
                if (update) P[e] = fmaf(-step, o[u], pv[u] * decay);
                if (out) out[e] = f32_to_bf16(o[u]);
            }
        }
    }
}

// T = ceil(m / 16) for m > 4; T = 0 selects the vector path (m <= 4).
template <int T, bool VEC>
__global__ __launch_bounds__(256) void k_small(SmallArgs a) {
    __shared__ __attribute__((aligned(16))) float buf0[kXMax];
    __shared__ __attribute__((aligned(16))) float buf1[kXMax];
    __shared__ __attribute__((aligned(16))) float Am[kLdA * kLdA];
    __shared__ __attribute__((aligned(16))) float Bm[kLdA * kLdA];
    __shared__ __attribute__((aligned(16))) float part[T == 0 ? 64 : kPartMax];
    __shared__ float red[4];

    const int t = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const bool momentum = a.mode != kPrepCast;
    const uint16_t* src;
    float* mom = nullptr;
    float* P = nullptr;
    uint16_t* out;
    float decay = a.decay, step = a.step;
    if (a.tab.n > 0) {
        const int64_t mi = blk / a.tab.v, sub = blk % a.tab.v;
        src = a.tab.src[mi] + sub * a.be;
        if (momentum) {
            mom = a.tab.mom[mi] + sub * a.be;
            P = a.tab.P[mi] + sub * a.be;
        }
        out = a.tab.out[mi] ? a.tab.out[mi] + sub * a.be : nullptr;
        decay = a.tab.decay[mi];
        step = a.tab.step[mi];
    } else {
        src = a.src + blk * a.be;
        if (momentum) {
            mom = a.mom + blk * a.be;
            P = a.P + blk * a.be;
        }
        out = a.out ? a.out + blk * a.be : nullptr;
    }
    const int m = a.m, n = a.n;
    const int be = static_cast<int>(a.be);
    const int ldx = (n + 63) & ~63;
    float* X = buf0;
    float* Y = buf1;

    float v[kPerThread];
    float ss = load_block<VEC>(a, src, mom, be, v);
    // The columns beyond n are zeroed: the products read them, and B X then
    // keeps them zero.
    const int pad = ldx - n;
    for (int e = t; e < m * pad; e += 256) X[sw(e / pad, n + e % pad, ldx)] = 0.f;
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    write_iterate<VEC>(a, be, ldx, v, 1.0f / (sqrtf(tot) + a.eps), X);

    for (int it = 0; it < a.steps; ++it) {
        __syncthreads();
        if constexpr (T == 0) {
            ns_iter_tiny(X, Y, ldx, m, Am, Bm, part, a.a, a.b, a.cc);
        } else {
            gram_mfma<T>(X, ldx, m, n, Am, part);        // A = X X^T
            __syncthreads();
            poly_mfma<T>(Am, m, a.a, a.b, a.cc, Bm);     // B' = a I + b A + c A A
            __syncthreads();
            bx_mfma<T>(Bm, X, Y, ldx, m);                // Y = B' X
        }
        float* tmp = X;
        X = Y;
        Y = tmp;
    }
    __syncthreads();
    store_block<VEC>(a, be, ldx, X, P, out, decay, step);
}

template <int T>
void launch_t(bool vec, dim3 grid, hipStream_t s, const SmallArgs& a) {
    if (vec)
        k_small<T, true><<<grid, dim3(256), 0, s>>>(a);
    else
        k_small<T, false><<<grid, dim3(256), 0, s>>>(a);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_small(const Plan& p, const SmallStep& st, hipStream_t s, const MatTable* tab) {
    if (p.nb > 0x7fffffff || p.m > kSmallMaxM || p.m * p.n > kSmallMaxElems) return hipErrorInvalidValue;
    if (st.mode != kPrepCast && st.mode != kPrepNesterov && st.mode != kPrepPlain) return hipErrorInvalidValue;
    SmallArgs a{};
    if (tab != nullptr) {
        if (tab->n < 1 || tab->n > kTabMax || tab->v != p.v || p.nb != int64_t(tab->n) * tab->v)
            return hipErrorInvalidValue;
        a.tab = *tab;
    }
    a.src = st.src;
    a.mom = st.mom;
    a.P = st.params;
    a.out = st.out;
    a.be = p.r * p.c;
    a.r = static_cast<int>(p.r);
    a.c = static_cast<int>(p.c);
    a.m = static_cast<int>(p.m);
    a.n = static_cast<int>(p.n);
    a.tall = p.tall;
    a.mode = st.mode;
    a.steps = st.ns_steps;
    a.mu = st.mu;
    a.omm = 1.0f - st.mu;
    a.decay = st.decay;
    a.step = st.step;
    a.a = st.a;
    a.b = st.b;
    a.cc = st.c;
    a.eps = st.eps;
    // 16-byte vector access needs whole 8-element groups inside one stored
    // row and every block's buffers on 16-byte boundaries.
    bool vec = a.be % 8 == 0 && a.c % 8 == 0;
    const bool momentum = st.mode != kPrepCast;
    if (tab != nullptr) {
        for (int i = 0; i < tab->n && vec; ++i)
            vec = aligned16(tab->src[i]) && (!momentum || (aligned16(tab->mom[i]) && aligned16(tab->P[i]))) &&
                  (tab->out[i] == nullptr || aligned16(tab->out[i]));
    } else {
        vec = vec && aligned16(st.src) && (!momentum || (aligned16(st.mom) && aligned16(st.params))) &&
              (st.out == nullptr || aligned16(st.out));
    }
    const dim3 grid(static_cast<unsigned>(p.nb));
    switch (p.m <= 4 ? 0 : (p.m + 15) / 16) {
        case 0: launch_t<0>(vec, grid, s, a); break;
        case 1: launch_t<1>(vec, grid, s, a); break;
        case 2: launch_t<2>(vec, grid, s, a); break;
        case 3: launch_t<3>(vec, grid, s, a); break;
        case 4: launch_t<4>(vec, grid, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace muon
