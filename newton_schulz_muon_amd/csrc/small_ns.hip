// Whole Muon step for small NS blocks (m <= 32, m * n <= 4096), one 256-thread
// workgroup per block, everything in LDS and fp32.
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
    int steps;
    float mu, omm, decay, step;
    float a, b, cc, eps;
};

template <int MODE>
__global__ __launch_bounds__(256) void k_small(SmallArgs a) {
    __shared__ float buf0[kSmallMaxElems];
    __shared__ float buf1[kSmallMaxElems];
    __shared__ float Am[kSmallMaxM * kSmallMaxM];
    __shared__ float Bm[kSmallMaxM * kSmallMaxM];
    __shared__ float red[4];

    const int t = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const uint16_t* src;
    float* mom = nullptr;
    float* P = nullptr;
    uint16_t* out;
    float decay = a.decay, step = a.step;
    if (a.tab.n > 0) {
        const int64_t mi = blk / a.tab.v, sub = blk % a.tab.v;
        src = a.tab.src[mi] + sub * a.be;
        if constexpr (MODE != kPrepCast) {
            mom = a.tab.mom[mi] + sub * a.be;
            P = a.tab.P[mi] + sub * a.be;
        }
        out = a.tab.out[mi] ? a.tab.out[mi] + sub * a.be : nullptr;
        decay = a.tab.decay[mi];
        step = a.tab.step[mi];
    } else {
        src = a.src + blk * a.be;
        if constexpr (MODE != kPrepCast) {
            mom = a.mom + blk * a.be;
            P = a.P + blk * a.be;
        }
        out = a.out ? a.out + blk * a.be : nullptr;
    }
    const int c = a.c, m = a.m, n = a.n;
    const int be = static_cast<int>(a.be);
    float* X = buf0;
    float* Y = buf1;

    float ss = 0.f;
    for (int e = t; e < be; e += 256) {
        const int bi = e / c, bj = e % c;
        const float g = bf16_to_f32(src[e]);
        float u = g;
        if constexpr (MODE != kPrepCast) {
            const float mo = mom[e];
            const float mn = fmaf(a.omm, g - mo, mo);
            mom[e] = mn;
            u = (MODE == kPrepNesterov) ? fmaf(a.mu, mn - g, g) : mn;
        }
        const int oi = a.tall ? bj : bi, oj = a.tall ? bi : bj;
        X[oi * n + oj] = u;
        ss = fmaf(u, u, ss);
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float inv = 1.0f / (sqrtf(tot) + a.eps);
    for (int e = t; e < m * n; e += 256) X[e] *= inv;

    for (int it = 0; it < a.steps; ++it) {
        __syncthreads();
        for (int e = t; e < m * m; e += 256) {
            const int i = e / m, j = e % m;
            float s = 0.f;
            for (int k = 0; k < n; ++k) s = fmaf(X[i * n + k], X[j * n + k], s);
            Am[e] = s;
        }
        __syncthreads();
        for (int e = t; e < m * m; e += 256) {
            const int i = e / m, j = e % m;
            float s = 0.f;
            for (int k = 0; k < m; ++k) s = fmaf(Am[i * m + k], Am[k * m + j], s);
            Bm[e] = fmaf(a.cc, s, a.b * Am[e]);
        }
        __syncthreads();
        for (int e = t; e < m * n; e += 256) {
            const int i = e / n, j = e % n;
            float s = 0.f;
            for (int k = 0; k < m; ++k) s = fmaf(Bm[i * m + k], X[k * n + j], s);
            Y[e] = fmaf(a.a, X[e], s);
        }
        float* tmp = X;
        X = Y;
        Y = tmp;
    }
    __syncthreads();

    for (int e = t; e < be; e += 256) {
        const int bi = e / c, bj = e % c;
        const int oi = a.tall ? bj : bi, oj = a.tall ? bi : bj;
        const float o = X[oi * n + oj];
        if constexpr (MODE == kPrepCast) {
            out[e] = f32_to_bf16(o);
        } else {
            P[e] = fmaf(-step, o, P[e] * decay);
            if (out) out[e] = f32_to_bf16(o);
        }
    }
}

}  // namespace

hipError_t launch_small(const Plan& p, const SmallStep& st, hipStream_t s, const MatTable* tab) {
    if (p.nb > 0x7fffffff || p.m > kSmallMaxM || p.m * p.n > kSmallMaxElems) return hipErrorInvalidValue;
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
    a.steps = st.ns_steps;
    a.mu = st.mu;
    a.omm = 1.0f - st.mu;
    a.decay = st.decay;
    a.step = st.step;
    a.a = st.a;
    a.b = st.b;
    a.cc = st.c;
    a.eps = st.eps;
    const dim3 grid(static_cast<unsigned>(p.nb)), block(256);
    switch (st.mode) {
        case kPrepCast: k_small<kPrepCast><<<grid, block, 0, s>>>(a); break;
        case kPrepNesterov: k_small<kPrepNesterov><<<grid, block, 0, s>>>(a); break;
        case kPrepPlain: k_small<kPrepPlain><<<grid, block, 0, s>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace muon
