// AdamW step for the non-matrix parameters (embeddings, head, scalars): one
// fused, HBM-bound launch over up to kAdamTab tensors.
//
// Per element, in the order of DistAdam.step in the article on moving the
// Adam gradient reduce-scatter into a backward hook (modded-nanogpt record of
// 2025-10-31, "change two"): decoupled decay first (p *= 1 - lr lr_mul wd
// wd_mul), the two moment updates, then p -= step m / (sqrt(v) + eps) with the
// bias corrections folded into step = lr lr_mul (1 - beta2^t)^0.5 /
// (1 - beta1^t).  The per-tensor decay and step are formed on the host in
// double precision.
//
// Traffic per element: p 4 + 4, g 2, m 4 + 4, v 4 + 4 = 26 bytes.  Each block
// owns a chunk of kAdamChunk consecutive elements of one tensor; a thread
// issues all loads of its share before any store.  Tensors whose four buffers
// are 16-byte aligned move 8 elements per 16-byte access.
#include "muon_internal.hpp"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kGroupsPerThread = 1;   // 8-element groups per thread (1 measured fastest; 2, 4, 8 slower)
constexpr int64_t kAdamChunk = int64_t(kThreads) * kGroupsPerThread * 8;

struct AdamArgs {
    AdamEntry t[kAdamTab];
    int n;
    float b1, omb1, b2, omb2, eps;
};

struct Moments {
    float b1, omb1, b2, omb2, eps;
};

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, float decay, float step,
                                          const Moments& k) {
    p *= decay;
    m = fmaf(k.omb1, g, k.b1 * m);
    v = fmaf(k.omb2 * g, g, k.b2 * v);
    p = fmaf(-step, m / (sqrtf(v) + k.eps), p);
}

__global__ __launch_bounds__(kThreads) void k_adamw(AdamArgs a) {
    const uint32_t chunk = blockIdx.x;
    int ti = 0;
    for (int i = 1; i < a.n; ++i)
        if (chunk >= a.t[i].first_chunk) ti = i;
    const AdamEntry& e = a.t[ti];
    const Moments k{a.b1, a.omb1, a.b2, a.omb2, a.eps};
    const int64_t base = int64_t(chunk - e.first_chunk) * kAdamChunk;
    const int64_t len = min(kAdamChunk, e.numel - base);
    float* P = e.p + base;
    const uint16_t* G = e.g + base;
    float* M = e.m + base;
    float* V = e.v + base;
    const int t = threadIdx.x;

    int64_t done = 0;
    if (e.vec) {
        const int ng = static_cast<int>(len >> 3);
        f32x4 p[2 * kGroupsPerThread], m[2 * kGroupsPerThread], v[2 * kGroupsPerThread];
        u16x8 g[kGroupsPerThread];
#pragma unroll
        for (int u = 0; u < kGroupsPerThread; ++u) {
            const int q = min(t + kThreads * u, max(ng - 1, 0));
            if (ng == 0) break;
            g[u] = *reinterpret_cast<const u16x8*>(G + 8 * q);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                p[2 * u + h] = *reinterpret_cast<const f32x4*>(P + 8 * q + 4 * h);
                m[2 * u + h] = *reinterpret_cast<const f32x4*>(M + 8 * q + 4 * h);
                v[2 * u + h] = *reinterpret_cast<const f32x4*>(V + 8 * q + 4 * h);
            }
        }
#pragma unroll
        for (int u = 0; u < kGroupsPerThread; ++u) {
            const int q = t + kThreads * u;
            if (q >= ng) continue;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 pp = p[2 * u + h], mm = m[2 * u + h], vv = v[2 * u + h];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float pj = pp[j], mj = mm[j], vj = vv[j];
                    adam_elem(pj, bf16_to_f32(g[u][4 * h + j]), mj, vj, e.decay, e.step, k);
                    pp[j] = pj;
                    mm[j] = mj;
                    vv[j] = vj;
                }
                *reinterpret_cast<f32x4*>(P + 8 * q + 4 * h) = pp;
                *reinterpret_cast<f32x4*>(M + 8 * q + 4 * h) = mm;
                *reinterpret_cast<f32x4*>(V + 8 * q + 4 * h) = vv;
            }
        }
        done = int64_t(ng) * 8;
    }
    // Element-wise: whole chunks of unaligned tensors, and the last < 8
    // elements of an aligned one.  Batches of 8 loads per thread in flight.
    for (int64_t i0 = done; i0 < len; i0 += int64_t(kThreads) * 8) {
        float p[8], g[8], m[8], v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = min(i0 + t + int64_t(kThreads) * u, len - 1);
            p[u] = P[i];
            g[u] = bf16_to_f32(G[i]);
            m[u] = M[i];
            v[u] = V[i];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t i = i0 + t + int64_t(kThreads) * u;
            if (i >= len) continue;
            adam_elem(p[u], g[u], m[u], v[u], e.decay, e.step, k);
            P[i] = p[u];
            M[i] = m[u];
            V[i] = v[u];
        }
    }
}

}  // namespace

int64_t adamw_chunks(int64_t numel) { return (numel + kAdamChunk - 1) / kAdamChunk; }

hipError_t launch_adamw(const AdamEntry* entries, int n, float beta1, float beta2, float eps, hipStream_t s) {
    if (n < 1 || n > kAdamTab) return hipErrorInvalidValue;
    AdamArgs a{};
    a.n = n;
    a.b1 = beta1;
    a.omb1 = 1.0f - beta1;
    a.b2 = beta2;
    a.omb2 = 1.0f - beta2;
    a.eps = eps;
    uint32_t chunks = 0;
    for (int i = 0; i < n; ++i) {
        a.t[i] = entries[i];
        a.t[i].first_chunk = chunks;
        const int64_t c = adamw_chunks(entries[i].numel);
        if (c < 1 || int64_t(chunks) + c > 0x7fffffff) return hipErrorInvalidValue;
        chunks += static_cast<uint32_t>(c);
    }
    k_adamw<<<dim3(chunks), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace muon
