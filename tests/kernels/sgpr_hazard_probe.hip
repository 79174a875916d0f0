// Test-only kernel: does a vector memory load see an SGPR that a VALU
// instruction wrote just before it?  The library's LDS DMA is inline
// assembly, outside the compiler's hazard recognizer, and the build rejects a
// DMA that reads an SGPR within five wait states of a VALU write of it; this
// probe measures what the hardware needs.
//
// Each lane of each wave, `reps` times: an SGPR holds offset 0 (written by
// the scalar unit long before), a VALU instruction writes a new offset into
// it (KIND 0: v_readfirstlane of a VGPR; KIND 1: v_readlane of a VGPR written
// long before, the pattern of an SGPR restored from a spill), GAP v_nop
// follow, then a buffer_load_dword uses the SGPR as its offset.  With
// src[k] = k the loaded word tells which offset the load used: out[0] counts
// loads that saw the new one, out[1] the old one.  Every address lies inside
// src (the buffer descriptor also bounds-checks).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 rsrc_of(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    return i32x4{static_cast<int>(static_cast<uint32_t>(b)), static_cast<int>((b >> 32) & 0xffffu),
                 static_cast<int>(bytes), 0x00020000};
}

template <int GAP, int KIND>
__global__ __launch_bounds__(256) void k_sgpr_hazard(const uint32_t* src, uint32_t n, uint32_t newoff, uint32_t* out,
                                                     int reps) {
    const i32x4 r = rsrc_of(src, n * 4);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t voff = lane * 4;
    uint32_t seen_new = 0, seen_old = 0;
    for (int i = 0; i < reps; ++i) {
        uint32_t v;
        const uint32_t nv = newoff + static_cast<uint32_t>(i & 7) * 256;
        if constexpr (KIND == 0) {
            asm volatile(
                "s_mov_b32 s40, 0\n\t"
                "s_nop 7\n\t"
                "v_readfirstlane_b32 s40, %1\n\t"
                ".rept %4\n\tv_nop\n\t.endr\n\t"
                "buffer_load_dword %0, %2, %3, s40 offen\n\t"
                "s_waitcnt vmcnt(0)"
                : "=v"(v) : "v"(nv), "v"(voff), "s"(r), "i"(GAP) : "s40", "memory");
        } else {
            asm volatile(
                "s_mov_b32 s40, 0\n\t"
                "v_mov_b32 v250, %1\n\t"
                "s_nop 7\n\t"
                "v_readlane_b32 s40, v250, 5\n\t"
                ".rept %4\n\tv_nop\n\t.endr\n\t"
                "buffer_load_dword %0, %2, %3, s40 offen\n\t"
                "s_waitcnt vmcnt(0)"
                : "=v"(v) : "v"(nv), "v"(voff), "s"(r), "i"(GAP) : "s40", "v250", "memory");
        }
        if (v == lane + nv / 4) ++seen_new;
        else if (v == lane) ++seen_old;
    }
    atomicAdd(&out[0], seen_new);
    atomicAdd(&out[1], seen_old);
}

template <int GAP>
static void launch(int kind, dim3 g, dim3 b, hipStream_t s, const uint32_t* src, uint32_t n, uint32_t newoff,
                   uint32_t* out, int reps) {
    if (kind == 0)
        k_sgpr_hazard<GAP, 0><<<g, b, 0, s>>>(src, n, newoff, out, reps);
    else
        k_sgpr_hazard<GAP, 1><<<g, b, 0, s>>>(src, n, newoff, out, reps);
}

// src: n words on the device holding src[k] = k, n >= 8192; out: two device
// words the caller zeroed; gap in {0, 1, 2, 5}; kind 0 (v_readfirstlane) or 1
// (v_readlane).  blocks x 256 threads, reps loads each.  Returns a hipError_t.
extern "C" int sgpr_hazard_probe_launch(const void* src, uint32_t n, void* out, int gap, int kind, int blocks,
                                        int reps, void* stream) {
    if (n < 8192 || blocks < 1 || reps < 1 || (kind != 0 && kind != 1)) return int(hipErrorInvalidValue);
    // new offsets 16384 + 256 (i % 8) bytes: words up to 4543 + 63 < 8192
    const uint32_t newoff = 16384;
    const dim3 g(blocks), b(256);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t* sp = static_cast<const uint32_t*>(src);
    uint32_t* op = static_cast<uint32_t*>(out);
    switch (gap) {
        case 0: launch<0>(kind, g, b, s, sp, n, newoff, op, reps); break;
        case 1: launch<1>(kind, g, b, s, sp, n, newoff, op, reps); break;
        case 2: launch<2>(kind, g, b, s, sp, n, newoff, op, reps); break;
        case 5: launch<5>(kind, g, b, s, sp, n, newoff, op, reps); break;
        default: return int(hipErrorInvalidValue);
    }
    return int(hipGetLastError());
}
