// Test-only kernel: one v_mfma_f32_32x32x16_bf16 per wave on caller-given
// fragments, so that GPU tests can pin how the matrix core rounds (sign
// symmetry of its fp32 accumulation, against the exactly rounded sum).
// Lane l of wave w reads a[(w*64 + l)*8 .. +7] and b[(w*64 + l)*8 .. +7]
// (bf16 bit patterns) and c0[(w*64 + l)*16 .. +15] and writes the 16 result
// registers to c at the same offsets.  Operand layout of the instruction:
// lane l supplies A[i = l % 32][k = 8 (l / 32) .. + 7] and
// B[k = 8 (l / 32) .. + 7][j = l % 32]; result register r of lane l is
// D[i = 8 (r / 4) + 4 (l / 32) + r % 4][j = l % 32].
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void k_mfma_probe(const uint16_t* a, const uint16_t* b, const float* c0, float* c) {
    const int64_t base = int64_t(blockIdx.x) * 64 + threadIdx.x;
    bf16x8 av, bv;
    for (int e = 0; e < 8; ++e) {
        av[e] = __builtin_bit_cast(__bf16, a[base * 8 + e]);
        bv[e] = __builtin_bit_cast(__bf16, b[base * 8 + e]);
    }
    f32x16 acc;
    for (int r = 0; r < 16; ++r) acc[r] = c0[base * 16 + r];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    for (int r = 0; r < 16; ++r) c[base * 16 + r] = acc[r];
}

// waves: independent 32x32x16 problems; all pointers are device memory with
// waves*64*8 (a, b) and waves*64*16 (c0, c) elements.  Returns a hipError_t.
extern "C" int mfma_probe_launch(const void* a, const void* b, const void* c0, void* c, int waves, void* stream) {
    if (waves < 1) return int(hipErrorInvalidValue);
    k_mfma_probe<<<dim3(waves), dim3(64), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b), static_cast<const float*>(c0),
        static_cast<float*>(c));
    return int(hipGetLastError());
}
