// clock_probe.hip - the shader clock under a matrix-core load, for pricing
// kernels against the peak at the clock the chip actually runs at (the
// published MI355X peaks assume 2.4 GHz; under sustained MFMA load the clock
// is lower).
//
// Every wave runs a long stream of independent v_mfma_f32_32x32x16_bf16 on
// register data (two waves per SIMD, every CU busy, like the attention
// kernel) and reads the shader cycle counter (s_memtime) and the constant
// rate counter (s_memrealtime) before and after.  The host divides the two
// deltas and scales by the constant counter's rate.
#include <hip/hip_runtime.h>

#include "bf16_util.h"

namespace dit {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_CHAINS = 4;

__global__ __launch_bounds__(PROBE_THREADS, 2) void clock_probe_kernel(int iters, unsigned long long* out) {
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    f32x16 acc[PROBE_CHAINS];
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c)
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(float)((threadIdx.x + e) & 7);
        b[e] = (__bf16)(float)((threadIdx.x * 3 + e) & 7);
    }
    const unsigned long long c0 = clock64();
    const unsigned long long r0 = wall_clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < PROBE_CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
    }
    float keep = 0.f;
#pragma unroll
    for (int c = 0; c < PROBE_CHAINS; ++c) keep += acc[c][threadIdx.x & 15];
    const unsigned long long c1 = clock64();
    const unsigned long long r1 = wall_clock64();
    const int wave = (blockIdx.x * PROBE_THREADS + threadIdx.x) >> 6;
    if ((threadIdx.x & 63) == 0) {
        out[3 * wave] = c1 - c0;
        out[3 * wave + 1] = r1 - r0;
        out[3 * wave + 2] = (unsigned long long)(keep != keep);  // keeps the MFMAs live; 0 for finite sums
    }
}

hipError_t launch_clock_probe(int blocks, int iters, void* out, hipStream_t stream) {
    clock_probe_kernel<<<blocks, PROBE_THREADS, 0, stream>>>(iters, static_cast<unsigned long long*>(out));
    return hipGetLastError();
}

}  // namespace dit
