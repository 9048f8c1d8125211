// bf16_util.h - bf16 <-> fp32 helpers and the interleaved-pair rotation used
// by the prologues of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest, ties to even) and pack lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Unpack 8 bf16 (one 16-byte chunk, element 0 in the low half of .x) to fp32.
__device__ __forceinline__ void unpack8(uint4 w, float (&x)[8]) {
    x[0] = bf16lo(w.x); x[1] = bf16hi(w.x);
    x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
    x[4] = bf16lo(w.z); x[5] = bf16hi(w.z);
    x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
}

// RoPE on 4 interleaved pairs: (x0 + i x1) * (c + i s), in fp32, each
// product rounded before the sum: no multiply-add is fused, so the rounding
// (and the bf16 value a caller rounds it to) does not depend on which product
// the compiler would otherwise fuse in a given build.
__device__ __forceinline__ void rotate4(float (&x)[8], float4 c, float4 s) {
#pragma clang fp contract(off)
    const float cc[4] = {c.x, c.y, c.z, c.w};
    const float ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float e = x[2 * i], o = x[2 * i + 1];
        x[2 * i] = e * cc[i] - o * ss[i];
        x[2 * i + 1] = e * ss[i] + o * cc[i];
    }
}

__device__ __forceinline__ uint4 pack8(const float (&x)[8]) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

}  // namespace dit
