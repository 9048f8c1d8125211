// fp8_util.h - OCP e4m3 <-> fp32 conversions on gfx950 (v_cvt_pk_f32_fp8,
// v_cvt_pk_fp8_f32: round to nearest even).  Values passed to the packing
// helpers are clamped to the finite e4m3 range [-448, 448] first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

constexpr float E4M3_MAX = 448.0f;

// Four e4m3 bytes (byte 0 = element 0) to fp32.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* f) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    f[0] = lo[0];
    f[1] = lo[1];
    f[2] = hi[0];
    f[3] = hi[1];
}

__device__ __forceinline__ float clamp_e4m3(float x) { return fminf(fmaxf(x, -E4M3_MAX), E4M3_MAX); }

// Four fp32 (already within [-448, 448]) to four e4m3 bytes.
__device__ __forceinline__ uint32_t f32x4_to_fp8(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

}  // namespace dit
