// gfx950.h - small gfx950 (MI355X) helpers shared by the kernels of this
// library: the CU count, the 32x32 MFMA accumulator type, an accumulator
// fence, the XCD-aware workgroup order, buffer resources, the direct-to-LDS
// copy and the half-wave reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace dit {

constexpr int MI355X_CUS = 256;       // compute units (256 in 8 XCDs of 32)

typedef float f32x16 __attribute__((ext_vector_type(16)));   // one 32x32 MFMA accumulator

// Materialise an accumulator here, with every lane active.  An MFMA reads its
// operands from all 64 lanes; if the compiler sank the last products into a
// branch taken by only some lanes (the store guard row < S of the epilogue),
// the inactive lanes' operand rows would be lost.  The empty volatile asm
// reads and writes the value, so every product feeding it stays before it.
__device__ __forceinline__ void settle(f32x16& x) { asm volatile("" : "+v"(x)); }

// Workgroup x of a launch -> logical index.  Workgroups are dispatched
// round-robin over the 8 XCDs; give each XCD a contiguous range of logical
// indices so the workgroups sharing an XCD's L2 work on neighbouring data
// (the attention kernels: the same head's K/V).
__device__ __forceinline__ int xcd_remap(int x, int total) {
    const int xcd = x & 7, slot = x >> 3;
    const int per = total >> 3, rem = total & 7;
    return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
}

__device__ __forceinline__ float swap_halves_max(float x) {
    // v_permlane32_swap exchanges lanes 0-31 of one operand with lanes 32-63 of
    // the other; with both operands = x, the two results hold x of this lane
    // and of lane ^ 32 (in some order).
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over `bytes` bytes from `base`, raw addressing (word 3 is the
// gfx9 raw-buffer format).  Accesses at or past `bytes` read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 1 KiB piece HBM -> LDS by the buffer form of the LDS DMA
// (buffer_load_dwordx4 ... lds): lane l moves bytes [soff + 16 l, soff + 16 l + 16)
// of the resource to lds_dst + 16 l.  The buffer form is counted on VM_CNT
// only; with the global form in flight the compiler can only wait for all
// outstanding LDS reads at once, which exposes the full LDS latency each time
// an MFMA operand is needed.
__device__ __forceinline__ void lds_piece(__amdgpu_buffer_rsrc_t rsrc, int soff, uint4* lds_dst, int lane) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_dst, 16, lane * 16,
                                             soff, 0, 0);
}

// Copy CHUNKS 16-byte chunks (whole 1 KiB pieces) starting at byte soff of the
// resource to lds_dst: wave w moves pieces w, w + NW, ...
template <int NW, int CHUNKS>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, int soff, uint4* lds_dst, int wave,
                                            int lane) {
    static_assert(CHUNKS % 64 == 0, "whole 1 KiB pieces");
#pragma unroll
    for (int i = 0; i < (CHUNKS / 64 + NW - 1) / NW; ++i) {
        const int piece = i * NW + wave;
        if (piece < CHUNKS / 64) lds_piece(rsrc, soff + piece * 1024, lds_dst + piece * 64, lane);
    }
}

// Debug builds (DIT_DEBUG_LDS_NAN=1) fill a kernel's LDS buffers with all-ones
// bytes before its first copy: a NaN in bf16 (0xFFFF) and in e4m3 (0xFF), so
// any operand read from LDS that the tile copies did not write poisons the
// output.  The fill ends with a barrier; normal builds compile it away.
#ifndef DIT_DEBUG_LDS_NAN
#define DIT_DEBUG_LDS_NAN 0
#endif
template <int THREADS>
__device__ __forceinline__ void debug_fill_lds(uint4* buf, int chunks) {
    if (DIT_DEBUG_LDS_NAN) {
        for (int i = threadIdx.x; i < chunks; i += THREADS) buf[i] = make_uint4(~0u, ~0u, ~0u, ~0u);
    }
}

}  // namespace dit
