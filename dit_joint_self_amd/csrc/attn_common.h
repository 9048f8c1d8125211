// attn_common.h - pieces shared by the bf16 and fp8 attention kernels:
// workgroup shape, launch plan, key-range partial format, XCD-aware workgroup
// order, direct-to-LDS copies and the half-wave reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "tile_layout.h"

namespace dit {

constexpr int NW = 8;                 // waves per workgroup (two per SIMD)
constexpr int QB = 1;                 // 32-query blocks per wave
constexpr int BM = NW * 32 * QB;      // queries per workgroup
constexpr int MI355X_CUS = 256;       // workgroups resident at once (one per CU)
constexpr float LN2 = 0.693147180559945309f;

typedef float f32x16 __attribute__((ext_vector_type(16)));   // one 32x32 MFMA accumulator

// Materialise an accumulator here, with every lane active.  An MFMA reads its
// operands from all 64 lanes; if the compiler sank the last products into a
// branch taken by only some lanes (the store guard row < S of the epilogue),
// the inactive lanes' operand rows would be lost.  The empty volatile asm
// reads and writes the value, so every product feeding it stays before it.
__device__ __forceinline__ void settle(f32x16& x) { asm volatile("" : "+v"(x)); }

// Longest sequence the kernels accept: keeps every byte offset inside one
// (batch, head) slice of prepared tiles below 2^31.
constexpr int MAX_SEQ = 1 << 21;
static_assert((int64_t)((MAX_SEQ + KV_TILE - 1) / KV_TILE) * TILE_BYTES < (int64_t)1 << 31, "slice offsets fit");

// Partial results of one key-range workgroup: O (unnormalised, fp32, row-major
// [BM][128]), then the offset m (base 2) and the weight sum l of each row.
constexpr int PART_FLOATS = BM * HEAD_DIM + 2 * BM;

// Workgroup x of a launch -> logical index.  Workgroups are dispatched
// round-robin over the 8 XCDs; give each XCD a contiguous range of logical
// indices so the workgroups sharing an XCD's L2 stream the same head's K/V.
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

// How one call is laid out over the GPU: `full` items run whole-key-range
// workgroups in full rounds; the remaining `split` items (fewer than a round)
// run nsplit key-range workgroups each (core_split), merged afterwards.  Both kinds share
// one launch, whole-range workgroups first, so a CU that finishes its last
// whole item early takes a key-range piece instead of idling until the
// slowest workgroup of the round ends.  Depends only on the shape, so the
// workspace size is known on the host.
struct CorePlan {
    int nqt, ntiles, items, full, split, nsplit;
};

// Number of key ranges for the r leftover items: the F in [1, min(8, ntiles)]
// that minimises ceil(r F / 256) rounds of pieces of 1/F item each, plus a
// fixed cost per piece of 1/32 item (prologue, partial write, merge):
// cost(F) = ceil(r F / 256) (32 + F) / (32 F); ties go to the smaller F.
inline int core_split(int rem, int ntiles) {
    int best = 1;
    int64_t best_num = 33, best_den = 32;  // cost(1) = 1 round x 33/32
    for (int f = 2; f <= std::min(8, ntiles); ++f) {
        const int64_t rounds = ((int64_t)rem * f + MI355X_CUS - 1) / MI355X_CUS;
        const int64_t num = rounds * (32 + f), den = 32 * (int64_t)f;
        if (num * best_den < best_num * den) {
            best = f;
            best_num = num;
            best_den = den;
        }
    }
    return best;
}

inline CorePlan core_plan(int BH, int S) {
    CorePlan p;
    p.ntiles = (int)num_kv_tiles(S);
    p.nqt = (S + BM - 1) / BM;
    p.items = BH * p.nqt;
    const int rem = p.items % MI355X_CUS;
    const int f = rem ? core_split(rem, p.ntiles) : 1;
    if (rem == 0 || f < 2) {
        p.full = p.items;
        p.split = 0;
        p.nsplit = 1;
    } else {
        p.full = p.items - rem;
        p.split = rem;
        p.nsplit = f;
    }
    return p;
}

// The work of workgroup x of the combined launch.  Whole-range workgroups
// [0, full) map through xcd_remap as before; key-range pieces [full, grid)
// map through their own xcd_remap (full is a multiple of 8, so piece x - full
// sits on the same XCD as workgroup x), which spreads the pieces evenly over
// the XCDs.  Piece p covers key range p % nsplit of item full + p / nsplit,
// the order the merge reads the partials in.
struct CoreWork {
    int item, f, nsplit, piece;
    bool partial;
};

__device__ __forceinline__ CoreWork core_work(int x, int grid, int full, int nsplit) {
    CoreWork w;
    if (x < full) {
        w.item = xcd_remap(x, full);
        w.f = 0;
        w.nsplit = 1;
        w.piece = 0;
        w.partial = false;
    } else {
        const int p = xcd_remap(x - full, grid - full);
        w.item = full + p / nsplit;
        w.f = p - (p / nsplit) * nsplit;
        w.nsplit = nsplit;
        w.piece = p;
        w.partial = true;
    }
    return w;
}

inline int core_grid(const CorePlan& p) { return p.full + p.split * p.nsplit; }

inline size_t core_partial_bytes_for(const CorePlan& p) {
    return (size_t)p.split * p.nsplit * PART_FLOATS * sizeof(float);
}

hipError_t launch_merge(const float* part, void* out, float* lse, int S, int nqt, int item0, int nsplit,
                        int split_items, hipStream_t stream);

}  // namespace dit
