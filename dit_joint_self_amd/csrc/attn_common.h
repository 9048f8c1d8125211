// attn_common.h - pieces shared by the bf16 and fp8 attention kernels:
// workgroup shape, launch plan and key-range partial format (the gfx950
// helpers they build on are in gfx950.h).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "gfx950.h"
#include "tile_layout.h"

namespace dit {

constexpr int NW = 8;                 // waves per workgroup (two per SIMD)
constexpr int QB = 1;                 // 32-query blocks per wave
constexpr int BM = NW * 32 * QB;      // queries per workgroup
constexpr float LN2 = 0.693147180559945309f;

// Longest sequence the kernels accept: keeps every byte offset inside one
// (batch, head) slice of prepared tiles below 2^31.
constexpr int MAX_SEQ = 1 << 21;
static_assert((int64_t)((MAX_SEQ + KV_TILE - 1) / KV_TILE) * K_PART_BYTES < (int64_t)1 << 31, "slice offsets fit");
static_assert((int64_t)MAX_SEQ * V_ROW_BYTES < (int64_t)1 << 31, "V offsets of one head fit");

// Partial results of one key-range workgroup: O (unnormalised, fp32, row-major
// [BM][128]), then the offset m (base 2) and the weight sum l of each row.
constexpr int PART_FLOATS = BM * HEAD_DIM + 2 * BM;

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

// ---------------------------------------------------------------------------
// Run-time hand-out (bf16 launch).  The whole-range workgroups of all but the
// last round keep the static XCD-aware order above.  The rest form a pool:
// the last round of whole items (when there are at least three rounds; with
// fewer, every whole item stays static so that each XCD streams its own
// heads' K and V) and then the key-range pieces.  The launch has two pool
// workgroups per pool unit; each takes the next unit from a counter, and
// those that find none left end at once.  Workgroups are dispatched
// round-robin over the XCDs and each XCD starts its share as its CUs free
// up, so an XCD that runs ahead takes more of the pool instead of idling
// while a slower XCD works through its share.  The counters sit in a
// CORE_CTL_BYTES block at the end of the workspace: ctl[0] is the next pool
// unit, ctl[CTL_STRIDE] the number of pool workgroups that have finished; the
// last one to finish clears both, so every call leaves them at zero
// (dit_attn_prepare_k zeroes them first).
// ---------------------------------------------------------------------------
constexpr int CORE_CTL_BYTES = 256;
constexpr int CTL_STRIDE = 16;  // ints between the two counters (64 bytes)

inline int core_pieces(const CorePlan& p) { return p.split * p.nsplit; }
// Whole items in the pool (the last round when there are three or more).
inline int core_pool_whole(const CorePlan& p) { return p.full >= 3 * MI355X_CUS ? MI355X_CUS : 0; }
inline int core_pool_units(const CorePlan& p) { return core_pool_whole(p) + core_pieces(p); }
inline int core_grid_dynamic(const CorePlan& p) { return p.full - core_pool_whole(p) + 2 * core_pool_units(p); }

__device__ __forceinline__ CoreWork whole_work(int item) {
    CoreWork w;
    w.item = item;
    w.f = 0;
    w.nsplit = 1;
    w.piece = 0;
    w.partial = false;
    return w;
}

__device__ __forceinline__ CoreWork piece_work(int p, int full, int nsplit) {
    CoreWork w;
    w.item = full + p / nsplit;
    w.f = p - (p / nsplit) * nsplit;
    w.nsplit = nsplit;
    w.piece = p;
    w.partial = true;
    return w;
}

// The pool unit of this workgroup, or -1 if none is left (every thread gets
// the same value; contains a barrier).
__device__ __forceinline__ int take_unit(int* ctl, int nunits) {
    __shared__ int taken;
    if (threadIdx.x == 0)
        taken = __hip_atomic_fetch_add(ctl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int u = __builtin_amdgcn_readfirstlane(taken);
    return u < nunits ? u : -1;
}

// Called once by every pool workgroup after its last access to ctl[0].
__device__ __forceinline__ void finish_pool_wg(int* ctl, int nwg) {
    if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(ctl + CTL_STRIDE, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == nwg - 1) {
            __hip_atomic_store(ctl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctl + CTL_STRIDE, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

inline size_t core_partial_bytes_for(const CorePlan& p) {
    return (size_t)p.split * p.nsplit * PART_FLOATS * sizeof(float);
}

hipError_t launch_merge(const float* part, void* out, float* lse, int S, int nqt, int item0, int nsplit,
                        int split_items, hipStream_t stream);

}  // namespace dit
