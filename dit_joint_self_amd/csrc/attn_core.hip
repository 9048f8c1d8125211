// attn_core.hip - non-causal joint self-attention on gfx950 matrix cores.
//
// Computes out = softmax(scale * Q' K'^T) V per (batch, head) over the whole
// joint text + latent sequence (xDiT paper, abstract: attention over the long
// token sequence is the growing cost; AMD RDNA 4 xDiT blog, Ulysses section:
// each GPU runs full-sequence attention on its heads).  The softmax is the
// streaming one of FlashAttention-2 (in the xDiT paper's reference list):
// running max and running sum per query, exact up to rounding.
//
// Work decomposition
//   * One workgroup = NW waves; wave w owns QB blocks of 32 queries, so a
//     workgroup covers BM = NW * 32 * QB consecutive queries of one head.
//   * Q prologue: each lane loads its query row's 8-dim chunks, applies RoPE
//     and the factor scale*log2(e) in fp32 and keeps them as bf16 MFMA
//     B operands for the whole kernel (Q-tile resident in VGPRs).
//   * K/V stream: 64-key tiles already rotated and laid out by
//     prepare_kv.hip, copied HBM -> LDS with global_load_lds_dwordx4 into a
//     double buffer (tile j+1 lands while tile j is consumed).
//   * S^T = K' Q'^T on v_mfma_f32_32x32x16_bf16: lane (n, hh) of the
//     accumulator owns query n and 16 keys, so a row max is in-lane max ops
//     plus one v_permlane32_swap, and the row sum stays per lane until the
//     epilogue.
//   * Online softmax in base 2 with a lazily moved offset: the offset m is
//     folded into the QK^T accumulator's initial value, the row max is only
//     taken for the first tile and when a tile's weights overflow 2^20, and
//     the row sum is accumulated from the bf16 weights with v_dot2c (see
//     attn_tile).  Weights stay <= 2^20, so fp32 and bf16 hold them with
//     their usual relative precision, and the final O / l is unchanged.
//   * O^T += V^T P^T on the same MFMA: P leaves the S accumulator already in
//     B-operand layout (see tile_layout.h), V^T comes from LDS.
//   * Epilogue: combine the two half-wave partial sums, scale by 1/l, round to
//     bf16, store rows < S.
//
// Roofline: MFMA bound.  Algorithmic work per (query block of BM rows, head):
// 4 * BM * S * 128 flop; per call 4 * B * H * S^2 * 128 flop.

#include <hip/hip_runtime.h>

#include "bf16_util.h"
#include "tile_layout.h"

namespace dit {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

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

// Copy `chunks` 16-byte chunks (a multiple of 64) HBM -> LDS: wave w copies
// the 1 KiB pieces w, w + NW, ...; each lane moves 16 bytes per piece.
template <int NW, int CHUNKS>
__device__ __forceinline__ void copy_to_lds_async(const uint4* __restrict__ src, uint4* lds_dst, int wave,
                                                  int lane) {
    static_assert(CHUNKS % 64 == 0, "whole 1 KiB pieces");
#pragma unroll
    for (int i = 0; i < (CHUNKS / 64 + NW - 1) / NW; ++i) {
        const int piece = i * NW + wave;
        if (piece < CHUNKS / 64) {
            __builtin_amdgcn_global_load_lds(
                (const void*)(src + piece * 64 + lane),
                (__attribute__((address_space(3))) void*)(lds_dst + piece * 64), 16, 0, 0);
        }
    }
}

template <int NW>
__device__ __forceinline__ void load_tile_async(const uint4* __restrict__ src, uint4* lds_dst,
                                                int wave, int lane) {
    copy_to_lds_async<NW, TILE_CHUNKS>(src, lds_dst, wave, lane);
}

// exp2 of one accumulator's 16 scores, rounded to bf16 as two PV B operands;
// the rounded values are also summed (v_dot2c_f32_bf16 against (1, 1)), so
// the row sum is the sum of exactly the weights the PV product uses.
__device__ __forceinline__ void exp_pack16(const f32x16& sc, bf16x8 (&pf)[2], float& sum) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = pack_bf16x2(__builtin_amdgcn_exp2f(sc[8 * t2 + 2 * i]),
                               __builtin_amdgcn_exp2f(sc[8 * t2 + 2 * i + 1]));
            sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[i]), ones, sum, false);
        }
        pf[t2] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// One 64-key tile: S^T = K' Q'^T, online softmax, O^T += V^T P^T.  `kt` is the
// tile's LDS image (K part then V^T part), `j` its index.
//
// Softmax bookkeeping (base 2, per query): m is the offset subtracted before
// exp2 and l the running sum of the bf16 weights.  negm holds -m in all 16
// registers of the lane's accumulator shape and enters as the C operand of the
// first QK^T MFMA, so the scores arrive already offset.  m is exact (the row
// max) after tile 0; afterwards it is only raised when a tile's weights sum past
// SUM_LIMIT in some lane (so no weight exceeds 2^20): then the tile's row max is
// taken, O and l are scaled by 2^(m_old - m_new) and the tile is redone.  The
// final O / l does not depend on when m moves.
constexpr float SUM_LIMIT = 1048576.0f;  // 2^20

template <int QB, bool MASKED>
__device__ __forceinline__ void attn_tile(const uint4* kt, int j, int S, int n, int hh,
                                          const bf16x8 (&qf)[QB][8], f32x16 (&o)[QB][4],
                                          f32x16 (&negm)[QB], float (&lsum)[QB]) {
    const uint4* vt = kt + K_PART_CHUNKS;

    // ---- S'^T = K' Q'^T - m for 64 keys x (32 * QB) queries: 16 MFMA steps
    // i = (dim step t = i / 2, key block kb = i % 2).  K operands rotate
    // through a 3-slot ring read two steps ahead; the scheduling fences keep
    // the compiler from sinking the reads back to their use.
    f32x16 s[QB][2];
    {
        bf16x8 ring[3];
        ring[0] = as_bf16x8(kt[k_chunk(n, hh)]);
        ring[1] = as_bf16x8(kt[k_chunk(32 + n, hh)]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 2 < 16) {
                const int t2 = (i + 2) >> 1, kb2 = (i + 2) & 1;
                ring[(i + 2) % 3] = as_bf16x8(kt[k_chunk(kb2 * 32 + n, 2 * t2 + hh)]);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int t = i >> 1, kb = i & 1;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % 3], qf[qb][t],
                                                                    t == 0 ? negm[qb] : s[qb][kb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- keys past S (last tile only): lane half hh, register r of key
    // block kb holds key 32 kb + 16 (r >> 3) + 8 hh + (r & 7).
    if (MASKED) {
        const int base = j * KV_TILE + 8 * hh;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (base + 32 * kb + 16 * (r >> 3) + (r & 7) >= S) s[qb][kb][r] = -INFINITY;
    }

    // ---- weights P = 2^(S'), bf16 B operands, row sums.
    bf16x8 pf[QB][2][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float t0 = 0.0f, t1 = 0.0f;
        bool slow = (j == 0);
        if (!slow) {
            exp_pack16(s[qb][0], pf[qb][0], t0);
            exp_pack16(s[qb][1], pf[qb][1], t1);
            slow = __builtin_amdgcn_ballot_w64(!(t0 + t1 <= SUM_LIMIT)) != 0;
        }
        if (slow) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][1][r]);
            mx = swap_halves_max(mx);
            const float shift = (j == 0) ? mx : fmaxf(mx, 0.0f);
            if (j > 0) {
                const float alpha = __builtin_amdgcn_exp2f(-shift);
                lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
            }
            s[qb][0] -= shift;
            s[qb][1] -= shift;
            negm[qb] -= shift;
            t0 = t1 = 0.0f;
            exp_pack16(s[qb][0], pf[qb][0], t0);
            exp_pack16(s[qb][1], pf[qb][1], t1);
        }
        lsum[qb] += t0 + t1;
    }

    // ---- O^T += V^T P^T: 128 dims x (32 * QB) queries, 64 keys: 16 MFMA
    // steps i = (16-key step u = i / 4, dim block db = i % 4), V^T operands
    // through the same kind of ring.
    {
        bf16x8 ring[3];
        ring[0] = as_bf16x8(vt[v_chunk(n, hh)]);
        ring[1] = as_bf16x8(vt[v_chunk(32 + n, hh)]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + 2 < 16) {
                const int u2 = (i + 2) >> 2, db2 = (i + 2) & 3;
                ring[(i + 2) % 3] = as_bf16x8(vt[v_chunk(db2 * 32 + n, 2 * u2 + hh)]);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int u = i >> 2, db = i & 3;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % 3], pf[qb][u >> 1][u & 1], o[qb][db],
                                                                    0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int NW, int QB>
__global__ __launch_bounds__(NW * 64) void attn_core_kernel(
    const uint4* __restrict__ q, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint4* __restrict__ ws, uint2* __restrict__ out, int S, int ntiles, int nqt,
    int total_wg, float qmul, int has_rope) {
    constexpr int BM = NW * 32 * QB;
    __shared__ uint4 lds0[TILE_CHUNKS];
    __shared__ uint4 lds1[TILE_CHUNKS];

    // Workgroups are dispatched round-robin over the 8 XCDs.  Give each XCD a
    // contiguous range of (head, query-tile) items so the workgroups sharing
    // an XCD's L2 stream the same head's K/V at the same time.
    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int per = total_wg >> 3, rem = total_wg & 7;
    const int item = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    const int64_t bh = item / nqt;
    const int qt = item - (int)bh * nqt;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const uint4* src = ws + bh * (int64_t)ntiles * TILE_CHUNKS;
    load_tile_async<NW>(src, lds0, wave, lane);

    // ---- Q prologue: RoPE, fold scale*log2(e), round to bf16, keep resident.
    bf16x8 qf[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qt * BM + (wave * QB + qb) * 32 + n;
        const bool ok = row < S;
        const uint4* qrow = q + (bh * S + row) * 16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = 2 * t + hh;
            float f[8];
            uint4 w = make_uint4(0, 0, 0, 0);
            if (ok) w = qrow[c];
            unpack8(w, f);
            if (has_rope && ok) rotate4(f, cos_t[(int64_t)row * 16 + c], sin_t[(int64_t)row * 16 + c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= qmul;
            qf[qb][t] = as_bf16x8(pack8(f));
        }
    }

    f32x16 o[QB][4], negm[QB];
    float lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        negm[qb] = f32x16{};
        lsum[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
    }

    // Two distinct LDS buffers and a loop unrolled by two: the tile being read
    // and the tile in flight are different objects, so the compiler does not
    // make the reads wait for the prefetch.  Tiles 0 .. ntiles-2 take the
    // unmasked path; the last tile always takes the masked one (a no-op mask
    // when S is a multiple of the tile).
    const int nfull = ntiles - 1;
    int j = 0;
    for (; j + 2 <= nfull; j += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 1) * TILE_CHUNKS, lds1, wave, lane);
        attn_tile<QB, false>(lds0, j, S, n, hh, qf, o, negm, lsum);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 2) * TILE_CHUNKS, lds0, wave, lane);
        attn_tile<QB, false>(lds1, j + 1, S, n, hh, qf, o, negm, lsum);
    }
    if (j < nfull) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 1) * TILE_CHUNKS, lds1, wave, lane);
        attn_tile<QB, false>(lds0, j, S, n, hh, qf, o, negm, lsum);
        ++j;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    attn_tile<QB, true>((j & 1) ? lds1 : lds0, j, S, n, hh, qf, o, negm, lsum);

    // ---- epilogue: lane (n, hh), register r of dim block db holds dim
    // 32 db + 8 (r >> 2) + 4 hh + (r & 3) of query n.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float inv = 1.0f / swap_halves_sum(lsum[qb]);
        const int row = qt * BM + (wave * QB + qb) * 32 + n;
        if (row < S) {
            uint2* orow = out + (bh * S + row) * 32;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16& acc = o[qb][db];
                    orow[db * 8 + g * 2 + hh] =
                        make_uint2(pack_bf16x2(acc[4 * g + 0] * inv, acc[4 * g + 1] * inv),
                                   pack_bf16x2(acc[4 * g + 2] * inv, acc[4 * g + 3] * inv));
                }
        }
    }
}

// ===========================================================================
// Software-pipelined kernel: 4 waves x 64 queries (BM = 256), one wave per
// SIMD.  Each K/V operand read from LDS feeds two MFMAs (two 32-query blocks),
// halving LDS traffic per flop against the 32-query-per-wave kernel above.
// With no second wave on the SIMD to hide latency, the wave overlaps its own
// work in 32-key steps: step u runs the softmax of step u (VALU) interleaved
// with S^T = K' Q'^T of step u+1 (MFMA), then O^T += V^T P^T of step u.  The
// 64-key tiles stream through a ring of three LDS buffers, each tile loaded a
// full tile-iteration before its first use.
// ===========================================================================

// Keep a value in the accumulation register file: the resident Q operands
// live in AGPRs (MFMA reads its A/B operands from either file), which leaves
// the architectural VGPRs to the scores, weights and softmax state.
__device__ __forceinline__ bf16x8 pin_to_agpr(bf16x8 v) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4 w = __builtin_bit_cast(i32x4, v);
    asm volatile("" : "=a"(w) : "0"(w));
    return __builtin_bit_cast(bf16x8, w);
}

constexpr int PL_NW = 4;
constexpr int PL_QB = 2;
// Per-lane, per-step weight sum beyond which the pass is redone with the
// exact row max (each weight is then <= 2^40, l <= 2^57, far from overflow).
constexpr float PL_SUM_LIMIT = 1099511627776.0f;  // 2^40
constexpr int PL_BM = PL_NW * 32 * PL_QB;

// Copy one tile HBM -> LDS: its K part to `kdst`, its V part to `vdst`.
__device__ __forceinline__ void pl_load_tile(const uint4* __restrict__ src, uint4* kdst, uint4* vdst, int wave,
                                             int lane) {
    copy_to_lds_async<PL_NW, K_PART_CHUNKS>(src, kdst, wave, lane);
    copy_to_lds_async<PL_NW, V_PART_CHUNKS>(src + K_PART_CHUNKS, vdst, wave, lane);
}

// Scores of key half `kb` (32 keys) of the tile at `kt`: 16 MFMAs, C starts
// at -m.  Eight K reads, each feeding the two query blocks.
__device__ __forceinline__ void pl_qk(const uint4* kt, int kb, int n, int hh, const bf16x8 (&qf)[PL_QB][8],
                                      const f32x16 (&negm)[PL_QB], f32x16 (&sn)[PL_QB]) {
    bf16x8 a[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) a[t] = as_bf16x8(kt[k_chunk(kb * 32 + n, 2 * t + hh)]);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int qb = 0; qb < PL_QB; ++qb)
            sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t], qf[qb][t], t == 0 ? negm[qb] : sn[qb], 0, 0, 0);
}

// O^T += V^T P^T over key half `kb` of the tile whose V part is at `vt`: 16 MFMAs.
__device__ __forceinline__ void pl_pv(const uint4* vt, int kb, int n, int hh, const bf16x8 (&pf)[PL_QB][2],
                                      f32x16 (&o)[PL_QB][4]) {
    bf16x8 a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int t2 = i >> 2, db = i & 3;
        a[i] = as_bf16x8(vt[v_chunk(db * 32 + n, 4 * kb + 2 * t2 + hh)]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int qb = 0; qb < PL_QB; ++qb)
            o[qb][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], pf[qb][i >> 2], o[qb][i & 3], 0, 0, 0);
    // Two reads ahead; then two MFMAs per read.
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
        if (i + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
}

__device__ __forceinline__ void pl_weights(const f32x16 (&sc)[PL_QB], bf16x8 (&pf)[PL_QB][2], float (&tsum)[PL_QB]) {
#pragma unroll
    for (int qb = 0; qb < PL_QB; ++qb) {
        tsum[qb] = 0.0f;
        exp_pack16(sc[qb], pf[qb], tsum[qb]);
    }
}

__device__ __forceinline__ float pl_rowmax(const f32x16& sc) {
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    return swap_halves_max(mx);
}

__device__ __forceinline__ void pl_mask(f32x16 (&sc)[PL_QB], int key0, int S, int hh) {
    const int base = key0 + 8 * hh;
#pragma unroll
    for (int qb = 0; qb < PL_QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (base + 16 * (r >> 3) + (r & 7) >= S) sc[qb][r] = -INFINITY;
}

// One 32-key step: weights of `sc` interleaved with the scores `sn` of the
// next step (K part `knext`, key half kbn), then PV of this step (V part
// `vcur`, key half kb).  With DO_NEXT = false the next scores are not computed.  A
// lane whose step weights sum past PL_SUM_LIMIT (or are not finite) sets the
// wave's overflow mask `ovf`.
template <bool DO_NEXT>
__device__ __forceinline__ void pl_step(const uint4* vcur, int kb, const uint4* knext, int kbn, int n, int hh,
                                        const bf16x8 (&qf)[PL_QB][8], const f32x16 (&negm)[PL_QB],
                                        f32x16 (&sc)[PL_QB], f32x16 (&sn)[PL_QB], f32x16 (&o)[PL_QB][4],
                                        float (&lsum)[PL_QB], uint64_t& ovf) {
    bf16x8 pf[PL_QB][2];
    float tsum[PL_QB];
    if (DO_NEXT) pl_qk(knext, kbn, n, hh, qf, negm, sn);
    pl_weights(sc, pf, tsum);
    if (DO_NEXT) {
        // Two K reads ahead; then per read two MFMAs, each followed by four
        // VALU slots (32 exp, 16 packs, 16 dot2 over the step), and the next read.
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            if (t + 2 < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    ovf |= __builtin_amdgcn_ballot_w64(!(tsum[0] <= PL_SUM_LIMIT) || !(tsum[1] <= PL_SUM_LIMIT));
    lsum[0] += tsum[0];
    lsum[1] += tsum[1];
    pl_pv(vcur, kb, n, hh, pf, o);
}

// Tile-iteration j (not the last): wait for tile j+1, prefetch tile j+2, then
// step 2j (weights of sa || scores of tile j keys 32..63 into sb, PV tile j
// keys 0..31) and step 2j+1 (weights of sb || scores of tile j+1 keys 0..31
// into sa, PV tile j keys 32..63).  kc/vc: tile j; kn: K part of tile j+1;
// kl/vl: where tile j+2 goes.
__device__ __forceinline__ void pl_tile(int j, int L, const uint4* src, const uint4* kc, const uint4* vc,
                                        const uint4* kn, uint4* kl, uint4* vl, int wave, int lane, int n, int hh,
                                        const bf16x8 (&qf)[PL_QB][8], const f32x16 (&negm)[PL_QB],
                                        f32x16 (&sa)[PL_QB], f32x16 (&sb)[PL_QB], f32x16 (&o)[PL_QB][4],
                                        float (&lsum)[PL_QB], uint64_t& ovf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (j + 2 <= L) pl_load_tile(src + (int64_t)(j + 2) * TILE_CHUNKS, kl, vl, wave, lane);
    pl_step<true>(vc, 0, kc, 1, n, hh, qf, negm, sa, sb, o, lsum, ovf);
    pl_step<true>(vc, 1, kn, 0, n, hh, qf, negm, sb, sa, o, lsum, ovf);
}

// Exact row max of the scaled scores over all keys (for the rare second
// attempt): stream every tile's K part through k0/k1 and take QK^T maxima.
__device__ __forceinline__ void pl_exact_rowmax(const uint4* src, int L, int S, uint4* k0, uint4* k1, int wave,
                                                int lane, int n, int hh, const bf16x8 (&qf)[PL_QB][8],
                                                float (&mrow)[PL_QB]) {
    const f32x16 zero[PL_QB] = {f32x16{}, f32x16{}};
    mrow[0] = mrow[1] = -INFINITY;
    for (int j = 0; j <= L; ++j) {
        uint4* kt = (j & 1) ? k1 : k0;
        __syncthreads();
        copy_to_lds_async<PL_NW, K_PART_CHUNKS>(src + (int64_t)j * TILE_CHUNKS, kt, wave, lane);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x16 sc[PL_QB];
            pl_qk(kt, kb, n, hh, qf, zero, sc);
            pl_mask(sc, j * KV_TILE + 32 * kb, S, hh);
#pragma unroll
            for (int qb = 0; qb < PL_QB; ++qb) mrow[qb] = fmaxf(mrow[qb], pl_rowmax(sc[qb]));
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(PL_NW * 64) void attn_fwd_pipelined_kernel(
    const uint4* __restrict__ q, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint4* __restrict__ ws, uint2* __restrict__ out, int S, int ntiles, int nqt, int total_wg, float qmul,
    int has_rope) {
    // Ring of three tiles; K parts and V parts in separate regions so that
    // every operand address is one per-lane base plus an offset below 64 KiB.
    __shared__ uint4 kb0[K_PART_CHUNKS];
    __shared__ uint4 kb1[K_PART_CHUNKS];
    __shared__ uint4 kb2[K_PART_CHUNKS];
    __shared__ uint4 vb0[V_PART_CHUNKS];
    __shared__ uint4 vb1[V_PART_CHUNKS];
    __shared__ uint4 vb2[V_PART_CHUNKS];

    const int x = blockIdx.x;
    const int xcd = x & 7, slot = x >> 3;
    const int per = total_wg >> 3, rem = total_wg & 7;
    const int item = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
    const int64_t bh = item / nqt;
    const int qt = item - (int)bh * nqt;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int L = ntiles - 1;

    const uint4* src = ws + bh * (int64_t)ntiles * TILE_CHUNKS;
    pl_load_tile(src, kb0, vb0, wave, lane);
    if (L >= 1) pl_load_tile(src + TILE_CHUNKS, kb1, vb1, wave, lane);

    // ---- Q prologue: RoPE, fold scale*log2(e), round to bf16, keep resident.
    bf16x8 qf[PL_QB][8];
#pragma unroll
    for (int qb = 0; qb < PL_QB; ++qb) {
        const int row = qt * PL_BM + (wave * PL_QB + qb) * 32 + n;
        const bool ok = row < S;
        const uint4* qrow = q + (bh * S + row) * 16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int c = 2 * t + hh;
            float f[8];
            uint4 w = make_uint4(0, 0, 0, 0);
            if (ok) w = qrow[c];
            unpack8(w, f);
            if (has_rope && ok) rotate4(f, cos_t[(int64_t)row * 16 + c], sin_t[(int64_t)row * 16 + c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] *= qmul;
            qf[qb][t] = pin_to_agpr(as_bf16x8(pack8(f)));
        }
    }

    // Softmax offset m (base 2) per query, fixed for a whole pass: the exact
    // row max of the first 32 keys.  If any weight of a later step exceeds
    // 2^40 relative to it, the workgroup redoes the pass with the exact row max
    // over all keys (second attempt), where no weight exceeds 1.
    f32x16 o[PL_QB][4], negm[PL_QB], sa[PL_QB], sb[PL_QB];
    float lsum[PL_QB];
    float mrow[PL_QB] = {0.0f, 0.0f};
    for (int attempt = 0;; ++attempt) {
#pragma unroll
        for (int qb = 0; qb < PL_QB; ++qb) {
            negm[qb] = f32x16{} - mrow[qb];
            lsum[qb] = 0.0f;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
        }
        uint64_t ovf = 0;
        if (attempt > 0) {
            pl_load_tile(src, kb0, vb0, wave, lane);
            if (L >= 1) pl_load_tile(src + TILE_CHUNKS, kb1, vb1, wave, lane);
        }

        // ---- first step's scores (tile 0, keys 0..31).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        pl_qk(kb0, 0, n, hh, qf, negm, sa);
        if (S < 32) pl_mask(sa, 0, S, hh);
        if (attempt == 0) {
#pragma unroll
            for (int qb = 0; qb < PL_QB; ++qb) {
                const float mx = pl_rowmax(sa[qb]);
                sa[qb] -= mx;
                negm[qb] -= mx;
            }
        }

        // ---- tile-iterations 0 .. L-1, three per trip so each LDS buffer is a
        // fixed object in each copy (tile j lives in buffer j mod 3).
        int j = 0;
        for (; j + 3 <= L; j += 3) {
            pl_tile(j, L, src, kb0, vb0, kb1, kb2, vb2, wave, lane, n, hh, qf, negm, sa, sb, o, lsum, ovf);
            pl_tile(j + 1, L, src, kb1, vb1, kb2, kb0, vb0, wave, lane, n, hh, qf, negm, sa, sb, o, lsum, ovf);
            pl_tile(j + 2, L, src, kb2, vb2, kb0, kb1, vb1, wave, lane, n, hh, qf, negm, sa, sb, o, lsum, ovf);
        }
        if (j < L) {
            pl_tile(j, L, src, kb0, vb0, kb1, kb2, vb2, wave, lane, n, hh, qf, negm, sa, sb, o, lsum, ovf);
            ++j;
            if (j < L) {
                pl_tile(j, L, src, kb1, vb1, kb2, kb0, vb0, wave, lane, n, hh, qf, negm, sa, sb, o, lsum, ovf);
                ++j;
            }
        }

        // ---- last tile L (keys past S masked): step 2L (scores in sa) and 2L+1.
        {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int r3 = L % 3;
            const uint4* kc = r3 == 0 ? kb0 : (r3 == 1 ? kb1 : kb2);
            const uint4* vc = r3 == 0 ? vb0 : (r3 == 1 ? vb1 : vb2);
            const bool ragged = (S & (KV_TILE - 1)) != 0;
            if (ragged) pl_mask(sa, L * KV_TILE, S, hh);
            if (L * KV_TILE + 32 < S) {
                pl_step<true>(vc, 0, kc, 1, n, hh, qf, negm, sa, sb, o, lsum, ovf);
                if (ragged) pl_mask(sb, L * KV_TILE + 32, S, hh);
                pl_step<false>(vc, 1, kc, 0, n, hh, qf, negm, sb, sa, o, lsum, ovf);
            } else {
                pl_step<false>(vc, 0, kc, 1, n, hh, qf, negm, sa, sb, o, lsum, ovf);
            }
        }

        // Attempt 1 uses the exact maxima; it is final whatever its flags say
        // (non-finite inputs propagate to the output).
        if (!__syncthreads_or(ovf != 0) || attempt > 0) break;
        pl_exact_rowmax(src, L, S, kb0, kb1, wave, lane, n, hh, qf, mrow);
    }

    // ---- epilogue: lane (n, hh), register r of dim block db holds dim
    // 32 db + 8 (r >> 2) + 4 hh + (r & 3) of query n of block qb.
#pragma unroll
    for (int qb = 0; qb < PL_QB; ++qb) {
        const float inv = 1.0f / swap_halves_sum(lsum[qb]);
        const int row = qt * PL_BM + (wave * PL_QB + qb) * 32 + n;
        if (row < S) {
            uint2* orow = out + (bh * S + row) * 32;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16& acc = o[qb][db];
                    orow[db * 8 + g * 2 + hh] =
                        make_uint2(pack_bf16x2(acc[4 * g + 0] * inv, acc[4 * g + 1] * inv),
                                   pack_bf16x2(acc[4 * g + 2] * inv, acc[4 * g + 3] * inv));
                }
        }
    }
}

// Tile configurations (waves per workgroup, 32-query blocks per wave).
struct CoreConfig {
    int nw, qb;
};

static int core_variant() {
    static int v = -1;
    if (v < 0) {
        const char* e = getenv("DIT_ATTN_CORE_VARIANT");
        v = e ? atoi(e) : 0;
        if (v < 0 || v > 2) v = 0;
    }
    return v;
}

int core_block_m() { return core_variant() == 1 ? 4 * 32 : 8 * 32; }  // both variants 1 and 2: see launchers

template <int NW, int QB>
static hipError_t launch_core_t(const void* q, const float* cos_t, const float* sin_t, const void* ws,
                                void* out, int BH, int S, float qmul, hipStream_t stream) {
    constexpr int BM = NW * 32 * QB;
    const int ntiles = (int)num_kv_tiles(S);
    const int nqt = (S + BM - 1) / BM;
    const int total = BH * nqt;
    attn_core_kernel<NW, QB><<<total, NW * 64, 0, stream>>>(
        static_cast<const uint4*>(q), reinterpret_cast<const float4*>(cos_t),
        reinterpret_cast<const float4*>(sin_t), static_cast<const uint4*>(ws), static_cast<uint2*>(out),
        S, ntiles, nqt, total, qmul, cos_t != nullptr);
    return hipGetLastError();
}

static hipError_t launch_pipelined(const void* q, const float* cos_t, const float* sin_t, const void* ws,
                                   void* out, int BH, int S, float qmul, hipStream_t stream) {
    const int ntiles = (int)num_kv_tiles(S);
    const int nqt = (S + PL_BM - 1) / PL_BM;
    const int total = BH * nqt;
    attn_fwd_pipelined_kernel<<<total, PL_NW * 64, 0, stream>>>(
        static_cast<const uint4*>(q), reinterpret_cast<const float4*>(cos_t),
        reinterpret_cast<const float4*>(sin_t), static_cast<const uint4*>(ws), static_cast<uint2*>(out),
        S, ntiles, nqt, total, qmul, cos_t != nullptr);
    return hipGetLastError();
}

hipError_t launch_attn_core(const void* q, const float* cos_t, const float* sin_t, const void* ws,
                            void* out, int BH, int S, float qmul, hipStream_t stream) {
    if (core_variant() == 2) return launch_pipelined(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
    if (core_variant() == 1) return launch_core_t<4, 1>(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
    return launch_core_t<8, 1>(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
}

}  // namespace dit
