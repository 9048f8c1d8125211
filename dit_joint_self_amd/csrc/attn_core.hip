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

#include "attn_common.h"
#include "bf16_util.h"
#include "tile_layout.h"

namespace dit {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

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

// MFMA operand ring: LDS reads run RING - 1 MFMA steps ahead of their use.
constexpr int RING = 4;

template <int QB, bool MASKED>
__device__ __forceinline__ void attn_tile(const uint4* kt, int j, bool first, int S, int n, int hh,
                                          const bf16x8 (&qf)[QB][8], f32x16 (&o)[QB][4],
                                          f32x16 (&negm)[QB], float (&lsum)[QB]) {
    const uint4* vt = kt + K_PART_CHUNKS;

    // ---- S'^T = K' Q'^T - m for 64 keys x (32 * QB) queries: 16 MFMA steps
    // i = (dim step t = i / 2, key block kb = i % 2).  K operands rotate
    // through a ring read RING - 1 steps ahead; the scheduling fences keep the
    // compiler from sinking the reads back to their use.
    f32x16 s[QB][2];
    {
        bf16x8 ring[RING];
#pragma unroll
        for (int i0 = 0; i0 < RING - 1; ++i0)
            ring[i0] = as_bf16x8(kt[k_chunk((i0 & 1) * 32 + n, 2 * (i0 >> 1) + hh)]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + RING - 1 < 16) {
                const int t2 = (i + RING - 1) >> 1, kb2 = (i + RING - 1) & 1;
                ring[(i + RING - 1) % RING] = as_bf16x8(kt[k_chunk(kb2 * 32 + n, 2 * t2 + hh)]);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int t = i >> 1, kb = i & 1;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % RING], qf[qb][t],
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
        bool slow = first;
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
            const float shift = first ? mx : fmaxf(mx, 0.0f);
            if (!first) {
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
        bf16x8 ring[RING];
#pragma unroll
        for (int i0 = 0; i0 < RING - 1; ++i0)
            ring[i0] = as_bf16x8(vt[v_chunk((i0 & 3) * 32 + n, 2 * (i0 >> 2) + hh)]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + RING - 1 < 16) {
                const int u2 = (i + RING - 1) >> 2, db2 = (i + RING - 1) & 3;
                ring[(i + RING - 1) % RING] = as_bf16x8(vt[v_chunk(db2 * 32 + n, 2 * u2 + hh)]);
            }
            __builtin_amdgcn_sched_barrier(0);
            const int u = i >> 2, db = i & 3;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
                o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % RING], pf[qb][u >> 1][u & 1], o[qb][db],
                                                                    0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One workgroup = BM queries of one (batch, head) against the key tiles
// [tb, te).  Items item0 + i / nsplit, key range i % nsplit of nsplit equal
// ranges.  PARTIAL = false: the whole key range, normalised bf16 output.
// PARTIAL = true: unnormalised O, m and l of the range to `part`.
template <bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void attn_core_kernel(
    const uint4* __restrict__ q, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint4* __restrict__ ws, uint2* __restrict__ out, float* __restrict__ part, int S, int ntiles, int nqt,
    int item0, int nsplit, float qmul, int has_rope) {
    __shared__ uint4 lds0[TILE_CHUNKS];
    __shared__ uint4 lds1[TILE_CHUNKS];

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int item = item0 + logical / nsplit;
    const int f = logical - (logical / nsplit) * nsplit;
    const int64_t bh = item / nqt;
    const int qt = item - (int)bh * nqt;
    const int tb = (int)((int64_t)f * ntiles / nsplit);
    const int te = (int)((int64_t)(f + 1) * ntiles / nsplit);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const uint4* src = ws + bh * (int64_t)ntiles * TILE_CHUNKS;
    load_tile_async<NW>(src + (int64_t)tb * TILE_CHUNKS, lds0, wave, lane);

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
            float fv[8];
            uint4 w = make_uint4(0, 0, 0, 0);
            if (ok) w = qrow[c];
            unpack8(w, fv);
            if (has_rope && ok) rotate4(fv, cos_t[(int64_t)row * 16 + c], sin_t[(int64_t)row * 16 + c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) fv[e] *= qmul;
            qf[qb][t] = as_bf16x8(pack8(fv));
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
    // make the reads wait for the prefetch.  Tiles tb .. te-2 take the
    // unmasked path; the range's last tile takes the masked one (a no-op mask
    // unless it is the sequence's ragged last tile).  Tile tb + i lives in
    // buffer i mod 2.
    const int last = te - 1;
    int j = tb;
    for (; j + 2 <= last; j += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 1) * TILE_CHUNKS, lds1, wave, lane);
        attn_tile<QB, false>(lds0, j, j == tb, S, n, hh, qf, o, negm, lsum);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 2) * TILE_CHUNKS, lds0, wave, lane);
        attn_tile<QB, false>(lds1, j + 1, false, S, n, hh, qf, o, negm, lsum);
    }
    if (j < last) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_tile_async<NW>(src + (int64_t)(j + 1) * TILE_CHUNKS, lds1, wave, lane);
        attn_tile<QB, false>(lds0, j, j == tb, S, n, hh, qf, o, negm, lsum);
        ++j;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    attn_tile<QB, true>(((j - tb) & 1) ? lds1 : lds0, j, j == tb, S, n, hh, qf, o, negm, lsum);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < 4; ++db) settle(o[qb][db]);

    // ---- epilogue: lane (n, hh), register r of dim block db holds dim
    // 32 db + 8 (r >> 2) + 4 hh + (r & 3) of query n.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = swap_halves_sum(lsum[qb]);
        const int rloc = (wave * QB + qb) * 32 + n;
        const int row = qt * BM + rloc;
        if (PARTIAL) {
            float* pw = part + (int64_t)logical * PART_FLOATS;
            float4* prow = reinterpret_cast<float4*>(pw + (int64_t)rloc * HEAD_DIM);
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x16& acc = o[qb][db];
                    prow[db * 8 + g * 2 + hh] =
                        make_float4(acc[4 * g + 0], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
                }
            if (hh == 0) {
                pw[BM * HEAD_DIM + rloc] = -negm[qb][0];
                pw[BM * HEAD_DIM + BM + rloc] = l;
            }
        } else if (row < S) {
            const float inv = 1.0f / l;
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

// Combine the nsplit key-range partials of each split item (the same streaming
// softmax merge, exact): M = max m_f, O = sum 2^(m_f - M) O_f / sum 2^(m_f - M) l_f.
// One workgroup per 16 rows of an item; 16 threads per row, 8 dims each.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part, uint4* __restrict__ out,
                                                         int S, int nqt, int item0, int nsplit) {
    const int item_local = blockIdx.x / (BM / 16);
    const int rloc = (blockIdx.x % (BM / 16)) * 16 + (threadIdx.x >> 4);
    const int seg = threadIdx.x & 15;
    const int item = item0 + item_local;
    const int64_t bh = item / nqt;
    const int row = (item - (int)bh * nqt) * BM + rloc;
    if (row >= S) return;
    const float* p0 = part + (int64_t)item_local * nsplit * PART_FLOATS;
    float M = -INFINITY;
    for (int f = 0; f < nsplit; ++f) M = fmaxf(M, p0[(int64_t)f * PART_FLOATS + BM * HEAD_DIM + rloc]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float L = 0.0f;
    for (int f = 0; f < nsplit; ++f) {
        const float* pf = p0 + (int64_t)f * PART_FLOATS;
        const float w = __builtin_amdgcn_exp2f(pf[BM * HEAD_DIM + rloc] - M);
        L += w * pf[BM * HEAD_DIM + BM + rloc];
        const float4* src = reinterpret_cast<const float4*>(pf + (int64_t)rloc * HEAD_DIM + seg * 8);
        const float4 a = src[0], b = src[1];
        acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
        acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    out[(bh * S + row) * 16 + seg] = pack8(acc);
}

hipError_t launch_merge(const float* part, void* out, int S, int nqt, int item0, int nsplit, int split_items,
                        hipStream_t stream) {
    attn_merge_kernel<<<split_items * (BM / 16), 256, 0, stream>>>(part, static_cast<uint4*>(out), S, nqt, item0,
                                                                   nsplit);
    return hipGetLastError();
}

size_t core_partial_bytes(int BH, int S) { return core_partial_bytes_for(core_plan(BH, S)); }

hipError_t launch_attn_core(const void* q, const float* cos_t, const float* sin_t, const void* ws, void* part,
                            void* out, int BH, int S, float qmul, hipStream_t stream) {
    const CorePlan p = core_plan(BH, S);
    const uint4* wsv = static_cast<const uint4*>(ws);
    const uint4* qv = static_cast<const uint4*>(q);
    const float4* cv = reinterpret_cast<const float4*>(cos_t);
    const float4* sv = reinterpret_cast<const float4*>(sin_t);
    const int rope = cos_t != nullptr;
    if (p.full > 0) {
        attn_core_kernel<false><<<p.full, NW * 64, 0, stream>>>(qv, cv, sv, wsv, static_cast<uint2*>(out), nullptr,
                                                               S, p.ntiles, p.nqt, 0, 1, qmul, rope);
    }
    if (p.split > 0) {
        float* pt = static_cast<float*>(part);
        attn_core_kernel<true><<<p.split * p.nsplit, NW * 64, 0, stream>>>(
            qv, cv, sv, wsv, nullptr, pt, S, p.ntiles, p.nqt, p.full, p.nsplit, qmul, rope);
        launch_merge(pt, out, S, p.nqt, p.full, p.nsplit, p.split, stream);
    }
    return hipGetLastError();
}

}  // namespace dit
