// attn_core_fp8.hip - joint self-attention with fp8 (OCP e4m3) Q/K/V and
// per-tensor scales on gfx950's v_mfma_scale_f32_32x32x64_f8f6f4.
//
// The same computation as attn_core.hip (non-causal softmax(scale q' k'^T) v
// over the whole joint sequence, RoPE on Q and K; xDiT paper abstract and the
// AMD RDNA 4 xDiT blog's fp8 attention backend), on fp8 operands:
//
//   * K' was re-quantised after RoPE by prepare_kv_fp8 (step sk, in the
//     workspace header); V keeps its codes (step v_scale).
//   * Q prologue: dequantise (x q_scale), RoPE in fp32, multiply by
//     scale*log2(e)*sk*2^-e and re-quantise, where 2^e is the power of two that
//     keeps the largest possible code within 448.  The QK^T MFMA applies 2^e
//     through its E8M0 B-operand scale, so its fp32 result is the base-2 score.
//   * Weights p' = 2^(s - m + 4) = 16 p are rounded to e4m3 for the PV MFMA;
//     m is the row max of the range's first tile and moves (with O and l
//     rescaled) only when a lane's step weights sum past 16 * 24, which keeps
//     every p' below 448.  l sums the fp32 p'; O = O_acc * v_scale / l.
//
// Work per workgroup, split plan and merge are the bf16 kernel's
// (attn_common.h), and so is the loop: K' and V^T parts in their own pairs of
// LDS buffers (K' one tile ahead), and per wave the QK^T MFMAs of tile j+1
// beside the exp2 / e4m3 packing of tile j, then O += P'V for tile j.  Per
// 64-key tile a wave issues 4 QK^T and 4 PV MFMAs of 32x32x64 (2 * 32 * 32 *
// 64 flop each).  Roofline: MFMA bound (fp8 peak); the softmax VALU work per
// MFMA is four times the bf16 kernel's.

#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "bf16_util.h"
#include "fp8_util.h"
#include "tile_layout.h"

namespace dit {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float F8_SUM_LIMIT = 384.0f;  // 16 * 24: every p' of the step is then < 448
constexpr int E8M0_ONE = 127;           // E8M0 scale code of 2^0

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0, scale_b);
}

__device__ __forceinline__ i32x8 lds_read32(const uint4* p) {
    const uint4 lo = p[0], hi = p[1];
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Weights of four scores, 4w .. 4w + 3 of the lane's 32 (key block w / 4,
// registers 4 (w % 4) ..): exp2, packed to e4m3 in the PV B-operand order
// (byte j of pf = key block j / 16, register j % 16); their fp32 sum is added
// to `sum`.  No clamp to 448: a weight above it makes the lane's sum exceed
// F8_SUM_LIMIT, and the tile is then redone with a moved offset (p' <= 16).
// cvt_pk replaces one half of its destination, so pf[w] of the previous tile
// serves as the untouched half and no register has to be cleared first.
__device__ __forceinline__ void f8_weight_quad(const f32x16 (&s)[2], int w, i32x8& pf, float& sum) {
    const f32x16& sc = s[w >> 2];
    const int r = (w & 3) * 4;
    const float a = __builtin_amdgcn_exp2f(sc[r]), b = __builtin_amdgcn_exp2f(sc[r + 1]);
    const float c = __builtin_amdgcn_exp2f(sc[r + 2]), d = __builtin_amdgcn_exp2f(sc[r + 3]);
    sum += (a + b) + (c + d);
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, pf[w], false);
    pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
}

// K' operand of QK^T step i (key block i & 1, 64-dim step i >> 1) and V^T
// operand of PV step db (32-dim block), for lane (n, hh): 32 bytes each.
__device__ __forceinline__ i32x8 f8_k_operand(const uint4* kt, int i, int n, int hh) {
    return lds_read32(kt + ((i & 1) * 32 + n) * F8_K_ROW_CHUNKS + (i >> 1) * 4 + hh * 2);
}
__device__ __forceinline__ i32x8 f8_v_operand(const uint4* vt, int db, int n, int hh) {
    return lds_read32(vt + (db * 32 + n) * F8_V_ROW_CHUNKS + hh * 2);
}

// The tile copies of one pipelined step (the K' part two tiles ahead, the V^T
// part one tile ahead), issued together at the start of the step: measured
// slightly faster than one piece per stage-A step.
struct F8TileCopies {
    static constexpr int KJ = (F8_K_PART_CHUNKS / 64 + NW - 1) / NW;  // K' pieces per wave (at most)
    static constexpr int VJ = (F8_V_PART_CHUNKS / 64 + NW - 1) / NW;  // V^T pieces per wave (at most)
    __amdgpu_buffer_rsrc_t rsrc;
    int ksoff, vsoff;
    uint4* kdst;
    uint4* vdst;
    bool kon;
    int wave, lane;
    __device__ __forceinline__ void at_step(int j) const {
        if (j < KJ) {
            const int p = j * NW + wave;
            if (kon && p < F8_K_PART_CHUNKS / 64) lds_piece(rsrc, ksoff + p * 1024, kdst + p * 64, lane);
        } else if (j < KJ + VJ) {
            const int p = (j - KJ) * NW + wave;
            if (p < F8_V_PART_CHUNKS / 64) lds_piece(rsrc, vsoff + p * 1024, vdst + p * 64, lane);
        }
    }
};

// Stage A: QK^T MFMA step i of the next tile (K' part kn) beside weight quads
// 2i, 2i + 1 of the current tile.
template <bool QK, bool EXP>
__device__ __forceinline__ void f8_stage_a(const uint4* kn, const i32x8 (&qf)[2], int qscale, const f32x16& negm,
                                           f32x16 (&sn)[2], const f32x16 (&sc)[2], i32x8& pf, float& sum, int n,
                                           int hh) {
    i32x8 a[4];
    if (QK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = f8_k_operand(kn, i, n, hh);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (QK) sn[i & 1] = mfma_f8(a[i], qf[i >> 1], (i >> 1) == 0 ? negm : sn[i & 1], qscale);
        if (EXP) {
            f8_weight_quad(sc, 2 * i, pf, sum);
            f8_weight_quad(sc, 2 * i + 1, pf, sum);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ float f8_tile_max(const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    return swap_halves_max(mx);
}

// Keys past S: lane half hh, register r of key block kb holds key
// 32 kb + 16 (r >> 3) + 8 hh + (r & 7) of tile j.
__device__ __forceinline__ void f8_mask_tail(f32x16 (&s)[2], int j, int S, int hh) {
    const int base = j * KV_TILE + 8 * hh;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (base + 32 * kb + 16 * (r >> 3) + (r & 7) >= S) s[kb][r] = -INFINITY;
}

// Between the stages: if some lane's weights sum past F8_SUM_LIMIT, move the
// offset to (row max - 4) of this tile (never down), rescale O and l, apply the
// move to the next tile's scores too and redo the weights; then add the sum.
template <bool QK>
__device__ __forceinline__ void f8_settle(f32x16 (&sc)[2], f32x16 (&sn)[2], i32x8& pf, float sum, f32x16 (&o)[4],
                                          f32x16& negm, float& lsum) {
    if (__builtin_amdgcn_ballot_w64(!(sum <= F8_SUM_LIMIT)) != 0) {
        const float shift = fmaxf(f8_tile_max(sc) - 4.0f, 0.0f);
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        sc[0] -= shift;
        sc[1] -= shift;
        negm -= shift;
        if (QK) {
            sn[0] -= shift;
            sn[1] -= shift;
        }
        sum = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) f8_weight_quad(sc, w, pf, sum);
    }
    lsum += sum;
}

// Stage B: O^T += V^T P'^T, four 32-dim blocks of 64 keys.
__device__ __forceinline__ void f8_stage_b(const uint4* vt, const i32x8& pf, f32x16 (&o)[4], int n, int hh) {
    i32x8 a[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) a[db] = f8_v_operand(vt, db, n, hh);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        __builtin_amdgcn_sched_barrier(0);
        o[db] = mfma_f8(a[db], pf, o[db], E8M0_ONE);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ void f8_tile_step(const uint4* kn, const uint4* vt, f32x16 (&sc)[2], f32x16 (&sn)[2],
                                             const i32x8 (&qf)[2], int qscale, i32x8& pf, f32x16 (&o)[4],
                                             f32x16& negm, float& lsum, int n, int hh, const F8TileCopies& cp) {
#pragma unroll
    for (int j = 0; j < F8TileCopies::KJ + F8TileCopies::VJ; ++j) cp.at_step(j);
    float sum = 0.0f;
    f8_stage_a<true, true>(kn, qf, qscale, negm, sn, sc, pf, sum, n, hh);
    f8_settle<true>(sc, sn, pf, sum, o, negm, lsum);
    f8_stage_b(vt, pf, o, n, hh);
}

__device__ __forceinline__ void f8_tile_step_last(const uint4* vt, f32x16 (&sc)[2], int j, int S,
                                                  const i32x8 (&qf)[2], int qscale, i32x8& pf, f32x16 (&o)[4],
                                                  f32x16& negm, float& lsum, int n, int hh) {
    f8_mask_tail(sc, j, S, hh);
    float sum = 0.0f;
    f32x16 none[2];
    f8_stage_a<false, true>(nullptr, qf, qscale, negm, none, sc, pf, sum, n, hh);
    f8_settle<false>(sc, none, pf, sum, o, negm, lsum);
    f8_stage_b(vt, pf, o, n, hh);
}

template <bool PARTIAL>
__global__ __launch_bounds__(NW * 64) void attn_core_fp8_kernel(
    const uint4* __restrict__ q, float q_scale, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint8_t* __restrict__ ws, uint2* __restrict__ out, float* __restrict__ part, int S, int ntiles, int nqt,
    int item0, int nsplit, float qmul, int has_rope) {
    // K' parts run one tile ahead of V^T parts, each through its own pair of
    // buffers (as in the bf16 kernel): distinct objects and a loop unrolled by
    // two keep every buffer static.
    __shared__ uint4 kb0[F8_K_PART_CHUNKS];
    __shared__ uint4 kb1[F8_K_PART_CHUNKS];
    __shared__ uint4 vb0[F8_V_PART_CHUNKS];
    __shared__ uint4 vb1[F8_V_PART_CHUNKS];

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int item = item0 + logical / nsplit;
    const int f = logical - (logical / nsplit) * nsplit;
    const int64_t bh = item / nqt;
    const int qt = item - (int)bh * nqt;
    const int tb = (int)((int64_t)f * ntiles / nsplit);
    const int te = (int)((int64_t)(f + 1) * ntiles / nsplit);
    const int nt = te - tb;  // >= 1

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 31;
    const int hh = lane >> 5;

    const float sk = reinterpret_cast<const float*>(ws)[0];
    const float sv = reinterpret_cast<const float*>(ws)[1];
    // The (batch, head) slice of tiles as a buffer resource (byte offsets < 2^31 for S <= MAX_SEQ).
    const __amdgpu_buffer_rsrc_t rsrc =
        raw_rsrc(ws + F8_HEADER_BYTES + bh * (int64_t)ntiles * F8_TILE_BYTES, (uint32_t)ntiles * F8_TILE_BYTES);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int tile0 = tb * F8_TILE_BYTES;
    auto copies = [&](int ki, uint4* kd, bool kon, int vi, uint4* vd) {
        F8TileCopies c;
        c.rsrc = rsrc;
        c.ksoff = tile0 + ki * F8_TILE_BYTES;
        c.vsoff = tile0 + vi * F8_TILE_BYTES + F8_K_PART_CHUNKS * 16;
        c.kdst = kd;
        c.vdst = vd;
        c.kon = kon;
        c.wave = wv;
        c.lane = lane;
        return c;
    };
    copy_to_lds<NW, F8_K_PART_CHUNKS>(rsrc, tile0, kb0, wv, lane);
    copy_to_lds<NW, F8_V_PART_CHUNKS>(rsrc, tile0 + F8_K_PART_CHUNKS * 16, vb0, wv, lane);
    if (nt > 1) copy_to_lds<NW, F8_K_PART_CHUNKS>(rsrc, tile0 + F8_TILE_BYTES, kb1, wv, lane);

    // ---- Q prologue.  Largest |q'| is 448 q_scale (times sqrt(2) with RoPE);
    // choose e so that it maps to at most 448 after the factor qmul * sk.
    const float qbound = E4M3_MAX * q_scale * (has_rope ? 1.41421356237309515f : 1.0f) * qmul * sk;
    const int e = qbound > 0.0f ? min(max((int)ceilf(log2f(qbound / E4M3_MAX)), -126), 126) : 0;
    const float qfac = qmul * sk * ldexpf(1.0f, -e);
    const int qscale = E8M0_ONE + e;
    i32x8 qf[2];
    {
        const int row = qt * BM + wave * 32 + n;
        const bool ok = row < S;
        const uint4* qrow = q + (bh * S + row) * 8;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // dims 64 kk + 32 hh + 16 h .. +15: chunk c of the row
                const int c = kk * 4 + hh * 2 + h;
                uint4 w = make_uint4(0, 0, 0, 0);
                if (ok) w = qrow[c];
                float fv[16];
                fp8x4_to_f32(w.x, fv);
                fp8x4_to_f32(w.y, fv + 4);
                fp8x4_to_f32(w.z, fv + 8);
                fp8x4_to_f32(w.w, fv + 12);
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    float t[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x) t[x] = fv[8 * g + x] * q_scale;
                    if (has_rope && ok)
                        rotate4(t, cos_t[(int64_t)row * 16 + 2 * c + g], sin_t[(int64_t)row * 16 + 2 * c + g]);
#pragma unroll
                    for (int x = 0; x < 8; ++x) fv[8 * g + x] = clamp_e4m3(t[x] * qfac);
                }
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    qf[kk][4 * h + x] = (int)f32x4_to_fp8(fv[4 * x], fv[4 * x + 1], fv[4 * x + 2], fv[4 * x + 3]);
            }
        }
    }

    f32x16 o[4], negm = f32x16{};
    float lsum = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};

    // Scores of tile 0, offset so that its largest weight is 2^4, then the
    // pipelined steps.  Step i's scores live in sA for even i and sB for odd i.
    f32x16 sA[2], sB[2];
    i32x8 pf = i32x8{};
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
        float sum = 0.0f;
        f8_stage_a<true, false>(kb0, qf, qscale, negm, sA, sB, pf, sum, n, hh);
    }
    if (nt == 1) f8_mask_tail(sA, te - 1, S, hh);
    {
        const float shift = f8_tile_max(sA) - 4.0f;
        sA[0] -= shift;
        sA[1] -= shift;
        negm -= shift;
    }
    int i = 0;
    for (; i + 2 <= nt - 1; i += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f8_tile_step(kb1, vb0, sA, sB, qf, qscale, pf, o, negm, lsum, n, hh, copies(i + 2, kb0, true, i + 1, vb1));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f8_tile_step(kb0, vb1, sB, sA, qf, qscale, pf, o, negm, lsum, n, hh,
                     copies(i + 3, kb1, i + 3 < nt, i + 2, vb0));
    }
    if (i < nt - 1) {  // i = nt - 2, even: one more full step, then the last tile from sB / vb1
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f8_tile_step(kb1, vb0, sA, sB, qf, qscale, pf, o, negm, lsum, n, hh, copies(i + 2, kb0, false, i + 1, vb1));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f8_tile_step_last(vb1, sB, te - 1, S, qf, qscale, pf, o, negm, lsum, n, hh);
    } else {  // i = nt - 1, even: the last tile from sA / vb0
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        f8_tile_step_last(vb0, sA, te - 1, S, qf, qscale, pf, o, negm, lsum, n, hh);
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) settle(o[db]);

    // ---- epilogue (as in the bf16 kernel), O scaled by the V step.
    const float l = swap_halves_sum(lsum);
    const int rloc = wave * 32 + n;
    const int row = qt * BM + rloc;
    if (PARTIAL) {
        float* pw = part + (int64_t)logical * PART_FLOATS;
        float4* prow = reinterpret_cast<float4*>(pw + (int64_t)rloc * HEAD_DIM);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                prow[db * 8 + g * 2 + hh] = make_float4(o[db][4 * g] * sv, o[db][4 * g + 1] * sv,
                                                        o[db][4 * g + 2] * sv, o[db][4 * g + 3] * sv);
        if (hh == 0) {
            pw[BM * HEAD_DIM + rloc] = -negm[0];
            pw[BM * HEAD_DIM + BM + rloc] = l;
        }
    } else if (row < S) {
        const float inv = sv / l;
        uint2* orow = out + (bh * S + row) * 32;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                orow[db * 8 + g * 2 + hh] = make_uint2(pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                                       pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
    }
}

size_t core_fp8_partial_bytes(int BH, int S) { return core_partial_bytes_for(core_plan(BH, S)); }

hipError_t launch_attn_core_fp8(const void* q, float q_scale, const float* cos_t, const float* sin_t, const void* ws,
                                void* part, void* out, int BH, int S, float qmul, hipStream_t stream) {
    const CorePlan p = core_plan(BH, S);
    const uint4* qv = static_cast<const uint4*>(q);
    const uint8_t* wsv = static_cast<const uint8_t*>(ws);
    const float4* cv = reinterpret_cast<const float4*>(cos_t);
    const float4* sv = reinterpret_cast<const float4*>(sin_t);
    const int rope = cos_t != nullptr;
    if (p.full > 0)
        attn_core_fp8_kernel<false><<<p.full, NW * 64, 0, stream>>>(qv, q_scale, cv, sv, wsv, static_cast<uint2*>(out),
                                                                   nullptr, S, p.ntiles, p.nqt, 0, 1, qmul, rope);
    if (p.split > 0) {
        float* pt = static_cast<float*>(part);
        attn_core_fp8_kernel<true><<<p.split * p.nsplit, NW * 64, 0, stream>>>(
            qv, q_scale, cv, sv, wsv, nullptr, pt, S, p.ntiles, p.nqt, p.full, p.nsplit, qmul, rope);
        launch_merge(pt, out, nullptr, S, p.nqt, p.full, p.nsplit, p.split, stream);
    }
    return hipGetLastError();
}

}  // namespace dit
