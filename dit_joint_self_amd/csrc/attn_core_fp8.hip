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
// (attn_common.h).  Whole 19 KiB tiles (K' then V^T) stream through three
// LDS buffers, each copied one tile ahead.  Per 64-key tile a wave issues 4
// QK^T and 4 PV MFMAs of 32x32x64 (2 * 32 * 32 * 64 flop each), and between
// them the exp2 / e4m3 work that needs the QK^T result and feeds PV.  The two
// waves of each SIMD belong to two groups that run half a tile apart (see
// the kernel), so one wave's exp2 work meets the other's MFMAs.  Roofline:
// MFMA bound (fp8 peak).

#include <hip/hip_runtime.h>

#include <type_traits>

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

// Registers whose previous content does not matter: the packing below
// overwrites both halves of every word (no instruction is emitted).
__device__ __forceinline__ i32x8 unset_i32x8() {
    i32x8 v;
    asm("" : "=v"(v));
    return v;
}

// exp2 of a lane's 32 scores (two key blocks), packed to e4m3 in the PV B
// operand order (byte j = key block j/16, register j%16); fp32 sum of p'.
// No clamp to 448: a weight above it makes the lane's sum exceed
// F8_SUM_LIMIT, and the tile is then redone with a moved offset (p' <= 16).
// cvt_pk replaces one half of its destination register and keeps the other,
// so the packing needs no cleared register: the second call overwrites the
// half the first one kept (the caller passes unset registers).
__device__ __forceinline__ void f8_weights(const f32x16 (&s)[2], i32x8& pf, float& sum) {
    float t0, t1;  // started by the first pair: 0 + x would cost an add (it is not folded, for -0)
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const f32x16& sc = s[w >> 2];
        const int r = (w & 3) * 4;
        const float a = __builtin_amdgcn_exp2f(sc[r]), b = __builtin_amdgcn_exp2f(sc[r + 1]);
        const float c = __builtin_amdgcn_exp2f(sc[r + 2]), d = __builtin_amdgcn_exp2f(sc[r + 3]);
        t0 = w == 0 ? a + b : t0 + (a + b);
        t1 = w == 0 ? c + d : t1 + (c + d);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, pf[w], false);
        pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
    }
    sum = t0 + t1;
}

// First half of a tile: scores from the K' part kt, then the e4m3 weights
// (returned in PV B-operand order) with the offset bookkeeping.
template <bool MASKED>
__device__ __forceinline__ i32x8 f8_scores_weights(const uint4* kt, int j, bool first, int S, int n, int hh,
                                                   int qscale, const i32x8 (&qf)[2], f32x16 (&o)[4], f32x16& negm,
                                                   float& lsum) {

    // ---- S'^T = K' Q''^T * 2^e - m + 4: per key block kb, two 64-dim steps.
    f32x16 s[2];
    {
        i32x8 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kb = i >> 1, kk = i & 1;
            a[i] = lds_read32(kt + (kb * 32 + n) * F8_K_ROW_CHUNKS + kk * 4 + hh * 2);
        }
        // The MFMA blocks of both halves run at raised wave priority.  The
        // s_setprio pair also fixes where the compiler places the operand
        // reads (all before the block): 1.650 -> 1.609 ms at 16896 tokens,
        // bit-identical (priority 1 alike; priority raised instead outside the
        // blocks 1.620; around the PV MFMAs alone 5% slower).
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kb = i >> 1, kk = i & 1;
            s[kb] = mfma_f8(a[i], qf[kk], kk == 0 ? negm : s[kb], qscale);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    if (MASKED) {
        const int base = j * KV_TILE + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (base + 32 * kb + 16 * (r >> 3) + (r & 7) >= S) s[kb][r] = -INFINITY;
    }

    i32x8 pf = unset_i32x8();
    float tsum = 0.0f;
    bool slow = first;
    if (!slow) {
        f8_weights(s, pf, tsum);
        slow = __builtin_amdgcn_ballot_w64(!(tsum <= F8_SUM_LIMIT)) != 0;
    }
    if (slow) {
        // Exact row max of this tile becomes the offset: p' <= 16 afterwards.
        float mx = s[0][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
        mx = swap_halves_max(mx);
        const float shift = first ? mx - 4.0f : fmaxf(mx - 4.0f, 0.0f);
        if (!first) {
            const float alpha = __builtin_amdgcn_exp2f(-shift);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) o[db] *= alpha;
        }
        s[0] -= shift;
        s[1] -= shift;
        negm -= shift;
        f8_weights(s, pf, tsum);
    }
    lsum += tsum;
    return pf;
}

// Second half: O^T += V^T P'^T from the V^T part vt.
__device__ __forceinline__ void f8_pv(const uint4* vt, const i32x8& pf, f32x16 (&o)[4], int n, int hh) {
    // ---- O^T += V^T P'^T: four 32-dim blocks, 64 keys each.
    {
        i32x8 a[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) a[db] = lds_read32(vt + (db * 32 + n) * F8_V_ROW_CHUNKS + hh * 2);
        __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma_f8(a[db], pf, o[db], E8M0_ONE);
        __builtin_amdgcn_s_setprio(0);
        // The 16-pass fp8 MFMA keeps reading its A operand after it has
        // issued, and the compiler does not hold back a later LDS load into
        // those registers: the next tile's K' reads, right after the
        // barrier, could land in a V^T operand still being read (seen as
        // run-to-run differences in the output).  Pin the four products here
        // and let 16 wait states pass before anything else issues.
        asm volatile("s_nop 15" : "+v"(o[0]), "+v"(o[1]), "+v"(o[2]), "+v"(o[3]));
    }
}

__global__ __launch_bounds__(NW * 64) void attn_core_fp8_kernel(
    const uint4* __restrict__ q, float q_scale, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint8_t* __restrict__ ws, uint2* __restrict__ out, float* __restrict__ part, int* __restrict__ ctl, int S,
    int ntiles, int nqt, int full, int nsplit, int pool_whole, float qmul, int has_rope) {
    // Tile k of the range lives in buf[k % 3] (see the two wave groups below);
    // stage: 8 KiB per wave for the Q prologue and the epilogue.
    __shared__ uint4 lds0[F8_TILE_CHUNKS];
    __shared__ uint4 lds1[F8_TILE_CHUNKS];
    __shared__ uint4 lds2[F8_TILE_CHUNKS];
    __shared__ uint4 stage_all[NW * 512];
    uint4* const buf[3] = {lds0, lds1, lds2};
    if (DIT_DEBUG_LDS_NAN) {
        for (int b = 0; b < 3; ++b) debug_fill_lds<NW * 64>(buf[b], F8_TILE_CHUNKS);
        debug_fill_lds<NW * 64>(stage_all, NW * 512);
        __syncthreads();
    }

    // Static whole items first, then the pool (as in the bf16 kernel; attn_common.h).
    const int nstatic = full - pool_whole;
    const int pool_wgs = (int)gridDim.x - nstatic;
    CoreWork cw;
    if ((int)blockIdx.x < nstatic) {
        cw = core_work(blockIdx.x, nstatic, nstatic, nsplit);
    } else {
        const int u = take_unit(ctl, pool_wgs / 2);
        if (u < 0) {
            finish_pool_wg(ctl, pool_wgs);
            return;
        }
        cw = u < pool_whole ? whole_work(nstatic + u) : piece_work(u - pool_whole, full, nsplit);
    }
    const int64_t bh = cw.item / nqt;
    const int qt = cw.item - (int)bh * nqt;
    const int tb = (int)((int64_t)cw.f * ntiles / cw.nsplit);
    const int te = (int)((int64_t)(cw.f + 1) * ntiles / cw.nsplit);

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
    copy_to_lds<NW, F8_TILE_CHUNKS>(rsrc, tb * F8_TILE_BYTES, lds0, wv, lane);

    // ---- Q prologue.  Largest |q'| is 448 q_scale (times sqrt(2) with RoPE);
    // choose e so that it maps to at most 448 in magnitude after the factor
    // qmul * sk (qmul carries the sign of the softmax scale, which may be
    // negative).
    const float qbound = fabsf(E4M3_MAX * q_scale * (has_rope ? 1.41421356237309515f : 1.0f) * qmul * sk);
    const int e = qbound > 0.0f ? min(max((int)ceilf(log2f(qbound / E4M3_MAX)), -126), 126) : 0;
    const float qfac = qmul * sk * ldexpf(1.0f, -e);
    const int qscale = E8M0_ONE + e;
    // The loads are coalesced as in the bf16 kernel: load i of lane l covers
    // 16-byte chunk l % 8 (16 codes, RoPE pairs 8c..8c+7) of row 8 i + l / 8
    // of the wave's 32 rows of 128 codes (8 whole cache lines per load), with
    // cos/sin chunks 2c and 2c + 1 of the same row.  Dequantise, rotate and
    // requantise run in that layout; the codes reach the MFMA layout (lane
    // (n, hh): chunks 4 kk + 2 hh + h of row n) through the wave's part of
    // `stage`, where row rho keeps chunk c in slot c ^ ((rho / 2) % 8) (both
    // directions spread over all LDS banks).  Rows past S read row S - 1 and
    // are zeroed.
    char* const stage = reinterpret_cast<char*>(stage_all) + wave * 8192;
    i32x8 qf[2];
    {
        const int row0 = qt * BM + wave * 32;  // the wave's first row
        const int c = lane & 7;
        uint4 qw[4];
        float4 cosw[4][2], sinw[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 8 * i + (lane >> 3);
            const int64_t rr = r < S ? r : S - 1;
            qw[i] = q[(bh * S + rr) * 8 + c];
            if (has_rope) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    cosw[i][u] = cos_t[rr * 16 + 2 * c + u];
                    sinw[i][u] = sin_t[rr * 16 + 2 * c + u];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 w = qw[i];
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
                if (has_rope) rotate4(t, cosw[i][g], sinw[i][g]);
#pragma unroll
                for (int x = 0; x < 8; ++x) fv[8 * g + x] = clamp_e4m3(t[x] * qfac);
            }
            uint32_t code[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) code[x] = f32x4_to_fp8(fv[4 * x], fv[4 * x + 1], fv[4 * x + 2], fv[4 * x + 3]);
            const int rho = 8 * i + (lane >> 3);
            const uint4 pk = row0 + rho < S ? make_uint4(code[0], code[1], code[2], code[3]) : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(stage + rho * 128 + ((c ^ ((rho >> 1) & 7)) << 4)) = pk;
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int slot = (4 * kk + 2 * hh + h) ^ ((n >> 1) & 7);
                const uint4 w = *reinterpret_cast<const uint4*>(stage + n * 128 + (slot << 4));
                qf[kk][4 * h + 0] = (int)w.x;
                qf[kk][4 * h + 1] = (int)w.y;
                qf[kk][4 * h + 2] = (int)w.z;
                qf[kk][4 * h + 3] = (int)w.w;
            }
    }

    f32x16 o[4], negm = f32x16{};
    float lsum = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};

    // Each tile is QK^T MFMAs, then exp2 / e4m3 work that needs their result,
    // then the PV MFMAs.  Two wave groups, one wave of each per SIMD, run half
    // a tile apart so that one wave's exp2 work meets the other wave's MFMAs.
    // With L = nt - 1 and barriers 0..L+1, the interval after barrier k holds
    //   group 0 (waves 0..NW/2-1): scores + weights of tile k, PV of tile k
    //   group 1 (the other waves):  PV of tile k - 1, scores + weights of tile k
    // so tiles k - 1 and k are read in it; the copy of tile k + 1 issued in it
    // goes to the buffer of tile k - 2, which both groups finished before the
    // barrier.  Both groups pass the same L + 2 barriers; group 1 carries the
    // weights of a tile across one.
    const int L = te - 1 - tb;
    const bool g1 = wv >= NW / 2;
    // The range's last tile (masked) is kept out of the loops, whose steps
    // then all look the same to the register allocator.
    using full_t = std::false_type;
    using last_t = std::true_type;
    auto scores_weights = [&](const uint4* kt, int k, auto lastc) __attribute__((always_inline)) {
        return f8_scores_weights<decltype(lastc)::value>(kt, tb + k, k == 0, S, n, hh, qscale, qf, o, negm, lsum);
    };
    // Only group 1 copies tiles (its four waves, one per SIMD, each a quarter
    // of the pieces), right after the barrier: issuing a copy holds up the
    // wave's next instructions, and meanwhile the group-0 wave of the SIMD
    // issues its score MFMAs (all eight waves copying: 1.592 -> 1.551 ms at
    // 16896 tokens; group 0 copying instead 1.602; group 1 copying after its
    // PV MFMAs 1.607; outputs identical).
    auto copy_tile = [&](int k, uint4* dst) __attribute__((always_inline)) {
        if (k <= L && g1) copy_to_lds<NW / 2, F8_TILE_CHUNKS>(rsrc, (tb + k) * F8_TILE_BYTES, dst, wv - NW / 2, lane);
    };
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (!g1) {
        auto step = [&](auto rc, int k, auto lastc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;  // k % 3
            copy_tile(k + 1, buf[(R + 1) % 3]);
            const i32x8 pf = scores_weights(buf[R], k, lastc);
            f8_pv(buf[R] + F8_K_PART_CHUNKS, pf, o, n, hh);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        };
        for (int k = 0;;) {
            if (k >= L) break;
            step(std::integral_constant<int, 0>{}, k++, full_t{});
            if (k >= L) break;
            step(std::integral_constant<int, 1>{}, k++, full_t{});
            if (k >= L) break;
            step(std::integral_constant<int, 2>{}, k++, full_t{});
        }
        switch (L % 3) {
            case 0: step(std::integral_constant<int, 0>{}, L, last_t{}); break;
            case 1: step(std::integral_constant<int, 1>{}, L, last_t{}); break;
            default: step(std::integral_constant<int, 2>{}, L, last_t{}); break;
        }
    } else {
        copy_tile(1, lds1);
        i32x8 pf = L == 0 ? scores_weights(lds0, 0, last_t{}) : scores_weights(lds0, 0, full_t{});
        auto step = [&](auto rc, int k, auto lastc) __attribute__((always_inline)) {
            constexpr int R = decltype(rc)::value;  // k % 3
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            copy_tile(k + 1, buf[(R + 1) % 3]);
            f8_pv(buf[(R + 2) % 3] + F8_K_PART_CHUNKS, pf, o, n, hh);
            pf = scores_weights(buf[R], k, lastc);
        };
        for (int k = 1;;) {
            if (k >= L) break;
            step(std::integral_constant<int, 1>{}, k++, full_t{});
            if (k >= L) break;
            step(std::integral_constant<int, 2>{}, k++, full_t{});
            if (k >= L) break;
            step(std::integral_constant<int, 0>{}, k++, full_t{});
        }
        if (L > 0) {
            switch (L % 3) {
                case 0: step(std::integral_constant<int, 0>{}, L, last_t{}); break;
                case 1: step(std::integral_constant<int, 1>{}, L, last_t{}); break;
                default: step(std::integral_constant<int, 2>{}, L, last_t{}); break;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        switch (L % 3) {
            case 0: f8_pv(lds0 + F8_K_PART_CHUNKS, pf, o, n, hh); break;
            case 1: f8_pv(lds1 + F8_K_PART_CHUNKS, pf, o, n, hh); break;
            default: f8_pv(lds2 + F8_K_PART_CHUNKS, pf, o, n, hh); break;
        }
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) settle(o[db]);

    // ---- epilogue (as in the bf16 kernel), O scaled by the V step, through
    // the wave's part of `stage` so the global stores are coalesced.  The
    // prologue's reads of it were done before the first barrier.
    const float l = swap_halves_sum(lsum);
    const int rloc = wave * 32 + n;
    const int row0 = qt * BM + wave * 32;
    if (cw.partial) {
        // fp32 rows in two passes of 64 dims (256 bytes per row): row n keeps
        // 16-byte piece p of the pass in slot p ^ (n % 16).
        float* pw = part + (int64_t)cw.piece * PART_FLOATS;
        float4* pwave = reinterpret_cast<float4*>(pw + (int64_t)wave * 32 * HEAD_DIM);
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int d2 = 0; d2 < 2; ++d2)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int db = 2 * pass + d2, piece = d2 * 8 + g * 2 + hh;
                    *reinterpret_cast<float4*>(stage + n * 256 + ((piece ^ (n & 15)) << 4)) =
                        make_float4(o[db][4 * g] * sv, o[db][4 * g + 1] * sv, o[db][4 * g + 2] * sv,
                                    o[db][4 * g + 3] * sv);
                }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rho = 4 * i + (lane >> 4), cc = lane & 15;
                pwave[rho * 32 + 16 * pass + cc] =
                    *reinterpret_cast<const float4*>(stage + rho * 256 + ((cc ^ (rho & 15)) << 4));
            }
        }
        if (hh == 0) {
            pw[BM * HEAD_DIM + rloc] = -negm[0];
            pw[BM * HEAD_DIM + BM + rloc] = l;
        }
    } else {
        // bf16 rows of 256 bytes: row n keeps 8-byte piece p (dims 4p..4p+3)
        // in slot p ^ n, so 16-byte chunk c sits in slot c ^ (n / 2), its
        // halves swapped when n is odd.
        const float inv = sv / l;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int piece = db * 8 + g * 2 + hh;
                *reinterpret_cast<uint2*>(stage + n * 256 + ((piece ^ n) << 3)) =
                    make_uint2(pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                               pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rho = 4 * i + (lane >> 4), cc = lane & 15;
            uint4 w = *reinterpret_cast<const uint4*>(stage + rho * 256 + ((cc ^ (rho >> 1)) << 4));
            if (rho & 1) w = make_uint4(w.z, w.w, w.x, w.y);
            if (row0 + rho < S) reinterpret_cast<uint4*>(out)[(bh * S + row0 + rho) * 16 + cc] = w;
        }
    }
    if ((int)blockIdx.x >= nstatic) finish_pool_wg(ctl, pool_wgs);
}

size_t core_fp8_partial_bytes(int BH, int S) { return core_partial_bytes_for(core_plan(BH, S)); }

hipError_t launch_attn_core_fp8(const void* q, float q_scale, const float* cos_t, const float* sin_t, const void* ws,
                                void* part, int* ctl, void* out, int BH, int S, float qmul, hipStream_t stream) {
    const CorePlan p = core_plan(BH, S);
    const uint4* qv = static_cast<const uint4*>(q);
    const uint8_t* wsv = static_cast<const uint8_t*>(ws);
    const float4* cv = reinterpret_cast<const float4*>(cos_t);
    const float4* sv = reinterpret_cast<const float4*>(sin_t);
    const int rope = cos_t != nullptr;
    float* pt = static_cast<float*>(part);
    attn_core_fp8_kernel<<<core_grid_dynamic(p), NW * 64, 0, stream>>>(qv, q_scale, cv, sv, wsv,
                                                                      static_cast<uint2*>(out), pt, ctl, S, p.ntiles,
                                                                      p.nqt, p.full, p.nsplit, core_pool_whole(p), qmul,
                                                                      rope);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.split > 0) e = launch_merge(pt, out, nullptr, S, p.nqt, p.full, p.nsplit, p.split, stream);
    return e;
}

}  // namespace dit
