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
//     accumulator owns query n and 16 keys, so the row max is 31 in-lane
//     max ops plus one v_permlane32_swap, and the row sum stays per lane
//     until the epilogue.
//   * Online softmax in base 2 with lazy rescaling: the running max used for
//     the exponent is only raised when a tile's max exceeds it by more than
//     RESCALE_THRESHOLD (then O and l are multiplied by 2^(m_old - m_new)).
//     Exponents stay <= 2^8, which fp32 and bf16 hold exactly as well as any
//     other value, and the final O / l is unchanged.
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

constexpr float RESCALE_THRESHOLD = 8.0f;

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

template <int NW>
__device__ __forceinline__ void load_tile_async(const uint4* __restrict__ src, uint4* lds_dst,
                                                int wave, int lane) {
    constexpr int PER_WAVE = TILE_CHUNKS / (NW * 64);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int chunk0 = (i * NW + wave) * 64;
        __builtin_amdgcn_global_load_lds(
            (const void*)(src + chunk0 + lane),
            (__attribute__((address_space(3))) void*)(lds_dst + chunk0), 16, 0, 0);
    }
}

template <int NW, int QB>
__global__ __launch_bounds__(NW * 64) void attn_core_kernel(
    const uint4* __restrict__ q, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    const uint4* __restrict__ ws, uint2* __restrict__ out, int S, int ntiles, int nqt,
    int total_wg, float qmul, int has_rope) {
    constexpr int BM = NW * 32 * QB;
    __shared__ uint4 lds[2 * TILE_CHUNKS];

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
    load_tile_async<NW>(src, lds, wave, lane);

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

    f32x16 o[QB][4];
    float m_used[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_used[qb] = -INFINITY;
        lsum[qb] = 0.0f;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[qb][db] = f32x16{};
    }

    for (int j = 0; j < ntiles; ++j) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (j + 1 < ntiles)
            load_tile_async<NW>(src + (int64_t)(j + 1) * TILE_CHUNKS, lds + ((j + 1) & 1) * TILE_CHUNKS,
                                wave, lane);
        const uint4* kt = lds + (j & 1) * TILE_CHUNKS;
        const uint4* vt = kt + TILE_CHUNKS / 2;

        // ---- S^T = K' Q'^T for 64 keys x (32 * QB) queries.
        f32x16 s[QB][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][0] = s[qb][1] = f32x16{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int rho = kb * 32 + n;
                const bf16x8 a = as_bf16x8(kt[k_chunk(rho, 2 * t + hh)]);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][t], s[qb][kb], 0, 0, 0);
            }
        }

        // ---- keys past S (last tile only): lane half hh, register r of key
        // block kb holds key 32 kb + 16 (r >> 3) + 8 hh + (r & 7).
        if (j == ntiles - 1 && (S & (KV_TILE - 1))) {
            const int base = j * KV_TILE + 8 * hh;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (base + 32 * kb + 16 * (r >> 3) + (r & 7) >= S) s[qb][kb][r] = -INFINITY;
        }

        // ---- online softmax (base 2), P to bf16 B operands.
        bf16x8 pf[QB][2][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = s[qb][0][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][0][r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][1][r]);
            mx = swap_halves_max(mx);
            const bool need = mx > m_used[qb] + RESCALE_THRESHOLD;
            if (__builtin_amdgcn_ballot_w64(need)) {
                const float m_new = fmaxf(m_used[qb], mx);
                const float alpha = __builtin_amdgcn_exp2f(m_used[qb] - m_new);
                lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < 4; ++db) o[qb][db] *= alpha;
                m_used[qb] = m_new;
            }
            const float m = m_used[qb];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    p[r] = __builtin_amdgcn_exp2f(s[qb][kb][r] - m);
                    lsum[qb] += p[r];
                }
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    const uint4 w = make_uint4(pack_bf16x2(p[8 * t2 + 0], p[8 * t2 + 1]),
                                               pack_bf16x2(p[8 * t2 + 2], p[8 * t2 + 3]),
                                               pack_bf16x2(p[8 * t2 + 4], p[8 * t2 + 5]),
                                               pack_bf16x2(p[8 * t2 + 6], p[8 * t2 + 7]));
                    pf[qb][kb][t2] = as_bf16x8(w);
                }
            }
        }

        // ---- O^T += V^T P^T: 128 dims x (32 * QB) queries, 64 keys.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int d = db * 32 + n;
                    const bf16x8 a = as_bf16x8(vt[v_chunk(d, kb * 4 + t2 * 2 + hh)]);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][kb][t2], o[qb][db], 0, 0, 0);
                }
            }
        }
    }

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

int core_block_m() {
    switch (core_variant()) {
        case 1: return 4 * 32 * 2;
        case 2: return 4 * 32 * 1;
        default: return 8 * 32 * 1;
    }
}

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

hipError_t launch_attn_core(const void* q, const float* cos_t, const float* sin_t, const void* ws,
                            void* out, int BH, int S, float qmul, hipStream_t stream) {
    switch (core_variant()) {
        case 1: return launch_core_t<4, 2>(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
        case 2: return launch_core_t<4, 1>(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
        default: return launch_core_t<8, 1>(q, cos_t, sin_t, ws, out, BH, S, qmul, stream);
    }
}

}  // namespace dit
