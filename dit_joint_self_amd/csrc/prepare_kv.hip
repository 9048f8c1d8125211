// prepare_kv.hip - RoPE on K and its re-layout into streamed K' tiles (bf16
// path); RoPE on K and the K'/V^T tiles of the fp8 path.
//
// bf16: one workgroup of 256 threads per (batch*head, 64-key tile).  It reads
// the tile's 64 rows of K once from HBM ([B, H, S, 128] bf16), rotates them
// per interleaved pair in fp32 (RoPE as read from the DiT pages: the xDiT
// paper's abstract and the AMD RDNA 4 xDiT blog describe attention over
// RoPE'd text + latent tokens; pair j = dims (2j, 2j+1) times
// exp(i phi[s][j])), rounds to bf16 (RNE), and writes the K' tile image of
// tile_layout.h with coalesced stores (consecutive threads write consecutive
// 16-byte chunks).  Keys at or past S are written as zeros.  V needs no
// preparation: the attention kernel copies its rows as they are.
//
// Roofline: HBM bound.  Algorithmic bytes per tile and head: read 16 KiB of K
// + 16 KiB of cos/sin rows (shared by all heads, L2/MALL resident), write
// K_PART_BYTES = 17 KiB (the rows with their padding chunk).

#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "bf16_util.h"
#include "fp8_util.h"
#include "tile_layout.h"

namespace dit {

// G heads per workgroup: the tile's cos/sin chunks are loaded once and reused
// for every head of the group, and each head's K loads are issued before the
// previous head's rotations and stores.
template <int G>
__global__ __launch_bounds__(256) void prepare_k_kernel(
    const uint4* __restrict__ k, const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    uint4* __restrict__ ws, int* __restrict__ ctl, int S, int ntiles, int BH, int has_rope) {
    const int tile = blockIdx.x;
    // The attention launch's piece counters start from zero.
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 2)
        __hip_atomic_store(ctl + threadIdx.x * CTL_STRIDE, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t bh0 = (int64_t)blockIdx.y * G;
    const int ng = (int)min((int64_t)G, (int64_t)BH - bh0);  // heads of this group (workgroup-uniform)
    const int tid = threadIdx.x;
    const int key0 = tile * KV_TILE;

    // Output chunk x = (row rho, chunk c); chunk 16 of a row is padding.  Every
    // load of the thread is issued before any is used, so the HBM latency is
    // paid about once per workgroup rather than once per chunk.
    constexpr int KI = (K_PART_CHUNKS + 255) / 256;  // chunks per thread (the last partly)
    int koff[KI];  // element offset (16-byte units) of the chunk in a head's K; -1: a zero chunk
    float4 cw[KI], sw[KI];
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int x = tid + i * 256;
        const int rho = x / K_ROW_CHUNKS;
        const int c = x - rho * K_ROW_CHUNKS;
        const int key = key0 + kperm(rho);
        const bool live = x < K_PART_CHUNKS && c < 16 && key < S;
        koff[i] = live ? key * 16 + c : -1;
        if (live && has_rope) {
            cw[i] = cos_t[(int64_t)key * 16 + c];
            sw[i] = sin_t[(int64_t)key * 16 + c];
        }
    }
    uint4 kw[2][KI];
    auto load = [&](int64_t bh, uint4 (&w)[KI]) __attribute__((always_inline)) {
        const uint4* ksrc = k + bh * (int64_t)S * 16;
#pragma unroll
        for (int i = 0; i < KI; ++i) w[i] = koff[i] >= 0 ? ksrc[koff[i]] : make_uint4(0, 0, 0, 0);
    };
    load(bh0, kw[0]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g >= ng) break;
        if (g + 1 < ng) load(bh0 + g + 1, kw[(g + 1) & 1]);
        uint4* dst = ws + ((bh0 + g) * ntiles + tile) * (int64_t)K_PART_CHUNKS;
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int x = tid + i * 256;
            if (x >= K_PART_CHUNKS) break;
            uint4 w = kw[g & 1][i];
            if (has_rope && koff[i] >= 0) {
                float f[8];
                unpack8(w, f);
                rotate4(f, cw[i], sw[i]);
                w = pack8(f);
            }
            dst[x] = w;
        }
    }
}

// ---------------------------------------------------------------------------
// fp8 tiles (scaled-e4m3 path).  K codes are dequantised (x k_scale), rotated
// in fp32 and re-quantised with step sk = k_scale * sqrt(2) when RoPE is on (a
// rotation grows a component by at most sqrt(2) of the pair's largest, so the
// codes stay within +-448), else copied.  V codes are only re-laid out (V^T,
// keys in f8_vkey order).  Block (0, 0) stores {sk, v_scale} in the header.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prepare_kv_fp8_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    uint8_t* __restrict__ ws, int* __restrict__ ctl, int S, int ntiles, int has_rope, float k_scale, float v_scale) {
    __shared__ uint4 vtile[KV_TILE * 8];  // 64 keys x 128 e4m3 codes, key-major

    const int tile = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int key0 = tile * KV_TILE;
    const float sk = has_rope ? k_scale * 1.41421356237309515f : k_scale;
    if (tile == 0 && bh == 0 && tid == 0) {
        reinterpret_cast<float*>(ws)[0] = sk;
        reinterpret_cast<float*>(ws)[1] = v_scale;
    }
    // The attention launch's pool counters start from zero.
    if (tile == 0 && bh == 0 && tid < 2)
        __hip_atomic_store(ctl + tid * CTL_STRIDE, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint4* dst = reinterpret_cast<uint4*>(ws + F8_HEADER_BYTES) + (bh * ntiles + tile) * (int64_t)F8_TILE_CHUNKS;
    const uint4* ksrc = k + bh * (int64_t)S * 8;
    const uint4* vsrc = v + bh * (int64_t)S * 8;

    // Every load of the thread is issued before any is used, as in the bf16 kernel.
    constexpr int KI = (F8_K_PART_CHUNKS + 255) / 256;  // K chunks per thread (the last partly)
    uint4 vw[2], kw[KI];
    float4 cw[KI][2], sw[KI][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int x = tid + i * 256;
        const int key = key0 + (x >> 3);
        vw[i] = make_uint4(0, 0, 0, 0);
        if (key < S) vw[i] = vsrc[(int64_t)key * 8 + (x & 7)];
    }
    // K part: chunk x = (row rho, chunk c) holds dims 16c..16c+15; c = 8 is padding.
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int x = tid + i * 256;
        const int rho = x / F8_K_ROW_CHUNKS;
        const int c = x - rho * F8_K_ROW_CHUNKS;
        const int key = key0 + kperm(rho);
        kw[i] = make_uint4(0, 0, 0, 0);
        if (x < F8_K_PART_CHUNKS && c < 8 && key < S) {
            kw[i] = ksrc[(int64_t)key * 8 + c];
            if (has_rope) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    cw[i][h] = cos_t[(int64_t)key * 16 + 2 * c + h];
                    sw[i][h] = sin_t[(int64_t)key * 16 + 2 * c + h];
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) vtile[tid + i * 256] = vw[i];

    const float inv_sk = 1.0f / sk;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
        const int x = tid + i * 256;
        if (x >= F8_K_PART_CHUNKS) break;
        const int rho = x / F8_K_ROW_CHUNKS;
        const int c = x - rho * F8_K_ROW_CHUNKS;
        const int key = key0 + kperm(rho);
        uint4 w = kw[i];
        if (has_rope && c < 8 && key < S) {
            float f[16];
            fp8x4_to_f32(w.x, f);
            fp8x4_to_f32(w.y, f + 4);
            fp8x4_to_f32(w.z, f + 8);
            fp8x4_to_f32(w.w, f + 12);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float g[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) g[e] = f[8 * h + e] * k_scale;
                rotate4(g, cw[i][h], sw[i][h]);
#pragma unroll
                for (int e = 0; e < 8; ++e) f[8 * h + e] = clamp_e4m3(g[e] * inv_sk);
            }
            w = make_uint4(f32x4_to_fp8(f[0], f[1], f[2], f[3]), f32x4_to_fp8(f[4], f[5], f[6], f[7]),
                           f32x4_to_fp8(f[8], f[9], f[10], f[11]), f32x4_to_fp8(f[12], f[13], f[14], f[15]));
        }
        dst[x] = w;
    }

    __syncthreads();

    // V^T part, stored in order: chunk x = (row d = x / 5, c = x % 5) holds
    // bytes 16c..16c+15 of row d, i.e. keys f8_vkey(hh, j) for byte 32 hh + j;
    // c = 4 is padding.  Consecutive threads build and store consecutive
    // chunks, so every store instruction writes whole lines (with lanes over d
    // instead, 80 bytes apart, each store touched about 40 lines).
    const uint8_t* vt8 = reinterpret_cast<const uint8_t*>(vtile);
    uint4* vdst = dst + F8_K_PART_CHUNKS;
    for (int x = tid; x < F8_V_PART_CHUNKS; x += 256) {
        const int d = x / F8_V_ROW_CHUNKS;
        const int c = x - d * F8_V_ROW_CHUNKS;
        uint32_t w[4] = {0, 0, 0, 0};
        if (c < 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t acc = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int p = 16 * c + 4 * e + b;
                    acc |= (uint32_t)vt8[f8_vkey(p >> 5, p & 31) * 128 + d] << (8 * b);
                }
                w[e] = acc;
            }
        }
        vdst[x] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_prepare_kv_fp8(const void* k, const void* v, const float* cos_t, const float* sin_t, void* ws,
                                 int* ctl, int BH, int S, float k_scale, float v_scale, hipStream_t stream) {
    const int ntiles = (int)num_kv_tiles(S);
    dim3 grid(ntiles, BH);
    prepare_kv_fp8_kernel<<<grid, 256, 0, stream>>>(
        static_cast<const uint4*>(k), static_cast<const uint4*>(v), reinterpret_cast<const float4*>(cos_t),
        reinterpret_cast<const float4*>(sin_t), static_cast<uint8_t*>(ws), ctl, S, ntiles, cos_t != nullptr, k_scale,
        v_scale);
    return hipGetLastError();
}

hipError_t launch_prepare_k(const void* k, const float* cos_t, const float* sin_t, void* ws, int* ctl, int BH,
                            int S, hipStream_t stream) {
    const int ntiles = (int)num_kv_tiles(S);
    const uint4* kk = static_cast<const uint4*>(k);
    const float4* cc = reinterpret_cast<const float4*>(cos_t);
    const float4* ss = reinterpret_cast<const float4*>(sin_t);
    uint4* w = static_cast<uint4*>(ws);
    const int rope = cos_t != nullptr;
    // Heads per workgroup (the tile's table rows are loaded once for all of
    // them), timed inside the step, after an attention call has displaced the
    // caches: with tables (S x 64 x 8 bytes) of up to 16 MB two heads are
    // fastest (16896 tokens: 44.9 us with one, 40.6 with two, 43.5 with four;
    // 3584 tokens: the same 12 us for all three), beyond that four (76112
    // tokens, 39 MB of tables: 79.9 us with one, 89.3 with two, 78.9 with four).
    if (rope && (int64_t)S * HEAD_DIM * 4 > ((int64_t)16 << 20) && BH > 1) {
        dim3 grid(ntiles, (BH + 3) / 4);
        prepare_k_kernel<4><<<grid, 256, 0, stream>>>(kk, cc, ss, w, ctl, S, ntiles, BH, rope);
    } else if (rope && BH > 1) {
        dim3 grid(ntiles, (BH + 1) / 2);
        prepare_k_kernel<2><<<grid, 256, 0, stream>>>(kk, cc, ss, w, ctl, S, ntiles, BH, rope);
    } else {
        dim3 grid(ntiles, BH);
        prepare_k_kernel<1><<<grid, 256, 0, stream>>>(kk, cc, ss, w, ctl, S, ntiles, BH, rope);
    }
    return hipGetLastError();
}

}  // namespace dit
