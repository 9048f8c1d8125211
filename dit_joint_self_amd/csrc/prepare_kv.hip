// prepare_kv.hip - RoPE on K and re-layout of K and V into streamed tiles.
//
// One workgroup of 256 threads per (batch*head, 64-key tile).  It reads the
// tile's 64 rows of K and V once from HBM ([B, H, S, 128] bf16), rotates K per
// interleaved pair in fp32 (RoPE as read from the DiT pages: the xDiT paper's
// abstract and the AMD RDNA 4 xDiT blog describe attention over RoPE'd text +
// latent tokens; pair j = dims (2j, 2j+1) times exp(i phi[s][j])), rounds to
// bf16 (RNE), and writes the tile in the LDS image described in tile_layout.h.
// V is transposed through LDS so the attention kernel can read it as the A
// operand of O^T = V^T P^T.  Keys at or past S are written as zeros so the
// PV product never multiplies a masked probability by garbage.
//
// Roofline: HBM bound.  Algorithmic bytes per tile and head: read 2 x 16 KiB
// (K, V) + 2 x 16 KiB (cos, sin rows when RoPE is on; shared by all heads),
// write TILE_BYTES = 35 KiB (the two parts with their row padding).

#include <hip/hip_runtime.h>

#include "bf16_util.h"
#include "tile_layout.h"

namespace dit {

__global__ __launch_bounds__(256) void prepare_kv_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const float4* __restrict__ cos_t, const float4* __restrict__ sin_t,
    uint4* __restrict__ ws, int S, int ntiles, int has_rope) {
    __shared__ uint4 vtile[KV_TILE * 16];  // 64 keys x 128 dims, key-major

    const int tile = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int key0 = tile * KV_TILE;
    uint4* dst = ws + (bh * ntiles + tile) * (int64_t)TILE_CHUNKS;
    const uint4* ksrc = k + bh * (int64_t)S * 16;
    const uint4* vsrc = v + bh * (int64_t)S * 16;

    // V rows into LDS (coalesced 16-byte loads).
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int x = tid + i * 256;
        const int key = key0 + (x >> 4);
        uint4 w = make_uint4(0, 0, 0, 0);
        if (key < S) w = vsrc[(int64_t)key * 16 + (x & 15)];
        vtile[x] = w;
    }

    // K part: output chunk x = (row rho, chunk c); chunk 16 of a row is padding.
    for (int x = tid; x < K_PART_CHUNKS; x += 256) {
        const int rho = x / K_ROW_CHUNKS;
        const int c = x - rho * K_ROW_CHUNKS;
        const int key = key0 + kperm(rho);
        uint4 w = make_uint4(0, 0, 0, 0);
        if (c < 16 && key < S) {
            w = ksrc[(int64_t)key * 16 + c];
            if (has_rope) {
                float f[8];
                unpack8(w, f);
                rotate4(f, cos_t[(int64_t)key * 16 + c], sin_t[(int64_t)key * 16 + c]);
                w = pack8(f);
            }
        }
        dst[x] = w;
    }

    __syncthreads();

    // V^T part: chunk (d, c) = keys 8c..8c+7 of head dim d.  Lanes run over d
    // so the 2-byte LDS gathers of one instruction hit one row.
    const unsigned short* vt16 = reinterpret_cast<const unsigned short*>(vtile);
    uint4* vdst = dst + K_PART_CHUNKS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int y = tid + i * 256;
        const int d = y & 127;
        const int c = y >> 7;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = vt16[(c * 8 + 2 * e) * 128 + d];
            const uint32_t hi = vt16[(c * 8 + 2 * e + 1) * 128 + d];
            w[e] = lo | (hi << 16);
        }
        vdst[v_chunk(d, c)] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (tid < HEAD_DIM) vdst[v_chunk(tid, 8)] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_prepare_kv(const void* k, const void* v, const float* cos_t, const float* sin_t,
                             void* ws, int BH, int S, hipStream_t stream) {
    const int ntiles = (int)num_kv_tiles(S);
    dim3 grid(ntiles, BH);
    prepare_kv_kernel<<<grid, 256, 0, stream>>>(
        static_cast<const uint4*>(k), static_cast<const uint4*>(v),
        reinterpret_cast<const float4*>(cos_t), reinterpret_cast<const float4*>(sin_t),
        static_cast<uint4*>(ws), S, ntiles, cos_t != nullptr);
    return hipGetLastError();
}

}  // namespace dit
