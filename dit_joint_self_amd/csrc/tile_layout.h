// tile_layout.h - the workspace tile format shared by the K/V preparation
// kernel (writer) and the attention kernel (reader), gfx950 only.
//
// The attention kernel streams K and V in tiles of KV_TILE = 64 keys.  Each
// tile occupies TILE_BYTES = 32 KiB of workspace, laid out exactly as it will
// sit in LDS, so the attention kernel copies it with linear 16-byte
// direct-to-LDS loads:
//
//   bytes [0, 16K)   K' part: 64 rows x 256 B.  Row rho holds rotated key
//                    kperm(rho) of the tile (kperm swaps bits 2 and 3 of the
//                    row index); its 16-byte chunk p holds dims 8c..8c+7 with
//                    c = p ^ (rho & 15).
//   bytes [16K, 32K) V^T part: 64 "row pairs" x 256 B.  Head dim d lives in
//                    row pair d >> 1 at logical chunk L = (d & 1) * 8 + c,
//                    stored at physical chunk L ^ (d & 15); logical chunk c
//                    holds keys 8c..8c+7 of the tile for that d.
//
// Why: the QK^T product is computed transposed (S^T = K' Q'^T) on
// v_mfma_f32_32x32x16_bf16 so each lane owns one query column.  In that
// accumulator layout lane half hh holds rows {4hh..4hh+3, 8+4hh..8+4hh+3} of
// every 16-row group; storing key kperm(rho) in row rho makes those rows the
// 8 consecutive keys 8hh..8hh+7, which is exactly the B-operand layout the PV
// product needs, so P goes from accumulator to MFMA operand without any lane
// exchange.  The XOR swizzles make the 32 lanes that read one MFMA operand
// touch distinct LDS banks (for both 128-byte and 256-byte bank periods).
// Keys at or past S in the last tile are stored as zeros.
#pragma once

#include <stdint.h>

namespace dit {

constexpr int HEAD_DIM = 128;
constexpr int KV_TILE = 64;                       // keys per streamed tile
constexpr int K_PART_BYTES = KV_TILE * HEAD_DIM * 2;
constexpr int V_PART_BYTES = KV_TILE * HEAD_DIM * 2;
constexpr int TILE_BYTES = K_PART_BYTES + V_PART_BYTES;
constexpr int TILE_CHUNKS = TILE_BYTES / 16;      // 16-byte chunks per tile

__host__ __device__ constexpr inline int kperm(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Chunk index (16 B units, inside the K part) holding dims 8c..8c+7 of row rho.
__host__ __device__ constexpr inline int k_chunk(int rho, int c) {
    return rho * 16 + (c ^ (rho & 15));
}

// Chunk index (inside the V part) holding keys 8c..8c+7 of head dim d.
__host__ __device__ constexpr inline int v_chunk(int d, int c) {
    return (d >> 1) * 16 + ((((d & 1) << 3) | c) ^ (d & 15));
}

__host__ __device__ constexpr inline int64_t num_kv_tiles(int S) {
    return (S + KV_TILE - 1) / KV_TILE;
}

}  // namespace dit
