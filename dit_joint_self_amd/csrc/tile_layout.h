// tile_layout.h - the workspace tile format shared by the K/V preparation
// kernel (writer) and the attention kernels (readers), gfx950 only.
//
// The attention kernels stream K and V in tiles of KV_TILE = 64 keys.  Each
// tile is stored in the workspace exactly as it will sit in LDS, so the
// kernels copy it with linear 16-byte direct-to-LDS loads:
//
//   K' part (K_PART_BYTES = 17408): 64 rows of 272 bytes.  Row rho holds the
//        rotated key kperm(rho) of the tile: 16-byte chunk c (c < 16) holds
//        dims 8c..8c+7, chunk 16 is zero padding.
//   V^T part (V_PART_BYTES = 18432): 128 rows of 144 bytes, one per head dim
//        d: chunk c (c < 8) holds keys 8c..8c+7 of the tile, chunk 8 is zero
//        padding.
//
// Why: the QK^T product is computed transposed (S^T = K' Q'^T) on
// v_mfma_f32_32x32x16_bf16 so each lane owns one query column.  In that
// accumulator layout lane half hh holds rows {4hh..4hh+3, 8+4hh..8+4hh+3} of
// every 16-row group; storing key kperm(rho) in row rho makes those rows the
// 8 consecutive keys 8hh..8hh+7, which is exactly the B-operand layout the PV
// product needs, so P goes from accumulator to MFMA operand without any lane
// exchange.  The padded row strides (17 and 9 chunks, both odd) put the rows
// read by consecutive lanes in distinct LDS banks, and keep every operand
// address of a lane equal to one base plus a compile-time offset.  Keys at or
// past S in the last tile are stored as zeros.
#pragma once

#include <stdint.h>

namespace dit {

constexpr int HEAD_DIM = 128;
constexpr int KV_TILE = 64;                              // keys per streamed tile
constexpr int K_ROW_CHUNKS = 17;                         // 16 data chunks + 1 pad
constexpr int V_ROW_CHUNKS = 9;                          // 8 data chunks + 1 pad
constexpr int K_PART_CHUNKS = KV_TILE * K_ROW_CHUNKS;    // 1088
constexpr int V_PART_CHUNKS = HEAD_DIM * V_ROW_CHUNKS;   // 1152
constexpr int K_PART_BYTES = K_PART_CHUNKS * 16;         // 17408
constexpr int V_PART_BYTES = V_PART_CHUNKS * 16;         // 18432
constexpr int TILE_CHUNKS = K_PART_CHUNKS + V_PART_CHUNKS;  // 2240 = 35 x 64
constexpr int TILE_BYTES = TILE_CHUNKS * 16;             // 35840

static_assert(K_PART_CHUNKS % 64 == 0 && V_PART_CHUNKS % 64 == 0, "parts are whole wave copies");

__host__ __device__ constexpr inline int kperm(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Chunk index (16 B units, inside the K part) holding dims 8c..8c+7 of row rho.
__host__ __device__ constexpr inline int k_chunk(int rho, int c) { return rho * K_ROW_CHUNKS + c; }

// Chunk index (inside the V part) holding keys 8c..8c+7 of head dim d.
__host__ __device__ constexpr inline int v_chunk(int d, int c) { return d * V_ROW_CHUNKS + c; }

__host__ __device__ constexpr inline int64_t num_kv_tiles(int S) {
    return (S + KV_TILE - 1) / KV_TILE;
}

}  // namespace dit
