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

// ---------------------------------------------------------------------------
// fp8 (OCP e4m3) tiles, one byte per element, for the scaled-fp8 path.
//
//   K' part (F8_K_PART_BYTES = 9216): 64 rows of 144 bytes.  Row rho holds key
//        kperm(rho): bytes 0..127 are dims 0..127 (re-quantized after RoPE),
//        bytes 128..143 zero padding.
//   V^T part (F8_V_PART_BYTES = 10240): 128 rows of 80 bytes, one per head dim
//        d.  Byte 32*hh + j (hh in {0,1}, j < 32) holds key f8_vkey(hh, j) of
//        the tile; bytes 64..79 zero padding.  f8_vkey lists, for lane half hh,
//        the keys its 32x32 score accumulator holds in register order, so the
//        bytes of P and of V^T pair up key by key in the PV product.
//   Bytes [0, 16) of the workspace hold two fp32 scales written by the
//   preparation kernel: the K' quantization step and the V step.
// ---------------------------------------------------------------------------
constexpr int F8_K_ROW_CHUNKS = 9;                             // 8 data chunks + 1 pad
constexpr int F8_V_ROW_CHUNKS = 5;                             // 4 data chunks + 1 pad
constexpr int F8_K_PART_CHUNKS = KV_TILE * F8_K_ROW_CHUNKS;    // 576
constexpr int F8_V_PART_CHUNKS = HEAD_DIM * F8_V_ROW_CHUNKS;   // 640
constexpr int F8_TILE_CHUNKS = F8_K_PART_CHUNKS + F8_V_PART_CHUNKS;  // 1216 = 19 x 64
constexpr int F8_TILE_BYTES = F8_TILE_CHUNKS * 16;             // 19456
constexpr int F8_HEADER_BYTES = 256;                           // scales, then the tiles

static_assert(F8_K_PART_CHUNKS % 64 == 0 && F8_V_PART_CHUNKS % 64 == 0, "parts are whole wave copies");

__host__ __device__ constexpr inline int f8_vkey(int hh, int j) { return 16 * (j >> 3) + 8 * hh + (j & 7); }

}  // namespace dit
