// tile_layout.h - the K' tile format shared by the K preparation kernel
// (writer) and the bf16 attention kernel (reader), and the LDS layout of the
// V tiles that kernel copies straight from V, gfx950 only.
//
// The attention kernel streams K and V in tiles of KV_TILE = 64 keys.
//
//   K' tile (K_PART_BYTES = 17408, prepared): 64 rows of 272 bytes, stored in
//        the workspace exactly as it sits in LDS, so the kernel copies it with
//        linear 16-byte direct-to-LDS loads.  Row rho holds the rotated key
//        kperm(rho) of the tile: 16-byte chunk c (c < 16) holds dims
//        8c..8c+7, chunk 16 is zero padding.  Keys at or past S are zeros.
//   V tile (V_LDS_BYTES = 17408, not prepared): the 64 key rows of V ([B, H,
//        S, 128] bf16, 256 bytes per key) in 16 pieces of 4 rows.  Piece p
//        holds keys p, p + 16, p + 32, p + 48 of the tile (row r = key >> 4)
//        and sits V_PIECE_BYTES = 1088 bytes (1024 + 64 of padding) after
//        piece p - 1.  One direct-to-LDS load fills one piece, each lane
//        gathering 16 bytes of a key row (rows past S read as zeros).
//
// Why: the QK^T product is computed transposed (S^T = K' Q'^T) on
// v_mfma_f32_32x32x16_bf16 so each lane owns one query column.  In that
// accumulator layout lane half hh holds rows {4hh..4hh+3, 8+4hh..8+4hh+3} of
// every 16-row group; storing key kperm(rho) in row rho makes those rows the
// 8 consecutive keys 8hh..8hh+7, which is exactly the B-operand layout the PV
// product needs, so P goes from accumulator to MFMA operand without any lane
// exchange.  The PV A operand (V^T: one head dim per row, 8 consecutive keys
// per lane) is read from the key-major V tile with ds_read_b64_tr_b16, whose
// 16-lane groups each return a transposed 4 (keys) x 16 (dims) block; the
// four keys of such a block (16u + 8hh + 4h + j, j = 0..3) sit in four
// consecutive pieces, and the 64-byte piece padding moves consecutive pieces
// 16 banks apart, so a group reads 16 distinct bank pairs.  The K' row stride
// (17 chunks, odd) puts the rows read by consecutive lanes in distinct LDS
// banks and keeps every K' operand address one base plus a compile-time
// offset.
#pragma once

#include <stdint.h>

namespace dit {

constexpr int HEAD_DIM = 128;
constexpr int KV_TILE = 64;                              // keys per streamed tile
constexpr int K_ROW_CHUNKS = 17;                         // 16 data chunks + 1 pad
constexpr int K_PART_CHUNKS = KV_TILE * K_ROW_CHUNKS;    // 1088
constexpr int K_PART_BYTES = K_PART_CHUNKS * 16;         // 17408: one prepared K' tile
constexpr int V_PIECES = KV_TILE / 4;                    // 16 pieces of 4 key rows
constexpr int V_PIECE_CHUNKS = 68;                       // 64 data chunks + 4 pad
constexpr int V_PIECE_BYTES = V_PIECE_CHUNKS * 16;       // 1088
constexpr int V_LDS_CHUNKS = V_PIECES * V_PIECE_CHUNKS;  // 1088
constexpr int V_LDS_BYTES = V_LDS_CHUNKS * 16;           // 17408
constexpr int V_ROW_BYTES = HEAD_DIM * 2;                // 256: one key row of V

static_assert(K_PART_CHUNKS % 64 == 0, "the K' tile is whole wave copies");

__host__ __device__ constexpr inline int kperm(int rho) {
    return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}

// Chunk index (16 B units, inside a K' tile) holding dims 8c..8c+7 of row rho.
__host__ __device__ constexpr inline int k_chunk(int rho, int c) { return rho * K_ROW_CHUNKS + c; }

// Byte offset, inside an LDS V tile, of dim d of tile key `key`.
__host__ __device__ constexpr inline int v_lds_byte(int key, int d) {
    return (key & 15) * V_PIECE_BYTES + (key >> 4) * V_ROW_BYTES + 2 * d;
}

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
