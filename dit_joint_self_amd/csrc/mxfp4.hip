// mxfp4.hip - MXFP4 (OCP Microscaling) activation quantisation and the
// block-scaled A4W4 GEMM of the DiT linear layers, gfx950.
//
// The MXFP4/Quark on MI350 blog quantises FLUX's linear layers to MXFP4 as
// the OCP MX specification defines it (section "MXFP4 Quantization": 32 FP4
// elements share one E8M0 scale; weights static, activations dynamic, blocks
// along the reduction axis), and runs them as an activation quantisation
// kernel plus an A4W4 matrix-core GEMM (section "MXFP4 Kernel").
//
// Formats (shared by the quantiser and the GEMM):
//   codes  [R, K/2] bytes, row-major: element k of a row in byte k/2, low
//          nibble for even k; E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit.
//   scales E8M0 biased exponent of each 32-element block, in tiles of 32 rows
//          x 8 blocks (256 contiguous bytes, row-major inside the tile):
//          block b of row r at byte ((r / 32) * G + b / 8) * 256 + (r % 32) * 8
//          + b % 8, with G = ceil(K / 256) tiles per row of tiles
//          (mx_scale_index).  A GEMM step (256 of K) of a 256-row operand tile
//          then reads eight whole 256-byte tiles instead of 8 bytes from each of
//          256 rows 96 bytes apart; bytes of rows past R or blocks past K/32 are
//          never read.
//
// Quantisation of a block V (the MX rule): X = floor(log2 max|V|) - 2 (the
// largest E2M1 exponent), clamped to [-127, 127] (an all-zero block takes
// -127); P_i = V_i * 2^-X rounded to the nearest E2M1 value, ties to the even
// code, magnitudes above 6 saturated to 6, sign bit kept.  Every step is
// exact (bf16 inputs, power-of-two scaling, then the hardware conversion's
// rounding, which follows that rule), so the codes do not depend on
// evaluation order.
//
// GEMM: C[M, N] (bf16) = deq(A)[M, K] deq(W)[N, K]^T on
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands.  In that instruction
// lane l supplies row/column l % 32 and the 32 elements of K-half l / 32 of
// the 64-deep step, and its E8M0 scale multiplies exactly those 32 elements:
// one MX block per lane, so the block scaling costs nothing.  The product is
// computed transposed (C^T = W A^T) so a lane's accumulator holds 4
// consecutive output columns, stored as one 8-byte write.
//
// Roofline: quantiser HBM bound (per 32-element block: 64 B read, 17 B
// written); GEMM MFMA bound at FLUX shapes (2 M N K flop; fp4 dense peak
// 10.1 PFLOP/s), with the bf16 output (2 M N bytes) its largest HBM term.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "gfx950.h"
#include "bf16_util.h"

namespace dit {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Byte of block b of row r in the tiled scale layout (G tiles per row of tiles).
__host__ __device__ __forceinline__ int64_t mx_scale_index(int64_t r, int b, int G) {
    return ((r >> 5) * G + (b >> 3)) * 256 + (r & 31) * 8 + (b & 7);
}
__host__ __device__ __forceinline__ int64_t mx_scale_size(int64_t rows, int K) {
    return ((rows + 31) / 32) * ((K + 255) / 256) * 256;
}
size_t mx_scale_bytes(int64_t rows, int K) { return (size_t)mx_scale_size(rows, K); }

// ---------------------------------------------------------------- quantiser

// Thread t: elements 8t .. 8t+7 of the flattened [R, K] input (K % 32 == 0, so
// 4 consecutive lanes hold one block).  Grid-stride.
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const uint4* __restrict__ x,
                                                             uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, int64_t groups, int K) {
    // groups is a multiple of 4 and t steps in multiples of 4, so the 4 lanes of
    // a block enter and leave the loop together (the shuffles need all four)
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < groups; t += (int64_t)gridDim.x * 256) {
        float v[8];
        unpack8(x[t], v);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
        a = fmaxf(a, __shfl_xor(a, 1, 4));
        a = fmaxf(a, __shfl_xor(a, 2, 4));
        // floor(log2 a) from the exponent field; zero and subnormal maxima clamp to -127
        const int X = max((int)((__float_as_uint(a) >> 23) & 0xff) - 127 - 2, -127);
        // v_cvt_scalef32_pk_fp4_f32 rounds two values divided by the scale to
        // E2M1 exactly as the MX rule does (nearest, ties to the even code,
        // magnitudes above 6 to 6, the sign kept, -0 included), for every
        // power-of-two scale 2^-127 .. 2^127 (checked against the rule on the
        // GPU value by value, at every rounding midpoint and either side of
        // it); the first value goes to the low nibble of the selected byte.
        // The scale's bits are built directly: 2^-127 is an fp32 subnormal.
        const float scale = __uint_as_float(X >= -126 ? (uint32_t)(X + 127) << 23 : 0x00400000u);
        uint32_t packed = 0;
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[0], v[1], scale, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], scale, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], scale, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], scale, 3);
        codes[t] = packed;
        if ((t & 3) == 0) {
            const int64_t blk = t >> 2, per_row = K / 32;
            const int64_t r = blk / per_row;
            scales[mx_scale_index(r, (int)(blk - r * per_row), (K + 255) / 256)] = (uint8_t)(X + 127);
        }
    }
}

hipError_t launch_mxfp4_quantize(const void* x, void* codes, void* scales, int64_t rows, int K,
                                 hipStream_t stream) {
    const int64_t groups = rows * (K / 8);
    const int64_t blocks = std::min<int64_t>((groups + 255) / 256, (int64_t)MI355X_CUS * 32);
    mxfp4_quantize_kernel<<<(int)blocks, 256, 0, stream>>>(static_cast<const uint4*>(x),
                                                           static_cast<uint32_t*>(codes),
                                                           static_cast<uint8_t*>(scales), groups, K);
    return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM

constexpr int GM = 256;      // rows of A (output rows) per workgroup
constexpr int GN = 256;      // rows of W (output columns) per workgroup
constexpr int GK = 256;      // K per pipeline step: four 64-deep MFMA steps, 128 bytes of each row
constexpr int GWAVES = 8;    // wave (wm, wn) = (w & 3, w >> 2): 64 rows x 128 columns each
constexpr int G_GROUP = 8;   // column tiles per group of the workgroup order
// Scales of a step: 8 whole scale tiles (256 rows x 8 bytes) per operand, two
// 1 KiB pieces each, copied by the step's four copying waves (A: the first
// two, W: the other two; the W part of a 128-wide tile is one piece, the third).
static_assert(GM == 256 && GN == 256 && GK == 256, "one scale tile column per step and 32-row tile");

// LDS image of a tile: rows of GK/2 = 128 bytes = eight 16-byte chunks; chunk c
// of row r sits at position c ^ ((r >> 1) & 7), so the 16 lanes of an LDS read
// quarter (rows r .. r+15, one chunk each) hit 16 distinct bank groups.  A copy
// piece is 8 whole rows: every global read of the copy is a full 128-byte line
// (pieces gathering half lines from 16 rows copy at half the rate).
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Per-lane global byte offset (without the step's K offset) of the chunk that
// lane `lane` of code piece p brings in: LDS chunk 64 p + lane = (row, position),
// global chunk = position un-swizzled.  Rows past the matrix repeat its last
// row (never stored); chunks past K (the last step when K % 256 == 128) are
// never read by the MFMAs.
__device__ __forceinline__ int piece_offset(int p, int lane, int row0, int rows, int rowbytes) {
    const int i = p * 64 + lane;
    const int r = i >> 3, q = i & 7;
    const int c = q ^ ((r >> 1) & 7);
    const int row = min(row0 + r, rows - 1);
    return row * rowbytes + c * 16;
}

__device__ __forceinline__ f32x16 mfma_fp4(const uint4& a, const uint4& b, const f32x16& c, int sa, int sb,
                                           int opsel) {
    const i32x8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    // cbsz = blgp = 4: both operands FP4 (E2M1); opsel picks the scale byte
    if (opsel == 0) return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 2, sa, 2, sb);
}

// One pipeline stage: the A tile (GM rows) and the W tile (GN rows) of a K
// step, and the step's eight block scales of every row (8 bytes per row, row
// r at byte 8 r: the step's eight scale tiles as they are in memory).  A lane
// reads the 8 bytes of each of its rows with one 8-byte LDS read (reading the
// 16-byte row pair instead moved twice the bytes: 1.6% slower).
struct GStage {
    uint4 a[GM * 8];
    uint4 w[GN * 8];
    uint4 sa[GM / 2];
    uint4 sw[GN / 2];
};

// One output tile of GM rows x TN columns (TN = 256, or 128 for the tiles
// of a last partial round), 8 waves; accumulators acc[nb][mb] of C^T (wave
// columns (TN / 2) wn + 32 nb, rows 64 wm + 32 mb).  Both tile widths use the
// kernel's two stage objects (a 128-wide tile fills the first half of their
// W parts).
template <int TN>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
                                          const uint8_t* __restrict__ w_codes, const uint8_t* __restrict__ w_scales,
                                          uint2* __restrict__ out, int M, int N, int K, int m0, int n0, GStage& st0,
                                          GStage& st1) {
    static_assert(TN == 256 || TN == 128, "tile widths");
    constexpr int NB = TN / 64;                          // 32-column blocks per wave
    constexpr int WCOLS = TN / 2;                        // columns per wave
    constexpr int CODE_PIECES = (GM + TN) / 8 / GWAVES;  // 1 KiB code pieces per wave and step, averaged over two steps (8 or 6)
    static_assert(CODE_PIECES * GWAVES * 8 == GM + TN, "pieces are spread evenly");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    const int n_lane = lane & 31, hh = lane >> 5;
    const int rowbytes = K / 2, G = (K + 255) / 256;  // G: scale tiles per row of tiles
    const int nk = (K + GK - 1) / GK;      // the last step is a half step when K % 256 == 128
    const bool half_last = (K % GK) != 0;

    const __amdgpu_buffer_rsrc_t ra = raw_rsrc(a_codes, (uint32_t)((int64_t)M * rowbytes));
    const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w_codes, (uint32_t)((int64_t)N * rowbytes));
    const __amdgpu_buffer_rsrc_t rsa = raw_rsrc(a_scales, (uint32_t)mx_scale_size(M, K));
    const __amdgpu_buffer_rsrc_t rsw = raw_rsrc(w_scales, (uint32_t)mx_scale_size(N, K));

    // One wave of each SIMD issues a step's copies: waves 0-3 those of even
    // steps, waves 4-7 those of odd ones (waves w and w + 4 share a SIMD).
    // Issuing a copy holds up the wave's next instructions, so while one wave
    // of the SIMD issues them the other keeps the matrix core busy (all eight
    // waves issuing their share at once: 263.9 -> 250.3 us, outputs identical).
    // Code pieces of a copying wave w4 = wave & 3: pieces w4 + 4 j of the
    // step's (GM + TN) / 8 (A: 0..31, then W); their per-lane offsets are
    // recomputed at each step (a few integer ops) to spare registers.
    // Scale pieces (four 32-row scale tiles, 1 KiB): w4 = 0 and 1 copy piece
    // q = wave & 1 of A, w4 = 2 .. 2 + TN / 128 - 1 piece q of W; piece q
    // covers the operand's row tiles 4 q .. 4 q + 3 and lane l brings 16-byte
    // chunk l % 16 of tile 4 q + l / 16 (row tiles past the matrix repeat its
    // last one, never stored).  The step adds kk * 256 bytes.
    const int w4 = wave & 3;
    const bool scale_copier = w4 < 2 + TN / 128, scale_of_a = w4 < 2;
    int soff = 0;
    {
        const int q = wave & 1, t = 4 * q + (lane >> 4);
        const int rt0 = (scale_of_a ? m0 : n0) / 32, nrt = ((scale_of_a ? M : N) + 31) / 32;
        soff = min(rt0 + t, nrt - 1) * G * 256 + (lane & 15) * 16;
    }

    auto copy_stage = [&](int kk, GStage& d) {
        if ((wave >> 2) != (kk & 1)) return;  // wave-uniform: waves 0-3 copy even steps, 4-7 odd ones
        if (scale_copier) {  // wave-uniform
            if (scale_of_a)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsa, (__attribute__((address_space(3))) void*)(d.sa + 64 * (wave & 1)), 16, soff, kk * 256, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsw, (__attribute__((address_space(3))) void*)(d.sw + 64 * (wave & 1)), 16, soff, kk * 256, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2 * CODE_PIECES; ++j) {
            const int p = w4 + (GWAVES / 2) * j;
            if (p < GM / 8)  // wave-uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(d.a + p * 64),
                                                         16, piece_offset(p, lane, m0, M, rowbytes), kk * (GK / 2),
                                                         0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rw, (__attribute__((address_space(3))) void*)(d.w + (p - GM / 8) * 64), 16,
                    piece_offset(p - GM / 8, lane, n0, N, rowbytes), kk * (GK / 2), 0, 0);
        }
    };

    f32x16 acc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};

    // A step's MFMAs must run between its barriers: otherwise the compiler sinks
    // them below the next step's wait for the copies in flight, and memory
    // latency and compute stop overlapping.  settle() (an ordered volatile asm
    // reading every accumulator) and the scheduling fences pin them there.
    // NSUB = 4 MFMA steps per pipeline step, 2 for the half step.
    // issue_copies: the next step's copies, issued once this step's first LDS
    // reads are on their way.
    auto compute = [&](const GStage& t, auto nsub_c, auto&& issue_copies) {
        constexpr int NSUB = decltype(nsub_c)::value;
        __builtin_amdgcn_sched_barrier(0);
        // scale words (mb, word) of this lane's A rows and (nb, word) of its W
        // rows: the row's 8 scale bytes of the step, one 8-byte LDS read each
        uint32_t sa_w[2][2], sw_w[NB][2];
        const uint2* const sa8 = reinterpret_cast<const uint2*>(t.sa);
        const uint2* const sw8 = reinterpret_cast<const uint2*>(t.sw);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const uint2 v = sa8[64 * wm + 32 * mb + n_lane];
            sa_w[mb][0] = v.x;
            sa_w[mb][1] = v.y;
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint2 v = sw8[WCOLS * wn + 32 * nb + n_lane];
            sw_w[nb][0] = v.x;
            sw_w[nb][1] = v.y;
        }
        // Operand fragments: two sets, MFMA step s uses set s & 1.  Step s
        // issues half of its MFMAs, then the reads of step s + 1's fragments,
        // then its other half, so a read has half a step of MFMAs (and the
        // other wave of the SIMD) to land, and the reads into a set issue after
        // half a step of this wave's MFMAs (four; two in a 128-wide tile)
        // behind the last MFMA that reads that set (fenced: the compiler may
        // not hoist the reads further).  Reading them right before their own
        // MFMAs was 2.4-3.5% slower; placing the reads after a quarter or
        // three quarters of the MFMAs, or spreading them over the step, 7-22%
        // slower.
        uint4 fa[2][2], fw[2][NB];
        auto read_frags = [&](int s, uint4 (&a)[2], uint4 (&w)[NB]) {
            const int c = 2 * s + hh;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) a[mb] = t.a[swz(64 * wm + 32 * mb + n_lane, c)];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) w[nb] = t.w[swz(WCOLS * wn + 32 * nb + n_lane, c)];
        };
        read_frags(0, fa[0], fw[0]);
        __builtin_amdgcn_sched_barrier(0);
        issue_copies();
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            // MFMA step s covers blocks 2 s and 2 s + 1: word s >> 1, bytes 2 (s & 1) + hh
            int sca[2], scw[NB];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) sca[mb] = (int)(sa_w[mb][s >> 1] >> (8 * hh));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) scw[nb] = (int)(sw_w[nb][s >> 1] >> (8 * hh));
#pragma unroll
            for (int nb = 0; nb < NB / 2; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = mfma_fp4(fw[s & 1][nb], fa[s & 1][mb], acc[nb][mb], scw[nb], sca[mb], 2 * (s & 1));
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < NSUB) read_frags(s + 1, fa[(s + 1) & 1], fw[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int nb = NB / 2; nb < NB; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = mfma_fp4(fw[s & 1][nb], fa[s & 1][mb], acc[nb][mb], scw[nb], sca[mb], 2 * (s & 1));
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) settle(acc[nb][mb]);
        __builtin_amdgcn_sched_barrier(0);
    };

    // Step i: wait for its copies (the only ones in flight), barrier (every
    // wave's pieces have landed, and every wave is done with the stage step
    // i + 1 will overwrite), read step i's scales and first fragments, issue
    // step i + 1's copies, compute step i (issuing the copies after those
    // reads instead of before: 265.0 -> 259.6 us, outputs identical).  __syncthreads()
    // serves: its fence waits for outstanding memory operations, and at the
    // barrier those are exactly the copies step i needs.  Full steps run in the
    // loop; a final half step (K % 256 == 128) has its own copy of the code, as
    // one shared step with both variants behind a branch exhausts the registers.
    copy_stage(0, st0);
    auto step = [&](int i, const GStage& cur, GStage& nxt, auto nsub_c) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        compute(cur, nsub_c, [&] { if (i + 1 < nk) copy_stage(i + 1, nxt); });
    };
    const std::integral_constant<int, 4> full_step;
    const std::integral_constant<int, 2> half_step;
    const int nfull = half_last ? nk - 1 : nk;
    int i = 0;
    for (; i + 2 <= nfull; i += 2) {
        step(i, st0, st1, full_step);
        step(i + 1, st1, st0, full_step);
    }
    if (i < nfull) {
        step(i, st0, st1, full_step);
        ++i;
    }
    if (half_last) {  // step i = nk - 1 lives in stage i & 1
        if (i & 1)
            step(i, st1, st0, half_step);
        else
            step(i, st0, st1, half_step);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) settle(acc[nb][mb]);

    // acc[nb][mb]: lane (n_lane, hh), register r holds C[m][n .. n+3] with
    // m = m0 + 64 wm + 32 mb + n_lane, n = n0 + WCOLS wn + 32 nb + 8 (r >> 2) + 4 hh + (r & 3).
    // The wave's 64 x WCOLS block (rows of TN bytes = QPR 16-byte chunks)
    // leaves through LDS (64 TN bytes per wave in the stages, free once every
    // wave is past its last step), so each store instruction covers whole row
    // segments instead of 32 rows: row rho keeps chunk c (columns 8c..8c+7) in
    // slot c ^ (rho % QPR), which spreads both the 8-byte writes (32 rows per
    // lane group) and the 16-byte reads (the chunks of a row) over the LDS
    // banks.  16-byte stores when every row starts 16-byte aligned (half the
    // store instructions of 8-byte ones: 251.8 -> 246.1 us at 16896 x 9216 x
    // 3072, outputs identical), else 8-byte stores of the same slots.
    constexpr int PPR = TN / 8;         // 8-byte pieces per row
    constexpr int QPR = TN / 16;        // 16-byte chunks per row
    auto slot = [&](int rho, int piece) { return rho * TN + (((piece >> 1) ^ (rho & (QPR - 1))) << 4) + ((piece & 1) << 3); };
    __syncthreads();
    char* const blk = reinterpret_cast<char*>(wave < 4 ? &st0 : &st1) + (wave & 3) * (64 * TN);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int rho = 32 * mb + n_lane, piece = 8 * nb + 2 * gq + hh;
                const f32x16& c = acc[nb][mb];
                *reinterpret_cast<uint2*>(blk + slot(rho, piece)) =
                    make_uint2(pack_bf16x2(c[4 * gq], c[4 * gq + 1]), pack_bf16x2(c[4 * gq + 2], c[4 * gq + 3]));
            }
    if ((N & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        constexpr int RPQ = 64 / QPR;   // rows per 16-byte store instruction
        uint4* const out16 = reinterpret_cast<uint4*>(out);
#pragma unroll
        for (int i = 0; i < QPR; ++i) {
            const int rho = RPQ * i + lane / QPR, ch = lane & (QPR - 1);
            const int m = m0 + 64 * wm + rho, n = n0 + WCOLS * wn + 8 * ch;
            const uint4 v = *reinterpret_cast<const uint4*>(blk + rho * TN + ((ch ^ (rho & (QPR - 1))) << 4));
            if (m < M && n < N) out16[(int64_t)m * (N / 8) + n / 8] = v;
        }
    } else {
        constexpr int RPI = 64 / PPR;   // rows per 8-byte store instruction
#pragma unroll
        for (int i = 0; i < PPR; ++i) {
            const int rho = RPI * i + lane / PPR, piece = lane & (PPR - 1);
            const int m = m0 + 64 * wm + rho, n = n0 + WCOLS * wn + 4 * piece;
            const uint2 v = *reinterpret_cast<const uint2*>(blk + slot(rho, piece));
            if (m < M && n < N) out[(int64_t)m * (N / 4) + n / 4] = v;
        }
    }
}

// The launch: tiles of 256 x 256 in full rounds of the 256 CUs, and when the
// last round would be at most half full (rem <= 128 tiles) its tiles run as
// 2 rem tiles of 256 x 128 instead, which end in about half the time.  The
// half tiles are dispatched first: the CUs that take one then run half a tile
// out of phase with the others for the rest of the launch, so the tiles'
// output stores and first copies come in two waves instead of one burst per
// round (267 -> 261 us at 16896 x 9216 x 3072).
struct GemmPlan {
    int tiles, nbig, halves;
};
inline GemmPlan gemm_plan(int M, int N) {
    GemmPlan g;
    g.tiles = ((M + GM - 1) / GM) * ((N + GN - 1) / GN);
    const int rem = g.tiles % MI355X_CUS;
    const bool split = rem > 0 && rem <= MI355X_CUS / 2;
    g.nbig = split ? g.tiles - rem : g.tiles;
    g.halves = split ? 2 * rem : 0;
    return g;
}

// Tile order: groups of G_GROUP column tiles, row tiles fastest-but-one
// inside a group (logical r -> row tile r / gw, column tile r % gw), and
// each XCD a contiguous range of the order.  The ~32 workgroups an XCD runs
// at once then cover 4 row tiles x 8 column tiles: the group's W tiles stay
// in that XCD's L2 while it sweeps down the rows.  Logical tiles from nbig
// on are the half-tile ones (two workgroups each, the first gridDim - nbig
// workgroups of the launch).
__global__ __launch_bounds__(GWAVES * 64) void mxfp4_gemm_kernel(const uint8_t* __restrict__ a_codes,
                                                                const uint8_t* __restrict__ a_scales,
                                                                const uint8_t* __restrict__ w_codes,
                                                                const uint8_t* __restrict__ w_scales,
                                                                uint2* __restrict__ out, int M, int N, int K,
                                                                int nbig) {
    // two distinct stage objects, statically indexed (the loop is unrolled by
    // two), so the compiler never makes an LDS read wait for the copy in flight
    __shared__ GStage st0, st1;
    const int m_tiles = (M + GM - 1) / GM, n_tiles = (N + GN - 1) / GN;
    const int halves = (int)gridDim.x - nbig;
    const bool big = (int)blockIdx.x >= halves;
    const int h = (int)blockIdx.x;
    const int logical = big ? xcd_remap((int)blockIdx.x - halves, nbig) : nbig + (h >> 1);
    const int g = logical / (G_GROUP * m_tiles);
    const int gw = min(G_GROUP, n_tiles - g * G_GROUP);
    const int r = logical - g * G_GROUP * m_tiles;
    const int m0 = (r / gw) * GM;
    const int n0 = (g * G_GROUP + r % gw) * GN;
    if (big) {
        gemm_tile<256>(a_codes, a_scales, w_codes, w_scales, out, M, N, K, m0, n0, st0, st1);
    } else {
        const int n0h = n0 + 128 * (h & 1);
        if (n0h >= N) return;  // the whole workgroup: a half past the matrix
        gemm_tile<128>(a_codes, a_scales, w_codes, w_scales, out, M, N, K, m0, n0h, st0, st1);
    }
}

hipError_t launch_mxfp4_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                             void* out, int M, int N, int K, hipStream_t stream) {
    const GemmPlan g = gemm_plan(M, N);
    mxfp4_gemm_kernel<<<g.nbig + g.halves, GWAVES * 64, 0, stream>>>(
        static_cast<const uint8_t*>(a_codes), static_cast<const uint8_t*>(a_scales),
        static_cast<const uint8_t*>(w_codes), static_cast<const uint8_t*>(w_scales), static_cast<uint2*>(out), M,
        N, K, g.nbig);
    return hipGetLastError();
}

}  // namespace dit
