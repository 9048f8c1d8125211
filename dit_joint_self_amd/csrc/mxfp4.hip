// mxfp4.hip - MXFP4 (OCP Microscaling) activation quantisation and the
// block-scaled A4W4 GEMM of the DiT linear layers, gfx950.
//
// The MXFP4/Quark on MI350 blog quantises FLUX's linear layers to MXFP4 as
// the OCP MX specification defines it (section "MXFP4 Quantization": 32 FP4
// elements share one E8M0 scale; weights static, activations dynamic, blocks
// along the reduction axis), and runs them as an activation quantisation
// kernel plus an A4W4 matrix-core GEMM (section "MXFP4 Kernel").
//
// Formats (row-major, shared by the quantiser and the GEMM):
//   codes  [R, K/2] bytes: element k of a row in byte k/2, low nibble for even
//          k; E2M1 = sign, 2 exponent bits (bias 1), 1 mantissa bit.
//   scales [R, K/32] bytes: E8M0 biased exponent of each 32-element block.
//
// Quantisation of a block V (the MX rule): X = floor(log2 max|V|) - 2 (the
// largest E2M1 exponent), clamped to [-127, 127] (an all-zero block takes
// -127); P_i = V_i * 2^-X rounded to the nearest E2M1 value, ties to the even
// code, magnitudes above 6 saturated to 6, sign bit kept.  Every step is
// exact in fp32 (bf16 inputs, power-of-two scaling, comparisons against the
// midpoints), so the codes do not depend on evaluation order.
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

#include "attn_common.h"
#include "bf16_util.h"

namespace dit {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- quantiser

// Thread t: elements 8t .. 8t+7 of the flattened [R, K] input (K % 32 == 0, so
// 4 consecutive lanes hold one block).  Grid-stride.
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const uint4* __restrict__ x,
                                                             uint32_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, int64_t groups) {
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
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float y = fabsf(ldexpf(v[i], -X));
            // number of rounding midpoints passed; a tie goes to the even code
            uint32_t c = (y > 0.25f) + (y >= 0.75f) + (y > 1.25f) + (y >= 1.75f) + (y > 2.5f) + (y >= 3.5f) +
                         (y > 5.0f);
            c |= (__float_as_uint(v[i]) >> 28) & 8u;   // sign bit
            packed |= c << (4 * i);
        }
        codes[t] = packed;
        if ((t & 3) == 0) scales[t >> 2] = (uint8_t)(X + 127);
    }
}

hipError_t launch_mxfp4_quantize(const void* x, void* codes, void* scales, int64_t rows, int K,
                                 hipStream_t stream) {
    const int64_t groups = rows * (K / 8);
    const int64_t blocks = std::min<int64_t>((groups + 255) / 256, (int64_t)MI355X_CUS * 32);
    mxfp4_quantize_kernel<<<(int)blocks, 256, 0, stream>>>(static_cast<const uint4*>(x),
                                                           static_cast<uint32_t*>(codes),
                                                           static_cast<uint8_t*>(scales), groups);
    return hipGetLastError();
}

// ---------------------------------------------------------------- GEMM

constexpr int GM = 128;  // rows of A (output rows) per workgroup
constexpr int GN = 256;  // rows of W (output columns) per workgroup
constexpr int GK = 128;  // K per pipeline step (two 64-deep MFMA steps, four MX blocks)

// LDS image of a tile: rows of GK/2 = 64 bytes = four 16-byte chunks; chunk c
// of row r sits at position c ^ ((r >> 2) & 3), so the 16 lanes of an LDS read
// quarter (rows r .. r+15, one chunk each) hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Per-lane global byte offset of the chunk that lane `lane` of copy piece p
// brings in: LDS chunk 64 p + lane = (row, position), global chunk = position
// un-swizzled.  Rows past the matrix repeat its last row (never stored).
__device__ __forceinline__ int piece_offset(int p, int lane, int row0, int rows, int rowbytes) {
    const int i = p * 64 + lane;
    const int r = i >> 2, q = i & 3;
    const int c = q ^ ((r >> 2) & 3);
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

// Workgroup: 4 waves, wave (wm, wn) = (w & 1, w >> 1) computes output rows
// m0 + 64 wm .. +63 and columns n0 + 128 wn .. +127 as 2 x 4 blocks of 32 x 32
// (accumulators acc[nb][mb] of C^T).
__global__ __launch_bounds__(256, 2) void mxfp4_gemm_kernel(const uint8_t* __restrict__ a_codes,
                                                         const uint8_t* __restrict__ a_scales,
                                                         const uint8_t* __restrict__ w_codes,
                                                         const uint8_t* __restrict__ w_scales,
                                                         uint2* __restrict__ out, int M, int N, int K) {
    __shared__ uint4 sa0[GM * 4];
    __shared__ uint4 sa1[GM * 4];
    __shared__ uint4 sw0[GN * 4];
    __shared__ uint4 sw1[GN * 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const int n_tiles = (N + GN - 1) / GN;
    const int m0 = (blockIdx.x / n_tiles) * GM;
    const int n0 = (blockIdx.x % n_tiles) * GN;
    const int rowbytes = K / 2, srow = K / 32;
    const int nk = K / GK;

    const __amdgpu_buffer_rsrc_t ra = raw_rsrc(a_codes, (uint32_t)((int64_t)M * rowbytes));
    const __amdgpu_buffer_rsrc_t rw = raw_rsrc(w_codes, (uint32_t)((int64_t)N * rowbytes));
    // copy pieces of this wave: A pieces wave, wave + 4 (of 8); W pieces wave + 4 j (of 16)
    int offa[2], offw[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) offa[j] = piece_offset(wave + 4 * j, lane, m0, M, rowbytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) offw[j] = piece_offset(wave + 4 * j, lane, n0, N, rowbytes);
    auto copy_tile = [&](int kk, uint4* da, uint4* dw) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(da + (wave + 4 * j) * 64),
                                                     16, offa[j], kk * (GK / 2), 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(dw + (wave + 4 * j) * 64),
                                                     16, offw[j], kk * (GK / 2), 0, 0);
    };

    // scale rows of this lane: output rows (B operand) and columns (A operand)
    const int n_lane = lane & 31, hh = lane >> 5;
    const uint8_t* sa_row[2];
    const uint8_t* sw_row[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sa_row[mb] = a_scales + (int64_t)min(m0 + 64 * wm + 32 * mb + n_lane, M - 1) * srow;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) sw_row[nb] = w_scales + (int64_t)min(n0 + 128 * wn + 32 * nb + n_lane, N - 1) * srow;
    // the four block scales of step kk, shifted so byte 0 / byte 2 belong to this lane's K-half
    auto load_scales = [&](int kk, uint32_t (&sa)[2], uint32_t (&sw)[4]) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sa[mb] = *reinterpret_cast<const uint32_t*>(sa_row[mb] + 4 * kk);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) sw[nb] = *reinterpret_cast<const uint32_t*>(sw_row[nb] + 4 * kk);
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};

    // A step's MFMAs must run between its barriers: otherwise the compiler sinks
    // them below the next step's wait for the copies in flight, and memory
    // latency and compute stop overlapping.  settle() (an ordered volatile asm
    // reading every accumulator) and the scheduling fences pin them there.
    auto compute = [&](const uint4* ta, const uint4* tw, const uint32_t (&sa)[2], const uint32_t (&sw)[4]) {
        __builtin_amdgcn_sched_barrier(0);
        int sca[2], scw[4];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) sca[mb] = (int)(sa[mb] >> (8 * hh));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) scw[nb] = (int)(sw[nb] >> (8 * hh));
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 2 * s + hh;
            uint4 fa[2], fw[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) fa[mb] = ta[swz(64 * wm + 32 * mb + n_lane, c)];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) fw[nb] = tw[swz(128 * wn + 32 * nb + n_lane, c)];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    acc[nb][mb] = mfma_fp4(fw[nb], fa[mb], acc[nb][mb], scw[nb], sca[mb], 2 * s);
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) settle(acc[nb][mb]);
        __builtin_amdgcn_sched_barrier(0);
    };

    uint32_t sa_0[2], sw_0[4], sa_1[2], sw_1[4];
    copy_tile(0, sa0, sw0);
    load_scales(0, sa_0, sw_0);
    int kk = 0;
    for (; kk + 2 <= nk; kk += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        copy_tile(kk + 1, sa1, sw1);
        load_scales(kk + 1, sa_1, sw_1);
        compute(sa0, sw0, sa_0, sw_0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kk + 2 < nk) {
            copy_tile(kk + 2, sa0, sw0);
            load_scales(kk + 2, sa_0, sw_0);
        }
        compute(sa1, sw1, sa_1, sw_1);
    }
    if (kk < nk) {  // odd number of steps: the last one is in buffer 0
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        compute(sa0, sw0, sa_0, sw_0);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) settle(acc[nb][mb]);

    // acc[nb][mb]: lane (n_lane, hh), register r holds C[m][n .. n+3] with
    // m = m0 + 64 wm + 32 mb + n_lane, n = n0 + 128 wn + 32 nb + 8 (r >> 2) + 4 hh + (r & 3).
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 64 * wm + 32 * mb + n_lane;
        if (m >= M) continue;
        uint2* orow = out + (int64_t)m * (N / 4);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + 128 * wn + 32 * nb + 8 * g + 4 * hh;
                if (n < N) {
                    const f32x16& c = acc[nb][mb];
                    orow[n / 4] = make_uint2(pack_bf16x2(c[4 * g], c[4 * g + 1]), pack_bf16x2(c[4 * g + 2], c[4 * g + 3]));
                }
            }
    }
}

hipError_t launch_mxfp4_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                             void* out, int M, int N, int K, hipStream_t stream) {
    const int64_t grid = (int64_t)((M + GM - 1) / GM) * ((N + GN - 1) / GN);
    mxfp4_gemm_kernel<<<(int)grid, 256, 0, stream>>>(
        static_cast<const uint8_t*>(a_codes), static_cast<const uint8_t*>(a_scales),
        static_cast<const uint8_t*>(w_codes), static_cast<const uint8_t*>(w_scales), static_cast<uint2*>(out), M,
        N, K);
    return hipGetLastError();
}

}  // namespace dit
