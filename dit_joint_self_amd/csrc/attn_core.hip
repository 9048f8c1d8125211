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
//   * Q prologue: coalesced loads of the Q rows and their cos/sin rows (each
//     load covers whole cache lines), RoPE and the factor scale*log2(e) in
//     fp32, then through LDS into the MFMA B-operand layout, where the bf16
//     Q' tile stays for the whole kernel (Q-tile resident in VGPRs).
//   * K/V stream: 64-key tiles, K' already rotated and laid out by
//     prepare_kv.hip, V straight from the caller's tensor; both copied
//     HBM -> LDS by buffer_load_dwordx4 ... lds into four K' and four V
//     buffers (K' three tiles ahead, V two), one barrier per two tiles; the
//     copies of a step are issued one at a time between its MFMAs.
//   * Software pipeline per wave: the QK^T MFMAs of tile j+1 run beside the
//     exp2 / bf16 / row-sum work of tile j, then O += P V for tile j.
//   * S^T = K' Q'^T on v_mfma_f32_32x32x16_bf16: lane (n, hh) of the
//     accumulator owns query n and 16 keys, so a row max is in-lane max ops
//     plus one v_permlane32_swap, and the row sum stays per lane until the
//     epilogue.
//   * Online softmax in base 2 with a lazily moved offset: the offset m is
//     folded into the QK^T accumulator's initial value, the row max is only
//     taken for the first tile and when a tile's weights overflow 2^20, and
//     the row sum is accumulated from the bf16 weights with v_dot2c (see
//     weight_pair and settle_weights).  Weights stay <= 2^20, so fp32 and bf16 hold them with
//     their usual relative precision, and the final O / l is unchanged.
//   * O^T += V^T P^T on the same MFMA: P leaves the S accumulator already in
//     B-operand layout (see tile_layout.h); the V^T A operand is read from
//     the key-major V tile with the transposing LDS read ds_read_b64_tr_b16.
//   * Epilogue: combine the two half-wave partial sums, scale by 1/l, round to
//     bf16, and store rows < S through LDS, so the stores are coalesced.
//
// Roofline: MFMA bound.  Algorithmic work per (query block of BM rows, head):
// 4 * BM * S * 128 flop; per call 4 * B * H * S^2 * 128 flop.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_common.h"
#include "bf16_util.h"
#include "tile_layout.h"

namespace dit {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// One 64-key tile step of the software-pipelined loop.
//
// Softmax bookkeeping (base 2, per query): m is the offset subtracted before
// exp2 and l the running sum of the bf16 weights.  negm holds -m in all 16
// registers of the lane's accumulator shape and enters as the C operand of the
// first QK^T MFMA, so the scores arrive already offset.  m is exact (the row
// max) after the first tile; afterwards it is only raised when a tile's
// weights sum past SUM_LIMIT in some lane (so no weight exceeds 2^20): then
// the tile's row max is taken, O and l are scaled by 2^(m_old - m_new) and the
// tile's weights are redone.  The final O / l does not depend on when m moves.
//
// Pipelining: while the matrix cores compute the NEXT tile's scores, the VALU
// turns the CURRENT tile's scores into weights (stage A, 16 fenced steps of
// one MFMA + one score pair each); then O^T += V^T P^T for the current tile
// (stage B).  The next tile's scores were offset with the m in force before
// stage A, so a move of m in between is applied to them too.
constexpr float SUM_LIMIT = 1048576.0f;  // 2^20

// MFMA operand ring: LDS reads run RING - 1 MFMA steps ahead of their use.
constexpr int RING = 6;

// K' operand of QK^T step i (dim step i >> 1, key block i & 1), for lane (n, hh).
__device__ __forceinline__ bf16x8 k_operand(const uint4* kt, int i, int n, int hh) {
    return as_bf16x8(kt[k_chunk((i & 1) * 32 + n, 2 * (i >> 1) + hh)]);
}

// V^T operand of PV step i (16-key step u = i >> 2, dim block db = i & 3):
// lane (n, hh) needs V[16u + 8hh + t][32 db + n], t = 0..7, as bf16x8.  Two
// ds_read_b64_tr_b16 (t = 0..3, then 4..7): in each 16-lane group (lanes 16g
// .. 16g + 15: n0 = 16 (g & 1), hh = g >> 1) the transposing read hands
// result lane i the element i % 4 of source lanes i / 4 + 4 j, j = 0..3, so
// source lane s = 4 j + a reads the four dims 32 db + n0 + 4a .. + 3 of key
// 16u + 8hh + 4h + j.  `vlane` is the lane's byte offset for u = db = h = 0
// (v_lane_offset); the rest is a compile-time offset.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ int v_lane_offset(int lane) {
    const int g = lane >> 4, s = lane & 15;
    return v_lds_byte(8 * (g >> 1) + (s >> 2), 16 * (g & 1) + 4 * (s & 3));
}
__device__ __forceinline__ bf16x8 v_operand(const uint4* vt, int i, int vlane) {
    const int u = i >> 2, db = i & 3;
    const char* base = reinterpret_cast<const char*>(vt) + vlane + u * V_ROW_BYTES + 64 * db;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 4 * V_PIECE_BYTES));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, w);
}

// Two weights of score pair p (0..15) of the current tile: pair p of key
// block p >> 3 holds registers 2 (p & 7) and 2 (p & 7) + 1.  w[p] is the bf16
// pair; its sum (v_dot2c against (1, 1)) is added to `sum`, so l sums exactly
// the weights the PV product uses.
__device__ __forceinline__ void weight_pair(const f32x16 (&sc)[2], int p, uint32_t (&w)[16], float& sum) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const f32x16& a = sc[p >> 3];
    const int r = 2 * (p & 7);
    w[p] = pack_bf16x2(__builtin_amdgcn_exp2f(a[r]), __builtin_amdgcn_exp2f(a[r + 1]));
    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[p]), ones, sum, false);
    // Pin the pair here.  The steps that issue tile copies end in a branch;
    // without the pin the compiler sinks those steps' exp2 work past the
    // branches and runs it in one burst after the last copy, instead of one
    // pair beside each score MFMA.  The empty asm emits no instruction.
    asm volatile("" : "+v"(w[p]), "+v"(sum));
}

// Piece p of a V tile: lane l moves 16 bytes of key p + 16 (l >> 4), chunk
// l & 15, from V (tile byte offset vtoff) to the piece's l-th LDS chunk.
// vgather is the lane's source offset inside the tile for p = 0
// (v_gather_offset); rows past S read as zeros.
__device__ __forceinline__ int v_gather_offset(int lane) { return (lane >> 4) * 16 * V_ROW_BYTES + (lane & 15) * 16; }
__device__ __forceinline__ void v_piece(__amdgpu_buffer_rsrc_t vrsrc, int vtoff, int p, uint4* vdst, int vgather) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vrsrc, (__attribute__((address_space(3))) void*)(vdst + p * V_PIECE_CHUNKS),
                                             16, vgather, vtoff + p * V_ROW_BYTES, 0, 0);
}

// The tile copies one pipelined step issues, spread over stage A: piece j of
// the K' part three tiles ahead at step 2j + 1, piece j of the V tile two
// tiles ahead at step 2 (KJ + j) + 1.  Issued one at a time between MFMAs
// instead of in a burst after the barrier, the copies do not hold up the
// wave's first MFMAs.
struct TileCopies {
    static constexpr int KJ = (K_PART_CHUNKS / 64 + NW - 1) / NW;  // K' pieces per wave (at most)
    static constexpr int VJ = (V_PIECES + NW - 1) / NW;            // V pieces per wave (at most)
    __amdgpu_buffer_rsrc_t krsrc, vrsrc;
    int ksoff, vsoff;  // byte offsets of the K' tile in the workspace slice, of the V tile in the head's V
    uint4* kdst;
    uint4* vdst;
    bool kon;          // the K' tile exists (wave-uniform)
    bool von;          // the V tile exists (wave-uniform)
    int wave, lane, vgather;
    __device__ __forceinline__ void at_step(int i) const {
        if ((i & 1) == 0) return;
        const int j = i >> 1;
        if (j < KJ) {
            const int p = j * NW + wave;
            if (kon && p < K_PART_CHUNKS / 64) lds_piece(krsrc, ksoff + p * 1024, kdst + p * 64, lane);
        } else if (j < KJ + VJ) {
            const int p = (j - KJ) * NW + wave;
            if (von && p < V_PIECES) v_piece(vrsrc, vsoff, p, vdst, vgather);
        }
    }
};
static_assert(2 * (TileCopies::KJ + TileCopies::VJ) <= 16, "the copies fit in the 16 steps of stage A");

// Stage A: QK MFMA step i of the next tile (K' part kn) with weight pair i of
// the current tile, and the step's share of the tile copies (cp may be null).
// QK = false: weights only (the range's last tile); EXP = false: scores only
// (the range's first tile, before the loop).
template <bool QK, bool EXP>
__device__ __forceinline__ void stage_a(const uint4* kn, const bf16x8 (&qf)[8], const f32x16& negm,
                                        f32x16 (&sn)[2], const f32x16 (&sc)[2], uint32_t (&w)[16], float& sum,
                                        int n, int hh, const TileCopies* cp = nullptr) {
    bf16x8 ring[RING];
    if (QK) {
#pragma unroll
        for (int i0 = 0; i0 < RING - 1; ++i0) ring[i0] = k_operand(kn, i0, n, hh);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (QK && i + RING - 1 < 16) ring[(i + RING - 1) % RING] = k_operand(kn, i + RING - 1, n, hh);
        __builtin_amdgcn_sched_barrier(0);
        if (QK)
            sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % RING], qf[i >> 1],
                                                                (i >> 1) == 0 ? negm : sn[i & 1], 0, 0, 0);
        if (EXP) weight_pair(sc, i, w, sum);
        if (cp) cp->at_step(i);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Row max of a tile's offset scores (all 64 keys: both lane halves).
__device__ __forceinline__ float tile_max(const f32x16 (&sc)[2]) {
    float mx = sc[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[1][r]);
    return swap_halves_max(mx);
}

// Keys past S (a no-op unless tile j is the sequence's ragged last tile).
// Lane half hh, register r of key block kb holds key 32 kb + 16 (r >> 3) +
// 8 hh + (r & 7) of the tile.
__device__ __forceinline__ void mask_tail(f32x16 (&sc)[2], int j, int S, int hh) {
    if ((j + 1) * KV_TILE <= S) return;          // a whole tile (wave-uniform)
    const int lim = S - (j * KV_TILE + 8 * hh);  // the lane's key offsets >= lim are past S
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (32 * kb + 16 * (r >> 3) + (r & 7) >= lim) sc[kb][r] = -INFINITY;
}

// Between the stages: move m if this tile's weights overflow, then add the
// tile's weight sum to l.  (The first tile's offset is set to its exact row
// max before the loop, so the weights computed in stage A are always the ones
// used on the fast path.)
template <bool QK>
__device__ __forceinline__ void settle_weights(f32x16 (&sc)[2], f32x16 (&sn)[2], uint32_t (&w)[16], float sum,
                                               f32x16 (&o)[4], f32x16& negm, float& lsum) {
    if (__builtin_amdgcn_ballot_w64(!(sum <= SUM_LIMIT)) != 0) {
        const float shift = fmaxf(tile_max(sc), 0.0f);
        const float alpha = __builtin_amdgcn_exp2f(-shift);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
        sc[0] -= shift;
        sc[1] -= shift;
        negm -= shift;
        if (QK) {
            sn[0] -= shift;
            sn[1] -= shift;
        }
        sum = 0.0f;
#pragma unroll
        for (int p = 0; p < 16; ++p) weight_pair(sc, p, w, sum);
    }
    lsum += sum;
}

// Stage B: O^T += V^T P^T over the tile's 64 keys (V tile vt): 16 MFMA steps;
// the weights of 16-key step u are w[4u .. 4u + 3], already in B-operand order.
__device__ __forceinline__ void stage_b(const uint4* vt, const uint32_t (&w)[16], f32x16 (&o)[4], int vlane) {
    bf16x8 pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pf[u] = as_bf16x8(make_uint4(w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]));
    bf16x8 ring[RING];
#pragma unroll
    for (int i0 = 0; i0 < RING - 1; ++i0) ring[i0] = v_operand(vt, i0, vlane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i + RING - 1 < 16) ring[(i + RING - 1) % RING] = v_operand(vt, i + RING - 1, vlane);
        __builtin_amdgcn_sched_barrier(0);
        o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[i % RING], pf[i >> 2], o[i & 3], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// A tile with a successor: scores sc (current), sn (next, written), K' tile of
// the next tile kn, V tile of the current tile vt, copies cp.
__device__ __forceinline__ void tile_step(const uint4* kn, const uint4* vt, f32x16 (&sc)[2], f32x16 (&sn)[2],
                                          const bf16x8 (&qf)[8], f32x16 (&o)[4], f32x16& negm, float& lsum, int n,
                                          int hh, int vlane, const TileCopies& cp) {
    uint32_t w[16];
    float sum = 0.0f;
    stage_a<true, true>(kn, qf, negm, sn, sc, w, sum, n, hh, &cp);
    settle_weights<true>(sc, sn, w, sum, o, negm, lsum);
    stage_b(vt, w, o, vlane);
}

// The range's last tile (index j), masked.
__device__ __forceinline__ void tile_step_last(const uint4* vt, f32x16 (&sc)[2], int j, int S,
                                               const bf16x8 (&qf)[8], f32x16 (&o)[4], f32x16& negm, float& lsum,
                                               int n, int hh, int vlane) {
    mask_tail(sc, j, S, hh);
    uint32_t w[16];
    float sum = 0.0f;
    f32x16 none[2];
    stage_a<false, true>(nullptr, qf, negm, none, sc, w, sum, n, hh);
    settle_weights<false>(sc, none, w, sum, o, negm, lsum);
    stage_b(vt, w, o, vlane);
}

// One workgroup = BM queries of one (batch, head) against the key tiles
// [tb, te) (core_work: whole-range items first, then the key-range pieces of
// the `split` items).  Whole range: normalised bf16 output.  Key range:
// unnormalised O, m and l of the range to `part`, merged afterwards.
__global__ __launch_bounds__(NW * 64) void attn_core_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ v, const float4* __restrict__ cos_t,
    const float4* __restrict__ sin_t, const uint4* __restrict__ ws, uint2* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part, int* __restrict__ ctl, int S, int ntiles, int nqt, int full, int nsplit,
    int pool_whole, float qmul, int has_rope) {
    static_assert(QB == 1, "one 32-query block per wave");
    // Tile t's K' part lives in kbuf[t % 4] and its V rows in vbuf[t % 4]
    // (136 KiB of LDS).  Distinct objects and a loop unrolled by four keep
    // every buffer static, so the compiler does not make LDS reads wait for
    // the copies.
    __shared__ uint4 kb0[K_PART_CHUNKS];
    __shared__ uint4 kb1[K_PART_CHUNKS];
    __shared__ uint4 kb2[K_PART_CHUNKS];
    __shared__ uint4 kb3[K_PART_CHUNKS];
    __shared__ uint4 vb0[V_LDS_CHUNKS];
    __shared__ uint4 vb1[V_LDS_CHUNKS];
    __shared__ uint4 vb2[V_LDS_CHUNKS];
    __shared__ uint4 vb3[V_LDS_CHUNKS];
    uint4* const kbuf[4] = {kb0, kb1, kb2, kb3};
    uint4* const vbuf[4] = {vb0, vb1, vb2, vb3};

    if (DIT_DEBUG_LDS_NAN) {
        for (int b = 0; b < 4; ++b) {
            debug_fill_lds<NW * 64>(kbuf[b], K_PART_CHUNKS);
            debug_fill_lds<NW * 64>(vbuf[b], V_LDS_CHUNKS);
        }
        __syncthreads();
    }

    // Static whole items first, then the pool (see attn_common.h).
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
    const int nt = te - tb;  // >= 1

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 31;
    const int hh = lane >> 5;

    // The (batch, head) slice of prepared K' tiles and the head's V rows as
    // buffer resources; K' tile tb + i starts at byte ktile0 + i * K_PART_BYTES
    // and V tile tb + i at vtile0 + i * KV_TILE * V_ROW_BYTES (both < 2^31 for
    // S <= MAX_SEQ).  V rows at or past S read as zeros.
    const __amdgpu_buffer_rsrc_t krsrc =
        raw_rsrc(ws + bh * (int64_t)ntiles * K_PART_CHUNKS, (uint32_t)ntiles * K_PART_BYTES);
    const __amdgpu_buffer_rsrc_t vrsrc = raw_rsrc(v + bh * (int64_t)S * (V_ROW_BYTES / 16), (uint32_t)S * V_ROW_BYTES);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int ktile0 = tb * K_PART_BYTES;
    const int vtile0 = tb * KV_TILE * V_ROW_BYTES;
    const int vgather = v_gather_offset(lane);
    const int vlane = v_lane_offset(lane);
    auto copies = [&](int ki, uint4* kd, bool kon, int vi, uint4* vd, bool von = true) {
        TileCopies c;
        c.krsrc = krsrc;
        c.vrsrc = vrsrc;
        c.ksoff = ktile0 + ki * K_PART_BYTES;
        c.vsoff = vtile0 + vi * KV_TILE * V_ROW_BYTES;
        c.kdst = kd;
        c.vdst = vd;
        c.kon = kon;
        c.von = von;
        c.wave = wv;
        c.lane = lane;
        c.vgather = vgather;
        return c;
    };
    auto copy_v = [&](int vi, uint4* vd) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TileCopies::VJ; ++i) {
            const int p = i * NW + wv;
            if (p < V_PIECES) v_piece(vrsrc, vtile0 + vi * KV_TILE * V_ROW_BYTES, p, vd, vgather);
        }
    };
    copy_to_lds<NW, K_PART_CHUNKS>(krsrc, ktile0, kb0, wv, lane);
    copy_v(0, vb0);
    if (nt > 1) copy_to_lds<NW, K_PART_CHUNKS>(krsrc, ktile0 + K_PART_BYTES, kb1, wv, lane);
    if (nt > 1) copy_v(1, vb1);
    if (nt > 2) copy_to_lds<NW, K_PART_CHUNKS>(krsrc, ktile0 + 2 * K_PART_BYTES, kb2, wv, lane);

    // ---- Q prologue: RoPE, fold scale*log2(e), round to bf16, keep resident.
    // The loads are coalesced: load i of lane l reads 16-byte chunk
    // 8 (i / 4) + l % 8 of row 8 (i % 4) + l / 8 of the wave's 32 rows, so one
    // load covers the same half of 8 consecutive rows, 8 whole cache lines (a
    // row per lane would touch 32 lines per load).  Chunk c of a Q row holds
    // the RoPE pairs 4c..4c+3, as chunk c of a cos/sin row does, so the
    // rotation runs in that layout.  The rotated chunks reach the MFMA layout
    // (lane (n, hh), register t: chunk 2t + hh of row n) through a 4 KiB area
    // per wave in kb3 / vb2, which no copy touches before the first loop
    // step, in two passes (chunks 0-7 of every row, then chunks 8-15).  Row
    // rho keeps chunk c' of a pass in slot c' ^ ((rho / 2) % 8), so the
    // writes (two rows per 16 lanes) and the reads (16 rows per 16 lanes)
    // both spread over all LDS banks.  Rows past S read row S - 1 and are zeroed.
    bf16x8 qf[8];
    const int rloc = wave * 32 + n;
    const int row = qt * BM + rloc;
    {
        const int row0 = qt * BM + wave * 32;  // the wave's first row
        uint4 qw[8];
        float4 cosw[8], sinw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = row0 + 8 * (i & 3) + (lane >> 3);
            const int c = 8 * (i >> 2) + (lane & 7);
            const int64_t rr = r < S ? r : S - 1;
            qw[i] = q[(bh * S + rr) * 16 + c];
            if (has_rope) {
                cosw[i] = cos_t[rr * 16 + c];
                sinw[i] = sin_t[rr * 16 + c];
            }
        }
        char* const stage =
            (wave < 4 ? reinterpret_cast<char*>(kb3) : reinterpret_cast<char*>(vb2)) + (wave & 3) * 4096;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int i = 4 * pass + i4;
                float fv[8];
                unpack8(qw[i], fv);
                if (has_rope) rotate4(fv, cosw[i], sinw[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) fv[e] *= qmul;
                const int rho = 8 * i4 + (lane >> 3);
                const uint4 pk = row0 + rho < S ? pack8(fv) : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(stage + rho * 128 + (((lane & 7) ^ ((rho >> 1) & 7)) << 4)) = pk;
            }
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) {
                const int slot = (2 * t4 + hh) ^ ((n >> 1) & 7);
                qf[4 * pass + t4] = as_bf16x8(*reinterpret_cast<const uint4*>(stage + n * 128 + (slot << 4)));
            }
        }
    }

    f32x16 o[4], negm = f32x16{};
    float lsum = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] = f32x16{};

    // Scores of tile 0 (offset 0), then the pipelined steps.  Tile t's
    // scores live in s[t % 2].
    f32x16 s[2][2];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    {
        uint32_t w[16];
        float sum = 0.0f;
        stage_a<true, false>(kb0, qf, negm, s[0], s[1], w, sum, n, hh);
    }
    // Offset of the first tile = its exact row max (masked first if it is
    // also the range's last tile, so the max is over real keys only).
    if (nt == 1) mask_tail(s[0], te - 1, S, hh);
    {
        const float mx = tile_max(s[0]);
        s[0][0] -= mx;
        s[0][1] -= mx;
        negm -= mx;
    }
    // One barrier per two tiles.  Tile t's K' part is in kbuf[t % 4], its V^T
    // part in vbuf[t % 4]; step t issues the copies of K'(t + 3) and V^T(t + 2).
    // Between the barriers before steps k and k + 2 (k even) the steps read
    // K'(k + 1), K'(k + 2), V^T(k), V^T(k + 1), all copied before the first of
    // them, and overwrite only parts read before it.
    const int L = nt - 1;
    auto step = [&](auto rc, int k) __attribute__((always_inline)) {
        constexpr int R = decltype(rc)::value;  // k % 4
        if (R % 2 == 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        tile_step(kbuf[(R + 1) % 4], vbuf[R], s[R % 2], s[(R + 1) % 2], qf, o, negm, lsum, n, hh, vlane,
                  copies(k + 3, kbuf[(R + 3) % 4], k + 3 <= L, k + 2, vbuf[(R + 2) % 4], k + 2 <= L));
    };
    for (int k = 0;;) {
        if (k >= L) break;
        step(std::integral_constant<int, 0>{}, k++);
        if (k >= L) break;
        step(std::integral_constant<int, 1>{}, k++);
        if (k >= L) break;
        step(std::integral_constant<int, 2>{}, k++);
        if (k >= L) break;
        step(std::integral_constant<int, 3>{}, k++);
    }
    if ((L & 1) == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }
    // No copy is in flight any more, so the last V tile may be picked at run
    // time; only the score registers need a static choice.
    const uint4* vlast = (L & 2) ? ((L & 1) ? vb3 : vb2) : ((L & 1) ? vb1 : vb0);
    if (L & 1)
        tile_step_last(vlast, s[1], te - 1, S, qf, o, negm, lsum, n, hh, vlane);
    else
        tile_step_last(vlast, s[0], te - 1, S, qf, o, negm, lsum, n, hh, vlane);
#pragma unroll
    for (int db = 0; db < 4; ++db) settle(o[db]);

    // ---- epilogue: lane (n, hh), register r of dim block db holds dim
    // 32 db + 8 (r >> 2) + 4 hh + (r & 3) of query n.  The rows go out
    // through LDS (the tile buffers are free once every wave is past its last
    // tile), so the global stores are coalesced like the Q loads: one store
    // covers 1 KiB of consecutive rows instead of touching 32 cache lines.
    const float l = swap_halves_sum(lsum);
    __syncthreads();
    const int row0 = qt * BM + wave * 32;  // the wave's first row
    if (cw.partial) {
        // fp32 rows of 512 bytes, 16 KiB per wave in buffer `wave`: row n
        // keeps 16-byte piece p (dims 4p..4p+3) in slot p ^ (n % 16).
        uint4* const sb = wave < 4 ? (wave < 2 ? (wave == 0 ? kb0 : kb1) : (wave == 2 ? kb2 : kb3))
                                   : (wave < 6 ? (wave == 4 ? vb0 : vb1) : (wave == 6 ? vb2 : vb3));
        char* const st = reinterpret_cast<char*>(sb);
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int piece = db * 8 + g * 2 + hh;
                *reinterpret_cast<float4*>(st + n * 512 + ((piece ^ (n & 15)) << 4)) =
                    make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
            }
        float* pw = part + (int64_t)cw.piece * PART_FLOATS;
        float4* pwave = reinterpret_cast<float4*>(pw + (int64_t)wave * 32 * HEAD_DIM);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rho = 2 * i + (lane >> 5), c = lane & 31;
            pwave[rho * 32 + c] = *reinterpret_cast<const float4*>(st + rho * 512 + ((c ^ (rho & 15)) << 4));
        }
        if (hh == 0) {
            pw[BM * HEAD_DIM + rloc] = -negm[0];
            pw[BM * HEAD_DIM + BM + rloc] = l;
        }
    } else {
        // Row log-sum-exp of the scaled scores (natural log): the kernel's
        // base-2 scores are scale * log2(e) * q'.k', offset by m, so
        // sum_j exp(scale q'.k_j) = 2^m * l.
        if (lse != nullptr && hh == 0 && row < S) lse[bh * S + row] = LN2 * (-negm[0] + __builtin_amdgcn_logf(l));
        // bf16 rows of 256 bytes, 8 KiB per wave: row n keeps 8-byte piece p
        // (dims 4p..4p+3) in slot p ^ n, so 16-byte chunk c sits in slot
        // c ^ (n / 2), its halves swapped when n is odd.
        uint4* const sb = wave < 4 ? (wave < 2 ? kb0 : kb1) : (wave < 6 ? kb2 : kb3);
        char* const st = reinterpret_cast<char*>(sb) + (wave & 1) * 8192;
        const float inv = 1.0f / l;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int piece = db * 8 + g * 2 + hh;
                *reinterpret_cast<uint2*>(st + n * 256 + ((piece ^ n) << 3)) =
                    make_uint2(pack_bf16x2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                               pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv));
            }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rho = 4 * i + (lane >> 4), c = lane & 15;
            uint4 w = *reinterpret_cast<const uint4*>(st + rho * 256 + ((c ^ (rho >> 1)) << 4));
            if (rho & 1) w = make_uint4(w.z, w.w, w.x, w.y);
            if (row0 + rho < S) reinterpret_cast<uint4*>(out)[(bh * S + row0 + rho) * 16 + c] = w;
        }
    }
    if ((int)blockIdx.x >= nstatic) finish_pool_wg(ctl, pool_wgs);
}

// Combine the nsplit key-range partials of each split item (the same streaming
// softmax merge, exact): M = max m_f, O = sum 2^(m_f - M) O_f / sum 2^(m_f - M) l_f.
// One workgroup per 16 rows of an item; 16 threads per row, 8 dims each.  A
// thread issues the loads of all nsplit (at most 8) partials before any
// arithmetic (1024x768: 150.5 -> 149.3 us for the call, bit-identical).
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part, uint4* __restrict__ out,
                                                         float* __restrict__ lse, int S, int nqt, int item0,
                                                         int nsplit) {
    const int item_local = blockIdx.x / (BM / 16);
    const int rloc = (blockIdx.x % (BM / 16)) * 16 + (threadIdx.x >> 4);
    const int seg = threadIdx.x & 15;
    const int item = item0 + item_local;
    const int64_t bh = item / nqt;
    const int row = (item - (int)bh * nqt) * BM + rloc;
    if (row >= S) return;
    const float* p0 = part + (int64_t)item_local * nsplit * PART_FLOATS;
    float mv[8], lv[8];
    float4 va[8], vb[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        if (f < nsplit) {
            const float* pf = p0 + (int64_t)f * PART_FLOATS;
            mv[f] = pf[BM * HEAD_DIM + rloc];
            lv[f] = pf[BM * HEAD_DIM + BM + rloc];
            const float4* src = reinterpret_cast<const float4*>(pf + (int64_t)rloc * HEAD_DIM + seg * 8);
            va[f] = src[0];
            vb[f] = src[1];
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int f = 0; f < 8; ++f)
        if (f < nsplit) M = fmaxf(M, mv[f]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float L = 0.0f;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        if (f < nsplit) {
            const float w = __builtin_amdgcn_exp2f(mv[f] - M);
            L += w * lv[f];
            const float4 a = va[f], b = vb[f];
            acc[0] += w * a.x; acc[1] += w * a.y; acc[2] += w * a.z; acc[3] += w * a.w;
            acc[4] += w * b.x; acc[5] += w * b.y; acc[6] += w * b.z; acc[7] += w * b.w;
        }
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    out[(bh * S + row) * 16 + seg] = pack8(acc);
    if (lse != nullptr && seg == 0) lse[bh * S + row] = LN2 * (M + __builtin_amdgcn_logf(L));
}

hipError_t launch_merge(const float* part, void* out, float* lse, int S, int nqt, int item0, int nsplit,
                        int split_items, hipStream_t stream) {
    attn_merge_kernel<<<split_items * (BM / 16), 256, 0, stream>>>(part, static_cast<uint4*>(out), lse, S, nqt, item0,
                                                                   nsplit);
    return hipGetLastError();
}

size_t core_partial_bytes(int BH, int S) { return core_partial_bytes_for(core_plan(BH, S)); }

hipError_t launch_attn_core(const void* q, const void* v, const float* cos_t, const float* sin_t, const void* ws,
                            void* part, int* ctl, void* out, float* lse, int BH, int S, float qmul,
                            hipStream_t stream) {
    const CorePlan p = core_plan(BH, S);
    const uint4* wsv = static_cast<const uint4*>(ws);
    const uint4* qv = static_cast<const uint4*>(q);
    const uint4* vv = static_cast<const uint4*>(v);
    const float4* cv = reinterpret_cast<const float4*>(cos_t);
    const float4* sv = reinterpret_cast<const float4*>(sin_t);
    const int rope = cos_t != nullptr;
    float* pt = static_cast<float*>(part);
    attn_core_kernel<<<core_grid_dynamic(p), NW * 64, 0, stream>>>(qv, vv, cv, sv, wsv, static_cast<uint2*>(out), lse,
                                                                  pt, ctl, S, p.ntiles, p.nqt, p.full, p.nsplit,
                                                                  core_pool_whole(p), qmul, rope);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && p.split > 0) e = launch_merge(pt, out, lse, S, p.nqt, p.full, p.nsplit, p.split, stream);
    return e;
}

}  // namespace dit
