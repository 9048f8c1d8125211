/*
 * dit_attn.h - C ABI of libditattn.so: non-causal joint self-attention of a
 * diffusion-transformer block on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The xDiT paper ("xDiT: an Inference Engine for Diffusion
 * Transformers (DiTs) with Massive Parallelism", abstract) names attention over
 * the long image/video token sequence of a DiT as the cost that grows with
 * resolution, and the AMD blog "How to Scale Diffusion Inference Across AMD
 * RDNA 4 GPUs" (section on Ulysses sequence parallelism) describes each GPU
 * running full-sequence attention for its share of the heads.  For every batch
 * b and head h this library computes, over the joint sequence of S = S_txt +
 * S_img tokens (text rows first, then the patchified latent rows):
 *
 *     q' = RoPE(q), k' = RoPE(k)                  (interleaved pairs, see below)
 *     out = softmax(scale * q' k'^T) v            (no mask, every row sees every key)
 *
 * The softmax is evaluated in the streaming form of FlashAttention-2 (cited in
 * the xDiT paper's reference list): exact up to floating-point rounding.
 *
 * RoPE.  Pair j of a head vector is the dims (2j, 2j+1), rotated as the complex
 * number x[2j] + i x[2j+1] times exp(i * phi[s][j]), with cos(phi) and sin(phi)
 * supplied as fp32 tables of shape [S, D/2].  dit_rope_tables() builds them
 * from integer token coordinates with per-axis frequencies theta^(-2i/d_a).
 *
 * Conventions shared by every entry point.
 *   - Tensor pointers are DEVICE memory owned by the caller; the library keeps
 *     no pointer after returning.  Layout is contiguous [B, H, S, D] (bf16),
 *     16-byte aligned.  `out` must not overlap any input.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on it; DIT_OK means "enqueued", not "finished".
 *   - Every argument is validated on the host BEFORE any HIP call; a bad
 *     argument returns its status and enqueues nothing.  No exception crosses
 *     the ABI.  dit_last_error() returns a thread-local message for the last
 *     non-OK status of the calling thread.
 *   - D must be 128 and S at most 2^21 = 2097152 (DIT_ERR_UNSUPPORTED
 *     otherwise; the kernels address one head's prepared tiles with 32-bit
 *     byte offsets).  Index arithmetic is 64-bit; B*H*ceil(S/256) must fit in
 *     a signed 32-bit int and B*H must be at most 65535.
 *   - NaN/Inf inputs propagate to the output; they are not trapped.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIT_DTYPE_BF16 = 0,
    DIT_DTYPE_FP8_E4M3 = 1
} dit_dtype_t;

typedef enum {
    DIT_OK = 0,
    DIT_ERR_INVALID_ARG = 1,   /* NULL, misaligned, negative or inconsistent argument */
    DIT_ERR_UNSUPPORTED = 2,   /* valid but not implemented (D != 128, dtype) */
    DIT_ERR_NO_DEVICE = 3,     /* no usable HIP device */
    DIT_ERR_OUT_OF_MEMORY = 4, /* workspace allocation failed */
    DIT_ERR_LAUNCH = 5         /* a HIP call or kernel launch reported an error */
} dit_status_t;

/* Thread-local message describing the last non-OK status ("" if none). */
const char* dit_last_error(void);

/* Version of this ABI; bumped when a signature or layout changes. */
int dit_abi_version(void);

/*
 * dit_rope_tables - cos/sin tables of multi-axis RoPE.
 *
 * The pages name RoPE'd DiTs (FLUX, Wan) but never write RoPE out; the form
 * used here is the plainest multi-axis reading: the head's D = sum(axes_dim)
 * dims are split into consecutive per-axis blocks; local pair i of axis a has
 * frequency theta^(-2i/axes_dim[a]); its angle at token s is
 * pos[s][a] * frequency.  Angles, cos and sin are evaluated in fp64 on the
 * device and stored rounded to fp32.
 *
 *   pos        device int32 [S, n_axes]: token coordinates (text tokens 0).
 *   S          number of tokens, >= 1.
 *   n_axes     1..4.
 *   axes_dim   HOST int32 [n_axes]: even, positive; sum = D (any even D).
 *   theta      base frequency, > 0 (10000 for the FLUX/Wan-style shapes).
 *   rope_cos, rope_sin  device fp32 [S, D/2] outputs, 16-byte aligned.
 */
dit_status_t dit_rope_tables(const int32_t* pos, int S, int n_axes, const int32_t* axes_dim,
                             float theta, float* rope_cos, float* rope_sin, void* stream);

/*
 * dit_attn_forward - the whole path: RoPE on Q and K, then joint attention.
 *
 *   q, k, v    device bf16 [B, H, S, D], S = S_txt + S_img (S_txt, S_img >= 0, S >= 1).
 *   rope_cos, rope_sin  device fp32 [S, D/2], shared by all (b, h); both NULL
 *              means no RoPE; exactly one NULL is DIT_ERR_INVALID_ARG.
 *   out        device bf16 [B, H, S, D], written in full.
 *   scale      softmax scale (normally 1/sqrt(D)); finite.
 *   dtype      a dit_dtype_t value, passed as int (any other value is
 *              DIT_ERR_INVALID_ARG); must be DIT_DTYPE_BF16: DIT_DTYPE_FP8_E4M3
 *              returns DIT_ERR_UNSUPPORTED (fp8 inputs need their scales:
 *              dit_attn_forward_fp8).
 *
 * Rounding: rotated K is rounded to bf16 (RNE); rotated Q is multiplied by
 * scale*log2(e) in fp32 and rounded to bf16; QK^T and PV accumulate in fp32
 * on the matrix cores; softmax state is fp32; P is rounded to bf16 for PV;
 * the output is rounded to bf16 (RNE).
 *
 * A workspace of dit_attn_workspace_bytes() is taken from the stream-ordered
 * allocator (hipMallocAsync/hipFreeAsync on `stream`), so calls on different
 * streams do not share it.  Allocation failure returns DIT_ERR_OUT_OF_MEMORY.
 */
dit_status_t dit_attn_forward(const void* q, const void* k, const void* v,
                              const float* rope_cos, const float* rope_sin, void* out,
                              int B, int H, int S_txt, int S_img, int D,
                              float scale, int dtype, void* stream);

/*
 * The two stages of dit_attn_forward, for callers that own the workspace
 * (for example, to reuse one workspace across layers, to capture the calls in
 * a HIP graph, or to time the stages).
 * dit_attn_forward(...) == prepare_k then core, on one workspace.
 *
 * dit_attn_workspace_bytes  bytes needed for B, H, S, D (0 on invalid sizes).
 *
 * dit_attn_prepare_k  rotates K (bf16 RNE) and lays it out in the workspace
 *   in the tile order the attention kernel streams.  V needs no preparation.
 *   The workspace layout is private to this library and may change between
 *   versions.  workspace: device, 256-byte aligned, >= dit_attn_workspace_bytes(B,H,S,D).
 *
 * dit_attn_core  attention of q (rotated and scaled in its prologue) against
 *   the prepared K and the caller's v (bf16 [B, H, S, D], read as it is); the
 *   rope tables must be the ones given to prepare_k.
 *   The call also WRITES the workspace: past the prepared tiles it keeps the
 *   partial results of the query tiles whose keys it splits into ranges
 *   (shapes whose work does not fill whole rounds of the GPU's compute
 *   units; 24 heads of 16896 tokens is one), and two counters with which its
 *   workgroups share out those ranges at run time.  dit_attn_prepare_k clears
 *   the counters and every core call leaves them cleared, so a workspace must
 *   have been prepared (for the same B, H, S) before its first core call, and
 *   core calls that may run at the same time (on different streams) must not
 *   share a workspace, even when they read the same prepared keys.  q, v, out
 *   and the rope tables must not overlap the workspace, and out must not
 *   overlap q or v.
 */
size_t dit_attn_workspace_bytes(int B, int H, int S, int D);

dit_status_t dit_attn_prepare_k(const void* k, const float* rope_cos, const float* rope_sin,
                                void* workspace, size_t workspace_bytes,
                                int B, int H, int S, int D, void* stream);

dit_status_t dit_attn_core(const void* q, const void* v, const float* rope_cos, const float* rope_sin,
                           void* workspace, size_t workspace_bytes, void* out,
                           int B, int H, int S, int D, float scale, void* stream);

/*
 * Ring-attention building blocks.  The xDiT paper page lists "Ring Attention
 * with Blockwise Transformers for Near-Infinite Context" among its references
 * and the xDiT runner configuration in the MXFP4/Quark on MI350 blog has a
 * ring degree: a rank attends its query shard to one key/value block at a
 * time and folds the partial results together with their row log-sum-exp.
 *
 * dit_attn_core_lse  dit_attn_core plus lse: device fp32 [B, H, S], 4-byte
 *   aligned, written with the natural-log log-sum-exp of each query row's
 *   scaled scores, L = log(sum_j exp(scale * q'.k'_j)) over the keys of the
 *   workspace (computed from the same rounded Q'' and K' and the same bf16
 *   weights as out).  For a ring step, prepare the block's keys with the
 *   block's own RoPE tables (dit_attn_prepare_k), pass the block's v, and pass
 *   the query shard's tables here: RoPE of a row depends only on its own
 *   position.  The shard and the block have the same length S.  lse must not
 *   overlap q, v, out, the rope tables or the workspace.  Like dit_attn_core
 *   it writes key-range partials into the workspace, so ring steps that run
 *   concurrently need one workspace each.
 *
 * dit_attn_merge_lse  folds two partial results over disjoint key blocks:
 *   out = w_a o_a + w_b o_b with w_x = exp(lse_x - lse_out) and
 *   lse_out = log(exp(lse_a) + exp(lse_b)); fp32 arithmetic, out rounded to
 *   bf16 RNE.  o_a, o_b, out: device bf16 [B, H, S, D], 16-byte aligned;
 *   lse_a, lse_b, lse_out: device fp32 [B, H, S], 4-byte aligned.  out may be
 *   exactly o_a or o_b and lse_out exactly lse_a or lse_b (in-place folding);
 *   any other overlap is DIT_ERR_INVALID_ARG.  A row whose two LSEs are both
 *   -inf (no keys on either side) yields NaN.
 */
dit_status_t dit_attn_core_lse(const void* q, const void* v, const float* rope_cos, const float* rope_sin,
                               void* workspace, size_t workspace_bytes, void* out, float* lse,
                               int B, int H, int S, int D, float scale, void* stream);

dit_status_t dit_attn_merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                                void* out, float* lse_out, int B, int H, int S, int D, void* stream);

/*
 * fp8 path: Q, K, V as OCP e4m3 codes with one fp32 scale per tensor (the AMD
 * RDNA 4 xDiT blog's fp8 attention backend; the pages give no format, the
 * reading is OCP e4m3, max 448).  Real values are code * scale.
 *
 *   q8, k8, v8  device e4m3 [B, H, S, D] (one byte per element), 16-byte aligned.
 *   q_scale, k_scale, v_scale  finite, > 0.
 *   rope_cos, rope_sin, scale, out (bf16), S_txt, S_img, D, stream: as in
 *               dit_attn_forward (scale may have either sign).
 *   dit_attn_core_fp8 writes key-range partials into the workspace exactly as
 *   dit_attn_core does (same rule for concurrent calls).
 *
 * RoPE is applied to the dequantised values in fp32; rotated K is re-quantised
 * with step k_scale*sqrt(2) and rotated, scaled Q with a power-of-two-adjusted
 * step (applied back through the MFMA's E8M0 scale); QK^T and PV run on
 * v_mfma_scale_f32_32x32x64_f8f6f4 with fp32 accumulation; softmax state is
 * fp32; the weights are rounded to e4m3 for PV; the output is bf16.
 */
size_t dit_attn_workspace_bytes_fp8(int B, int H, int S, int D);

dit_status_t dit_attn_prepare_kv_fp8(const void* k8, const void* v8, float k_scale, float v_scale,
                                     const float* rope_cos, const float* rope_sin,
                                     void* workspace, size_t workspace_bytes,
                                     int B, int H, int S, int D, void* stream);

dit_status_t dit_attn_core_fp8(const void* q8, float q_scale, const float* rope_cos, const float* rope_sin,
                               void* workspace, size_t workspace_bytes, void* out,
                               int B, int H, int S, int D, float scale, void* stream);

dit_status_t dit_attn_forward_fp8(const void* q8, const void* k8, const void* v8,
                                  float q_scale, float k_scale, float v_scale,
                                  const float* rope_cos, const float* rope_sin, void* out,
                                  int B, int H, int S_txt, int S_img, int D, float scale, void* stream);

/*
 * MXFP4 linear layers around attention.  The MXFP4/Quark on MI350 blog runs
 * FLUX's linear layers (the projections on either side of attention and the
 * MLPs) in MXFP4 as the OCP Microscaling specification defines it: blocks of
 * 32 FP4 (E2M1) elements along the reduction axis K share one E8M0 scale;
 * weights are quantised once, activations per call, and the product is an
 * A4W4 matrix-core GEMM ("MXFP4 Quantization" and "MXFP4 Kernel" sections).
 *
 * Layouts (device memory):
 *   codes  [rows, K/2] bytes, row-major: element k in byte k/2, low nibble for
 *          even k.
 *   scales E8M0 (2^(s - 127)) of each 32-element block, in tiles of 32 rows x
 *          8 blocks: block b of row r is byte ((r / 32) * G + b / 8) * 256 +
 *          (r % 32) * 8 + b % 8, with G = ceil(K / 256); the tiles of one
 *          256-deep slice of K are contiguous per 32 rows, which is what one
 *          GEMM step reads.  dit_mxfp4_scale_bytes(rows, K) = ceil(rows / 32)
 *          * G * 256 bytes (0 on invalid sizes); bytes of rows past `rows` or
 *          blocks past K/32 are neither written nor used.
 *
 * dit_mxfp4_quantize  x: bf16 [rows, K], 16-byte aligned, K a multiple of 32,
 *   finite values.  Per block: X = floor(log2 max|x|) - 2 clamped to
 *   [-127, 127] (-127 for an all-zero block), codes = x * 2^-X rounded to the
 *   nearest E2M1 value (ties to the even code, magnitudes above 6 saturate,
 *   the sign bit is kept); scales = X + 127.  Used for the activations at run
 *   time and, once, for the weights.  codes 4-byte aligned; no overlaps.
 *
 * dit_mxfp4_gemm  out[M, N] (bf16 RNE) = deq(A)[M, K] deq(W)[N, K]^T with fp32
 *   accumulation: a_codes/a_scales the quantised activations [M, K], w_codes/
 *   w_scales the quantised weight [N, K] (the nn.Linear layout: one row per
 *   output feature).  K a multiple of 128, N a multiple of 4; rows * K / 2
 *   below 2^31 for both operands; codes 16-byte, scales 4-byte and out
 *   8-byte aligned; out must not overlap an input.
 *
 * dit_mxfp4_linear  quantise x (bf16 [M, K]) into a stream-ordered workspace
 *   (hipMallocAsync / hipFreeAsync on stream), then dit_mxfp4_gemm.
 */
size_t dit_mxfp4_scale_bytes(int rows, int K);

dit_status_t dit_mxfp4_quantize(const void* x, void* codes, void* scales, int rows, int K, void* stream);

dit_status_t dit_mxfp4_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                            void* out, int M, int N, int K, void* stream);

dit_status_t dit_mxfp4_linear(const void* x, const void* w_codes, const void* w_scales, void* out,
                              int M, int N, int K, void* stream);

/*
 * DBCache step caching.  The AMD RDNA 4 xDiT blog (section on skipping
 * transformer work when the model takes enough denoising steps) enables
 * DBCache with a residual diff threshold: after the first Fn transformer
 * blocks of a step, the residual those blocks produced is compared with the
 * previous step's, and the rest of the step reuses cached work when they are
 * close.  The page names the threshold (0.12 in its example) but no formula;
 * this library takes the relative L1 distance
 *
 *     diff  = sum_i |cur_i - prev_i| / sum_i |prev_i|   (+inf when prev is all zero)
 *     reuse = diff < threshold
 *
 * dit_dbcache_workspace_bytes  the fixed workspace size (bytes) that
 *   dit_dbcache_residual_diff needs, for any n.
 *
 * dit_dbcache_residual_diff  prev, cur: bf16 residuals of n elements each
 *   (any shape, contiguous, 16-byte aligned; n >= 0; n = 0 gives +inf and no
 *   reuse, and prev and cur may then be NULL).  ws: device workspace of at least dit_dbcache_workspace_bytes(),
 *   16-byte aligned, not overlapping the inputs or outputs; its contents are
 *   scratch.  diff: device double (8-byte aligned), written with the
 *   difference; reuse: device int32 (4-byte aligned) set to 1 or 0, or NULL.
 *   Sums of |.| are taken in fp32 over 8 elements and in fp64 beyond, in a
 *   fixed order: the result is reproducible for a given n.  NaN inputs give a
 *   NaN diff and reuse = 0.
 */
size_t dit_dbcache_workspace_bytes(void);

dit_status_t dit_dbcache_residual_diff(const void* prev, const void* cur, int64_t n, double threshold,
                                       void* ws, size_t ws_bytes, double* diff, int32_t* reuse, void* stream);

/*
 * dit_dbcache_residual_diff_noalloc - dit_dbcache_residual_diff for callers
 *   that cannot allocate device memory (code under HIP graph capture, tight
 *   serving loops, harnesses that forbid hipMalloc): the same kernels and the
 *   same result, bit for bit, but the per-workgroup partial sums go to a
 *   static device array of the library (128 KiB per GPU, the most the
 *   partials launch can use for any n, held until the process ends) instead
 *   of a caller workspace.  Arguments and errors as in
 *   dit_dbcache_residual_diff without ws / ws_bytes.  The call makes no
 *   allocation of its own.  All calls on one GPU share that array: calls that
 *   may overlap on one GPU (different streams, or different threads) race and
 *   must be serialised by the caller; it needs no clearing between calls.
 */
dit_status_t dit_dbcache_residual_diff_noalloc(const void* prev, const void* cur, int64_t n, double threshold,
                                               double* diff, int32_t* reuse, void* stream);

/*
 * Clock probe (measurement aid, not part of the attention path).  The
 * published MI355X peaks assume a 2.4 GHz shader clock; under a sustained
 * matrix-core load the chip runs slower, and a roofline can also be priced at
 * the clock it actually runs at.
 *
 * dit_clock_probe  runs `blocks` workgroups of 256 threads (4 waves each, two
 *   workgroups per CU) that each issue iters x 4 independent
 *   v_mfma_f32_32x32x16_bf16 between two reads of the shader cycle counter
 *   and of the constant-rate counter.  out: device buffer of at least
 *   blocks x 4 x 24 bytes, 8-byte aligned; per wave three uint64: shader
 *   cycles, constant-rate ticks, 0.  blocks in [1, 65535], iters in
 *   [1, 2^24].
 * dit_wall_clock_khz  the constant-rate counter's frequency (kHz) of the
 *   current device.
 */
dit_status_t dit_clock_probe(void* out, size_t out_bytes, int blocks, int iters, void* stream);

dit_status_t dit_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
