// lse_merge.hip - exact merge of two partial attention results over disjoint
// key blocks, for ring attention ("Ring Attention with Blockwise Transformers
// for Near-Infinite Context", in the reference list of the xDiT paper page;
// the xDiT runner configuration in the MXFP4/Quark on MI350 blog has a ring
// degree).  Each rank folds the result of every key/value block it receives
// into its running result.
//
// For a query row with partial results (O_a, L_a) and (O_b, L_b), L the
// natural-log log-sum-exp of the row's scaled scores over the block's keys,
// softmax over the union of the blocks gives block a the total weight
// e^L_a / (e^L_a + e^L_b), so
//
//     O = w_a O_a + w_b O_b,  w_x = e^(L_x - L),  L = log(e^L_a + e^L_b).
//
// Weights and sums in fp32 (offset by max(L_a, L_b)), O rounded to bf16 RNE.
//
// Roofline: HBM bound.  Algorithmic bytes per row: 2 x 256 B + 8 B read,
// 256 B + 4 B written (D = 128, bf16).
#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "bf16_util.h"

namespace dit {

constexpr float LOG2E = 1.44269504088896341f;

// 16 threads per row, thread t of a row: dims 8t .. 8t + 7.  The row's 16
// threads are consecutive lanes of one wave, so every read of a row happens
// before any write of it: out may be o_a or o_b, and lse_out may be lse_a or
// lse_b (in-place folding).  Grid-stride over rows.
__global__ __launch_bounds__(256) void lse_merge_kernel(const uint4* o_a, const float* lse_a, const uint4* o_b,
                                                        const float* lse_b, uint4* out, float* lse_out,
                                                        int64_t rows) {
    const int seg = threadIdx.x & 15;
    for (int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4); row < rows; row += (int64_t)gridDim.x * 16) {
        const float a = lse_a[row], b = lse_b[row];
        const float mx = fmaxf(a, b);
        const float ea = exp2f((a - mx) * LOG2E), eb = exp2f((b - mx) * LOG2E);
        const float sum = ea + eb;
        const float wa = ea / sum, wb = eb / sum;
        float fa[8], fb[8];
        unpack8(o_a[row * 16 + seg], fa);
        unpack8(o_b[row * 16 + seg], fb);
#pragma unroll
        for (int e = 0; e < 8; ++e) fa[e] = wa * fa[e] + wb * fb[e];
        out[row * 16 + seg] = pack8(fa);
        if (seg == 0) lse_out[row] = mx + log2f(sum) * LN2;
    }
}

hipError_t launch_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* out,
                            float* lse_out, int64_t rows, hipStream_t stream) {
    const int64_t blocks = std::min<int64_t>((rows + 15) / 16, (int64_t)MI355X_CUS * 64);
    lse_merge_kernel<<<(int)blocks, 256, 0, stream>>>(static_cast<const uint4*>(o_a), lse_a,
                                                      static_cast<const uint4*>(o_b), lse_b, static_cast<uint4*>(out),
                                                      lse_out, rows);
    return hipGetLastError();
}

}  // namespace dit
