// abi_check.cpp - drives the argument checks of libditattn's C ABI on the
// host, for a build whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every call below is rejected before any HIP
// call (pointers are never dereferenced); the expected status of each is
// checked.  Without a device, calls with valid arguments must stop at the
// device check; with a device they are skipped (nothing is launched here).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "dit_attn.h"

static int failures = 0;

#define EXPECT(call, status)                                                                    \
    do {                                                                                        \
        const int got_ = (int)(call);                                                           \
        if (got_ != (int)(status)) {                                                            \
            std::printf("FAIL line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, got_, (int)(status), \
                        dit_last_error());                                                      \
            ++failures;                                                                         \
        } else if (got_ != DIT_OK && dit_last_error()[0] == '\0') {                             \
            std::printf("FAIL line %d: %s gave no message\n", __LINE__, #call);                 \
            ++failures;                                                                         \
        }                                                                                       \
    } while (0)

static void* P(uintptr_t x) { return reinterpret_cast<void*>(x); }
static float* FP(uintptr_t x) { return reinterpret_cast<float*>(x); }

int main(int argc, char** argv) {
    const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
    const uintptr_t A = 0x100000, WS = 0x10000000;
    const int E = DIT_ERR_INVALID_ARG, U = DIT_ERR_UNSUPPORTED, N = DIT_ERR_NO_DEVICE;

    // forward: NULLs, tables, shapes, overflows, scale, alignment, overlaps
    EXPECT(dit_attn_forward(nullptr, P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), FP(5 * A), nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 0, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 2147483647, 1, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 1 << 21, 1, 128, 0.1f, DIT_DTYPE_BF16, nullptr), U);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 70000, 1, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 60000, 1 << 20, 0, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 64, 0.1f, DIT_DTYPE_BF16, nullptr), U);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, NAN, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, 7, nullptr), E);
    EXPECT(dit_attn_forward(P(A + 2), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(2 * A + 256), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);
    EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), FP(4 * A + 256), FP(6 * A), P(4 * A), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), E);

    // split stages
    const size_t need = dit_attn_workspace_bytes(1, 2, 8, 128);
    if (need == 0) { std::printf("FAIL workspace size 0\n"); ++failures; }
    if (dit_attn_workspace_bytes(1, 1, (1 << 21) + 1, 128) != 0) { std::printf("FAIL oversize workspace\n"); ++failures; }
    EXPECT(dit_attn_prepare_k(P(A), nullptr, nullptr, P(WS), need - 1, 1, 2, 8, 128, nullptr), E);
    EXPECT(dit_attn_prepare_k(P(A), nullptr, nullptr, P(WS + 16), need, 1, 2, 8, 128, nullptr), E);
    EXPECT(dit_attn_prepare_k(P(A), FP(WS + 512), FP(5 * A), P(WS), need, 1, 2, 8, 128, nullptr), E);
    EXPECT(dit_attn_core(P(WS + 256), P(7 * A), nullptr, nullptr, P(WS), need, P(3 * A), 1, 2, 8, 128, 0.1f, nullptr), E);
    EXPECT(dit_attn_core(P(A), P(3 * A + 64), nullptr, nullptr, P(WS), need, P(3 * A), 1, 2, 8, 128, 0.1f, nullptr), E);
    EXPECT(dit_attn_core_lse(P(A), P(7 * A), nullptr, nullptr, P(WS), need, P(3 * A), FP(WS + 128), 1, 2, 8, 128, 0.1f, nullptr), E);
    EXPECT(dit_attn_core_lse(P(A), P(7 * A), nullptr, nullptr, P(WS), need, P(3 * A), FP(0x20000002), 1, 2, 8, 128, 0.1f, nullptr), E);
    EXPECT(dit_attn_merge_lse(P(0x30000000), FP(0x60000000), P(0x40000000), FP(0x70000000), P(0x30000010), FP(0x80000000), 1, 2, 8, 128, nullptr), E);

    // fp8
    const size_t need8 = dit_attn_workspace_bytes_fp8(1, 2, 8, 128);
    EXPECT(dit_attn_forward_fp8(P(A), P(2 * A), P(3 * A), 0.0f, 0.1f, 0.1f, nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, nullptr), E);
    EXPECT(dit_attn_prepare_kv_fp8(P(A), P(2 * A), 0.1f, NAN, nullptr, nullptr, P(WS), need8, 1, 2, 8, 128, nullptr), E);
    EXPECT(dit_attn_core_fp8(P(WS + 1024), 0.1f, nullptr, nullptr, P(WS), need8, P(3 * A), 1, 2, 8, 128, 0.1f, nullptr), E);

    // rope tables
    const int32_t dims[2] = {64, 64}, bad[2] = {63, 65};
    EXPECT(dit_rope_tables(reinterpret_cast<const int32_t*>(A), 4, 2, bad, 1e4f, FP(2 * A), FP(3 * A), nullptr), E);
    EXPECT(dit_rope_tables(reinterpret_cast<const int32_t*>(A), 4, 5, dims, 1e4f, FP(2 * A), FP(3 * A), nullptr), E);
    EXPECT(dit_rope_tables(reinterpret_cast<const int32_t*>(A), 4, 2, dims, 1e4f, FP(2 * A), FP(2 * A + 64), nullptr), E);

    // MXFP4
    EXPECT(dit_mxfp4_quantize(P(0x30000000), P(0x40000000), P(0x50000000), 1 << 20, 1 << 12, nullptr), U);
    EXPECT(dit_mxfp4_gemm(P(0x40000000), P(0x50000000), P(0x41000000), P(0x51000000), P(0x60000000), 8, 18, 256, nullptr), E);
    EXPECT(dit_mxfp4_linear(P(0x30000000), P(0x40000000), P(0x50000000), P(0x30000000), 8, 16, 256, nullptr), E);

    // DBCache, both entry points
    const uintptr_t p = 0x30000000, c = 0x40000000, w = 0x50000000, d = 0x60000000, r = 0x60000040;
    const size_t wsb = dit_dbcache_workspace_bytes();
    EXPECT(dit_dbcache_residual_diff(P(p), P(c), 1000, 0.12, P(w), wsb - 16, reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(r), nullptr), E);
    EXPECT(dit_dbcache_residual_diff(P(p), P(c), ((int64_t)1 << 40) + 1, 0.12, P(w), wsb, reinterpret_cast<double*>(d), reinterpret_cast<int32_t*>(r), nullptr), U);
    EXPECT(dit_dbcache_residual_diff_noalloc(P(p), P(c), -1, 0.12, reinterpret_cast<double*>(d), nullptr, nullptr), E);
    EXPECT(dit_dbcache_residual_diff_noalloc(P(p), P(c), 1000, 0.12, reinterpret_cast<double*>(c + 16), nullptr, nullptr), E);

    // clock probe
    EXPECT(dit_clock_probe(P(0x30000000), 8 * 4 * 24 - 1, 8, 10, nullptr), E);
    EXPECT(dit_wall_clock_khz(nullptr), E);

    if (no_device) {
        EXPECT(dit_attn_forward(P(A), P(2 * A), P(3 * A), nullptr, nullptr, P(4 * A), 1, 2, 3, 5, 128, 0.1f, DIT_DTYPE_BF16, nullptr), N);
        EXPECT(dit_attn_core(P(A), P(7 * A), FP(5 * A), FP(6 * A), P(WS), need, P(3 * A), 1, 2, 8, 128, -0.1f, nullptr), N);
        EXPECT(dit_dbcache_residual_diff_noalloc(nullptr, nullptr, 0, 0.12, reinterpret_cast<double*>(d), nullptr, nullptr), N);
        EXPECT(dit_mxfp4_linear(P(0x30000000), P(0x40000000), P(0x50000000), P(0x60000000), 8, 16, 256, nullptr), N);
    }
    std::printf("abi_check: %d failure(s)\n", failures);
    return failures == 0 ? 0 : 1;
}
