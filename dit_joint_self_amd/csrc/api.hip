// api.hip - host side of libditattn.so: argument validation, device checks,
// workspace management and kernel launches on the caller's stream.
//
// Every argument is checked before the first HIP call, so a bad call never
// touches the device.  Errors are reported as dit_status_t plus a
// thread-local message; no exception leaves this file.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "dit_attn.h"
#include "attn_common.h"
#include "tile_layout.h"

namespace dit {
hipError_t launch_prepare_k(const void* k, const float* cos_t, const float* sin_t, void* ws, int* ctl, int BH,
                            int S, hipStream_t stream);
hipError_t launch_lse_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* out,
                            float* lse_out, int64_t rows, hipStream_t stream);
hipError_t launch_mxfp4_quantize(const void* x, void* codes, void* scales, int64_t rows, int K, hipStream_t stream);
size_t mx_scale_bytes(int64_t rows, int K);
size_t residual_diff_workspace_bytes();
size_t residual_diff_scratch_bytes();
hipError_t residual_diff_scratch(int dev, void** ptr);
hipError_t launch_clock_probe(int blocks, int iters, void* out, hipStream_t stream);
hipError_t launch_residual_diff(const void* prev, const void* cur, int64_t n, double threshold, void* ws,
                                double* diff, int32_t* reuse, hipStream_t stream);
hipError_t launch_mxfp4_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                             void* out, int M, int N, int K, hipStream_t stream);
hipError_t launch_attn_core(const void* q, const void* v, const float* cos_t, const float* sin_t, const void* ws,
                            void* part, int* ctl, void* out, float* lse, int BH, int S, float qmul,
                            hipStream_t stream);
size_t core_partial_bytes(int BH, int S);
hipError_t launch_prepare_kv_fp8(const void* k, const void* v, const float* cos_t, const float* sin_t, void* ws,
                                 int* ctl, int BH, int S, float k_scale, float v_scale, hipStream_t stream);
hipError_t launch_attn_core_fp8(const void* q, float q_scale, const float* cos_t, const float* sin_t, const void* ws,
                                void* part, int* ctl, void* out, int BH, int S, float qmul, hipStream_t stream);
size_t core_fp8_partial_bytes(int BH, int S);
hipError_t launch_rope_tables(const int32_t* pos, int S, int n_axes, const int32_t* axes_dim,
                              double theta, float* cos_t, float* sin_t, hipStream_t stream);
}  // namespace dit

namespace {

constexpr int kAbiVersion = 6;
constexpr int kMaxDevices = 64;
// Smallest query tile any kernel variant uses; bounds the workgroup count.
constexpr int kMinBlockM = 128;

thread_local char g_err[512] = "";

dit_status_t fail(dit_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

dit_status_t ok() {
    g_err[0] = '\0';
    return DIT_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Host-only checks shared by the attention entry points.
dit_status_t check_shape(int B, int H, int S, int D) {
    if (B < 1 || H < 1) return fail(DIT_ERR_INVALID_ARG, "B and H must be >= 1 (got B=%d H=%d)", B, H);
    if (S < 1) return fail(DIT_ERR_INVALID_ARG, "S must be >= 1 (got %d)", S);
    if (D < 1) return fail(DIT_ERR_INVALID_ARG, "D must be >= 1 (got %d)", D);
    if (D != dit::HEAD_DIM) return fail(DIT_ERR_UNSUPPORTED, "only D = 128 is implemented (got %d)", D);
    if (S > dit::MAX_SEQ)
        return fail(DIT_ERR_UNSUPPORTED, "S = %d exceeds the longest supported sequence (%d)", S, dit::MAX_SEQ);
    const int64_t wgs = (int64_t)B * H * ((S + kMinBlockM - 1) / kMinBlockM);
    const int64_t tiles = (int64_t)B * H * dit::num_kv_tiles(S);
    if (wgs > INT_MAX || tiles > INT_MAX || (int64_t)B * H > 65535)
        return fail(DIT_ERR_INVALID_ARG, "B*H*S too large for one launch (B=%d H=%d S=%d)", B, H, S);
    return DIT_OK;
}

dit_status_t check_rope(const float* c, const float* s) {
    if ((c == nullptr) != (s == nullptr))
        return fail(DIT_ERR_INVALID_ARG, "rope_cos and rope_sin must both be NULL or both non-NULL");
    if (c && (!aligned16(c) || !aligned16(s)))
        return fail(DIT_ERR_INVALID_ARG, "rope tables must be 16-byte aligned");
    return DIT_OK;
}

// The rope tables (when given) against up to two regions the call writes.
dit_status_t check_tables_apart(const float* c, const float* s, int S, const void* a, size_t na, const void* b,
                                size_t nb) {
    if (!c) return DIT_OK;
    const size_t tb = (size_t)S * (dit::HEAD_DIM / 2) * sizeof(float);
    if (overlaps(c, tb, a, na) || overlaps(s, tb, a, na) || (b && (overlaps(c, tb, b, nb) || overlaps(s, tb, b, nb))))
        return fail(DIT_ERR_INVALID_ARG, "a rope table overlaps a region the call writes");
    return DIT_OK;
}

// Device present and gfx950; the result is cached per device ordinal.
dit_status_t check_device() {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return fail(DIT_ERR_NO_DEVICE, "no HIP device is visible");
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(DIT_ERR_NO_DEVICE, "hipGetDevice failed");
    static std::mutex mu;
    static signed char arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
    if (dev < 0 || dev >= kMaxDevices) return fail(DIT_ERR_NO_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (arch_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(DIT_ERR_NO_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        if (arch_ok[dev] < 0)
            return fail(DIT_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                        prop.gcnArchName);
        // Keep freed workspace in the stream-ordered pool between calls.
        hipMemPool_t pool;
        if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
            uint64_t keep = UINT64_MAX;
            (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
        }
    }
    if (arch_ok[dev] < 0) return fail(DIT_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return DIT_OK;
}

dit_status_t launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(DIT_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char* dit_last_error(void) { return g_err; }

int dit_abi_version(void) { return kAbiVersion; }

dit_status_t dit_rope_tables(const int32_t* pos, int S, int n_axes, const int32_t* axes_dim, float theta,
                             float* rope_cos, float* rope_sin, void* stream) {
    if (!pos || !axes_dim || !rope_cos || !rope_sin)
        return fail(DIT_ERR_INVALID_ARG, "pos, axes_dim, rope_cos and rope_sin must be non-NULL");
    if (S < 1) return fail(DIT_ERR_INVALID_ARG, "S must be >= 1 (got %d)", S);
    if (n_axes < 1 || n_axes > 4) return fail(DIT_ERR_INVALID_ARG, "n_axes must be 1..4 (got %d)", n_axes);
    int64_t D = 0;
    for (int a = 0; a < n_axes; ++a) {
        if (axes_dim[a] < 2 || (axes_dim[a] & 1))
            return fail(DIT_ERR_INVALID_ARG, "axes_dim[%d] = %d must be even and >= 2", a, axes_dim[a]);
        D += axes_dim[a];
    }
    if (!(theta > 0.0f) || !std::isfinite(theta))
        return fail(DIT_ERR_INVALID_ARG, "theta must be finite and > 0");
    if ((int64_t)S * (D / 2) > (int64_t)INT_MAX * 256)
        return fail(DIT_ERR_INVALID_ARG, "S * D/2 too large");
    if (!aligned16(rope_cos) || !aligned16(rope_sin))
        return fail(DIT_ERR_INVALID_ARG, "rope tables must be 16-byte aligned");
    if (overlaps(rope_cos, (size_t)S * (D / 2) * 4, rope_sin, (size_t)S * (D / 2) * 4))
        return fail(DIT_ERR_INVALID_ARG, "rope_cos and rope_sin overlap");
    dit_status_t st = check_device();
    if (st != DIT_OK) return st;
    return launched(dit::launch_rope_tables(pos, S, n_axes, axes_dim, (double)theta, rope_cos, rope_sin,
                                            static_cast<hipStream_t>(stream)),
                    "rope_tables_kernel");
}

// Workspace: the K' tile stream, then (256-byte aligned) the key-range
// partials of the items that run split, then the attention launch's piece
// counters (CORE_CTL_BYTES).
static size_t tiles_bytes(int B, int H, int S) {
    return ((size_t)B * H * (size_t)dit::num_kv_tiles(S) * dit::K_PART_BYTES + 255) & ~(size_t)255;
}
static int* ctl_of(void* ws, int B, int H, int S) {
    return reinterpret_cast<int*>(static_cast<char*>(ws) + tiles_bytes(B, H, S) + dit::core_partial_bytes(B * H, S));
}

size_t dit_attn_workspace_bytes(int B, int H, int S, int D) {
    if (B < 1 || H < 1 || S < 1 || D != dit::HEAD_DIM) return 0;
    if (check_shape(B, H, S, D) != DIT_OK) return 0;
    return tiles_bytes(B, H, S) + dit::core_partial_bytes(B * H, S) + dit::CORE_CTL_BYTES;
}

dit_status_t dit_attn_prepare_k(const void* k, const float* rope_cos, const float* rope_sin, void* workspace,
                                size_t workspace_bytes, int B, int H, int S, int D, void* stream) {
    if (!k || !workspace) return fail(DIT_ERR_INVALID_ARG, "k and workspace must be non-NULL");
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if (!aligned16(k)) return fail(DIT_ERR_INVALID_ARG, "k must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(DIT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t need = dit_attn_workspace_bytes(B, H, S, D);
    if (workspace_bytes < need)
        return fail(DIT_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const size_t tbytes = (size_t)B * H * S * D * 2;
    if (overlaps(workspace, need, k, tbytes)) return fail(DIT_ERR_INVALID_ARG, "workspace overlaps k");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, workspace, need, nullptr, 0)) != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_prepare_k(k, rope_cos, rope_sin, workspace, ctl_of(workspace, B, H, S), B * H, S,
                                          static_cast<hipStream_t>(stream)),
                    "prepare_k_kernel");
}

static dit_status_t core_impl(const void* q, const void* v, const float* rope_cos, const float* rope_sin,
                              void* workspace, size_t workspace_bytes, void* out, float* lse, int B, int H, int S,
                              int D, float scale, void* stream) {
    if (!q || !v || !workspace || !out) return fail(DIT_ERR_INVALID_ARG, "q, v, workspace and out must be non-NULL");
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if (!std::isfinite(scale)) return fail(DIT_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q) || !aligned16(v) || !aligned16(out))
        return fail(DIT_ERR_INVALID_ARG, "q, v and out must be 16-byte aligned");
    const size_t need = dit_attn_workspace_bytes(B, H, S, D);
    if (workspace_bytes < need)
        return fail(DIT_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const size_t tbytes = (size_t)B * H * S * D * 2;
    if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, v, tbytes) || overlaps(out, tbytes, workspace, need))
        return fail(DIT_ERR_INVALID_ARG, "out overlaps q, v or the workspace");
    // The call writes key-range partials into the workspace while other
    // workgroups still read q, v and the tables.
    if (overlaps(q, tbytes, workspace, need) || overlaps(v, tbytes, workspace, need))
        return fail(DIT_ERR_INVALID_ARG, "q or v overlaps the workspace");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, workspace, need, out, tbytes)) != DIT_OK) return st;
    if (lse) {
        const size_t lbytes = (size_t)B * H * S * 4;
        if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(DIT_ERR_INVALID_ARG, "lse must be 4-byte aligned");
        if (overlaps(lse, lbytes, out, tbytes) || overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, v, tbytes) ||
            overlaps(lse, lbytes, workspace, need))
            return fail(DIT_ERR_INVALID_ARG, "lse overlaps q, v, out or the workspace");
        if ((st = check_tables_apart(rope_cos, rope_sin, S, lse, lbytes, nullptr, 0)) != DIT_OK) return st;
    }
    if ((st = check_device()) != DIT_OK) return st;
    const float qmul = (float)((double)scale * 1.4426950408889634073599);  // scale * log2(e)
    void* part = static_cast<char*>(workspace) + tiles_bytes(B, H, S);
    return launched(dit::launch_attn_core(q, v, rope_cos, rope_sin, workspace, part, ctl_of(workspace, B, H, S), out,
                                          lse, B * H, S, qmul, static_cast<hipStream_t>(stream)),
                    "attn_core_kernel");
}

dit_status_t dit_attn_core(const void* q, const void* v, const float* rope_cos, const float* rope_sin,
                           void* workspace, size_t workspace_bytes, void* out, int B, int H, int S, int D, float scale,
                           void* stream) {
    return core_impl(q, v, rope_cos, rope_sin, workspace, workspace_bytes, out, nullptr, B, H, S, D, scale, stream);
}

dit_status_t dit_attn_core_lse(const void* q, const void* v, const float* rope_cos, const float* rope_sin,
                               void* workspace, size_t workspace_bytes, void* out, float* lse, int B, int H, int S,
                               int D, float scale, void* stream) {
    if (!lse) return fail(DIT_ERR_INVALID_ARG, "lse must be non-NULL");
    return core_impl(q, v, rope_cos, rope_sin, workspace, workspace_bytes, out, lse, B, H, S, D, scale, stream);
}

// Two regions either coincide exactly (an allowed in-place fold) or are disjoint.
static bool same_or_disjoint(const void* a, const void* b, size_t bytes) {
    return a == b || !overlaps(a, bytes, b, bytes);
}

dit_status_t dit_attn_merge_lse(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b, void* out,
                                float* lse_out, int B, int H, int S, int D, void* stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !out || !lse_out)
        return fail(DIT_ERR_INVALID_ARG, "o_a, lse_a, o_b, lse_b, out and lse_out must be non-NULL");
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(out))
        return fail(DIT_ERR_INVALID_ARG, "o_a, o_b and out must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse_a) | reinterpret_cast<uintptr_t>(lse_b) |
         reinterpret_cast<uintptr_t>(lse_out)) & 3u)
        return fail(DIT_ERR_INVALID_ARG, "lse arrays must be 4-byte aligned");
    const size_t tbytes = (size_t)B * H * S * D * 2, lbytes = (size_t)B * H * S * 4;
    if (!same_or_disjoint(out, o_a, tbytes) || !same_or_disjoint(out, o_b, tbytes))
        return fail(DIT_ERR_INVALID_ARG, "out must be o_a, o_b or disjoint from both");
    if (!same_or_disjoint(lse_out, lse_a, lbytes) || !same_or_disjoint(lse_out, lse_b, lbytes))
        return fail(DIT_ERR_INVALID_ARG, "lse_out must be lse_a, lse_b or disjoint from both");
    if (overlaps(out, tbytes, lse_a, lbytes) || overlaps(out, tbytes, lse_b, lbytes) ||
        overlaps(out, tbytes, lse_out, lbytes) || overlaps(lse_out, lbytes, o_a, tbytes) ||
        overlaps(lse_out, lbytes, o_b, tbytes))
        return fail(DIT_ERR_INVALID_ARG, "an output overlaps an input of the other kind");
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_lse_merge(o_a, lse_a, o_b, lse_b, out, lse_out, (int64_t)B * H * S,
                                          static_cast<hipStream_t>(stream)),
                    "lse_merge_kernel");
}

// ---------------------------------------------------------------- fp8

// fp8 workspace: header and tiles, the key-range partials, the pool counters.
static size_t fp8_tiles_bytes(int B, int H, int S) {
    return (dit::F8_HEADER_BYTES + (size_t)B * H * (size_t)dit::num_kv_tiles(S) * dit::F8_TILE_BYTES + 255) &
           ~(size_t)255;
}
static int* fp8_ctl_of(void* ws, int B, int H, int S) {
    return reinterpret_cast<int*>(static_cast<char*>(ws) + fp8_tiles_bytes(B, H, S) +
                                  dit::core_fp8_partial_bytes(B * H, S));
}

static dit_status_t check_scale(float s, const char* name) {
    if (!(s > 0.0f) || !std::isfinite(s)) return fail(DIT_ERR_INVALID_ARG, "%s must be finite and > 0", name);
    return DIT_OK;
}

size_t dit_attn_workspace_bytes_fp8(int B, int H, int S, int D) {
    if (B < 1 || H < 1 || S < 1 || D != dit::HEAD_DIM) return 0;
    if (check_shape(B, H, S, D) != DIT_OK) return 0;
    return fp8_tiles_bytes(B, H, S) + dit::core_fp8_partial_bytes(B * H, S) + dit::CORE_CTL_BYTES;
}

dit_status_t dit_attn_prepare_kv_fp8(const void* k8, const void* v8, float k_scale, float v_scale,
                                     const float* rope_cos, const float* rope_sin, void* workspace,
                                     size_t workspace_bytes, int B, int H, int S, int D, void* stream) {
    if (!k8 || !v8 || !workspace) return fail(DIT_ERR_INVALID_ARG, "k8, v8 and workspace must be non-NULL");
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if ((st = check_scale(k_scale, "k_scale")) != DIT_OK || (st = check_scale(v_scale, "v_scale")) != DIT_OK)
        return st;
    if (!aligned16(k8) || !aligned16(v8)) return fail(DIT_ERR_INVALID_ARG, "k8 and v8 must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(DIT_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t need = dit_attn_workspace_bytes_fp8(B, H, S, D);
    if (workspace_bytes < need)
        return fail(DIT_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const size_t tbytes = (size_t)B * H * S * D;
    if (overlaps(workspace, need, k8, tbytes) || overlaps(workspace, need, v8, tbytes))
        return fail(DIT_ERR_INVALID_ARG, "workspace overlaps k8 or v8");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, workspace, need, nullptr, 0)) != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_prepare_kv_fp8(k8, v8, rope_cos, rope_sin, workspace, fp8_ctl_of(workspace, B, H, S),
                                               B * H, S, k_scale, v_scale,
                                               static_cast<hipStream_t>(stream)),
                    "prepare_kv_fp8_kernel");
}

dit_status_t dit_attn_core_fp8(const void* q8, float q_scale, const float* rope_cos, const float* rope_sin,
                               void* workspace, size_t workspace_bytes, void* out, int B, int H, int S, int D,
                               float scale, void* stream) {
    if (!q8 || !workspace || !out) return fail(DIT_ERR_INVALID_ARG, "q8, workspace and out must be non-NULL");
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if ((st = check_scale(q_scale, "q_scale")) != DIT_OK) return st;
    if (!std::isfinite(scale)) return fail(DIT_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q8) || !aligned16(out)) return fail(DIT_ERR_INVALID_ARG, "q8 and out must be 16-byte aligned");
    const size_t need = dit_attn_workspace_bytes_fp8(B, H, S, D);
    if (workspace_bytes < need)
        return fail(DIT_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
    const size_t obytes = (size_t)B * H * S * D * 2;
    if (overlaps(out, obytes, q8, (size_t)B * H * S * D) || overlaps(out, obytes, workspace, need))
        return fail(DIT_ERR_INVALID_ARG, "out overlaps q8 or the workspace");
    if (overlaps(q8, (size_t)B * H * S * D, workspace, need))
        return fail(DIT_ERR_INVALID_ARG, "q8 overlaps the workspace");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, workspace, need, out, obytes)) != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;
    const float qmul = (float)((double)scale * 1.4426950408889634073599);
    void* part = static_cast<char*>(workspace) + fp8_tiles_bytes(B, H, S);
    return launched(dit::launch_attn_core_fp8(q8, q_scale, rope_cos, rope_sin, workspace, part,
                                              fp8_ctl_of(workspace, B, H, S), out, B * H, S, qmul,
                                              static_cast<hipStream_t>(stream)),
                    "attn_core_fp8_kernel");
}

dit_status_t dit_attn_forward_fp8(const void* q8, const void* k8, const void* v8, float q_scale, float k_scale,
                                  float v_scale, const float* rope_cos, const float* rope_sin, void* out, int B,
                                  int H, int S_txt, int S_img, int D, float scale, void* stream) {
    if (!q8 || !k8 || !v8 || !out) return fail(DIT_ERR_INVALID_ARG, "q8, k8, v8 and out must be non-NULL");
    if (S_txt < 0 || S_img < 0)
        return fail(DIT_ERR_INVALID_ARG, "S_txt and S_img must be >= 0 (got %d, %d)", S_txt, S_img);
    if ((int64_t)S_txt + S_img > INT_MAX) return fail(DIT_ERR_INVALID_ARG, "S_txt + S_img overflows int");
    const int S = S_txt + S_img;
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if ((st = check_scale(q_scale, "q_scale")) != DIT_OK || (st = check_scale(k_scale, "k_scale")) != DIT_OK ||
        (st = check_scale(v_scale, "v_scale")) != DIT_OK)
        return st;
    if (!std::isfinite(scale)) return fail(DIT_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(out))
        return fail(DIT_ERR_INVALID_ARG, "q8, k8, v8 and out must be 16-byte aligned");
    const size_t ibytes = (size_t)B * H * S * D, obytes = ibytes * 2;
    if (overlaps(out, obytes, q8, ibytes) || overlaps(out, obytes, k8, ibytes) || overlaps(out, obytes, v8, ibytes))
        return fail(DIT_ERR_INVALID_ARG, "out overlaps an input");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, out, obytes, nullptr, 0)) != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t need = dit_attn_workspace_bytes_fp8(B, H, S, D);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, need, s) != hipSuccess || ws == nullptr) {
        (void)hipGetLastError();
        return fail(DIT_ERR_OUT_OF_MEMORY, "hipMallocAsync of %zu workspace bytes failed", need);
    }
    hipError_t e =
        dit::launch_prepare_kv_fp8(k8, v8, rope_cos, rope_sin, ws, fp8_ctl_of(ws, B, H, S), B * H, S, k_scale, v_scale, s);
    if (e == hipSuccess) {
        const float qmul = (float)((double)scale * 1.4426950408889634073599);
        e = dit::launch_attn_core_fp8(q8, q_scale, rope_cos, rope_sin, ws, static_cast<char*>(ws) + fp8_tiles_bytes(B, H, S),
                                      fp8_ctl_of(ws, B, H, S), out, B * H, S, qmul, s);
    }
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess) return launched(e, "dit_attn_forward_fp8 kernels");
    return launched(ef, "hipFreeAsync of the workspace");
}

dit_status_t dit_attn_forward(const void* q, const void* k, const void* v, const float* rope_cos,
                              const float* rope_sin, void* out, int B, int H, int S_txt, int S_img, int D,
                              float scale, int dtype, void* stream) {
    if (!q || !k || !v || !out) return fail(DIT_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
    if (S_txt < 0 || S_img < 0)
        return fail(DIT_ERR_INVALID_ARG, "S_txt and S_img must be >= 0 (got %d, %d)", S_txt, S_img);
    if ((int64_t)S_txt + S_img > INT_MAX) return fail(DIT_ERR_INVALID_ARG, "S_txt + S_img overflows int");
    const int S = S_txt + S_img;
    dit_status_t st = check_shape(B, H, S, D);
    if (st != DIT_OK) return st;
    if ((st = check_rope(rope_cos, rope_sin)) != DIT_OK) return st;
    if (dtype == DIT_DTYPE_FP8_E4M3)
        return fail(DIT_ERR_UNSUPPORTED, "fp8 inputs go through dit_attn_forward_fp8 (it takes their scales)");
    if (dtype != DIT_DTYPE_BF16) return fail(DIT_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (!std::isfinite(scale)) return fail(DIT_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(DIT_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    const size_t tbytes = (size_t)B * H * S * D * 2;
    if (overlaps(out, tbytes, q, tbytes) || overlaps(out, tbytes, k, tbytes) || overlaps(out, tbytes, v, tbytes))
        return fail(DIT_ERR_INVALID_ARG, "out overlaps an input");
    if ((st = check_tables_apart(rope_cos, rope_sin, S, out, tbytes, nullptr, 0)) != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t need = dit_attn_workspace_bytes(B, H, S, D);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, need, s) != hipSuccess || ws == nullptr) {
        (void)hipGetLastError();
        return fail(DIT_ERR_OUT_OF_MEMORY, "hipMallocAsync of %zu workspace bytes failed", need);
    }
    hipError_t e = dit::launch_prepare_k(k, rope_cos, rope_sin, ws, ctl_of(ws, B, H, S), B * H, S, s);
    if (e == hipSuccess) {
        const float qmul = (float)((double)scale * 1.4426950408889634073599);
        e = dit::launch_attn_core(q, v, rope_cos, rope_sin, ws, static_cast<char*>(ws) + tiles_bytes(B, H, S),
                                  ctl_of(ws, B, H, S), out, nullptr, B * H, S, qmul, s);
    }
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e != hipSuccess) return launched(e, "dit_attn_forward kernels");
    return launched(ef, "hipFreeAsync of the workspace");
}

}  // extern "C"

// ---------------------------------------------------------------- MXFP4 linear layers

static dit_status_t check_mx_rows(int rows, int K, const char* what) {
    if (rows < 1 || K < 1) return fail(DIT_ERR_INVALID_ARG, "%s: rows and K must be >= 1 (got %d, %d)", what, rows, K);
    if ((int64_t)rows * K / 2 > INT_MAX)
        return fail(DIT_ERR_UNSUPPORTED, "%s: rows * K / 2 must be below 2^31 (got %d x %d)", what, rows, K);
    return DIT_OK;
}

static bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t dit_mxfp4_scale_bytes(int rows, int K) {
    if (rows < 1 || K < 32 || K % 32) return 0;
    return dit::mx_scale_bytes(rows, K);
}

dit_status_t dit_mxfp4_quantize(const void* x, void* codes, void* scales, int rows, int K, void* stream) {
    if (!x || !codes || !scales) return fail(DIT_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
    dit_status_t st = check_mx_rows(rows, K, "dit_mxfp4_quantize");
    if (st != DIT_OK) return st;
    if (K % 32) return fail(DIT_ERR_INVALID_ARG, "K must be a multiple of 32 (got %d)", K);
    if (!aligned16(x) || !aligned(codes, 4)) return fail(DIT_ERR_INVALID_ARG, "x must be 16-byte and codes 4-byte aligned");
    const size_t xb = (size_t)rows * K * 2, cb = (size_t)rows * K / 2, sb = dit::mx_scale_bytes(rows, K);
    if (overlaps(codes, cb, x, xb) || overlaps(scales, sb, x, xb) || overlaps(codes, cb, scales, sb))
        return fail(DIT_ERR_INVALID_ARG, "x, codes and scales must not overlap");
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_mxfp4_quantize(x, codes, scales, rows, K, static_cast<hipStream_t>(stream)),
                    "mxfp4_quantize_kernel");
}

static dit_status_t check_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                               const void* out, int M, int N, int K) {
    dit_status_t st;
    if ((st = check_mx_rows(M, K, "A")) != DIT_OK || (st = check_mx_rows(N, K, "W")) != DIT_OK) return st;
    if (K % 128) return fail(DIT_ERR_INVALID_ARG, "K must be a multiple of 128 (got %d)", K);
    if (N % 4) return fail(DIT_ERR_INVALID_ARG, "N must be a multiple of 4 (got %d)", N);
    if ((a_codes && !aligned16(a_codes)) || (w_codes && !aligned16(w_codes)))
        return fail(DIT_ERR_INVALID_ARG, "codes must be 16-byte aligned");
    if ((a_scales && !aligned(a_scales, 4)) || !aligned(w_scales, 4))
        return fail(DIT_ERR_INVALID_ARG, "scales must be 4-byte aligned");
    if (!aligned(out, 8)) return fail(DIT_ERR_INVALID_ARG, "out must be 8-byte aligned");
    const size_t ob = (size_t)M * N * 2;
    if ((a_codes && overlaps(out, ob, a_codes, (size_t)M * K / 2)) ||
        (a_scales && overlaps(out, ob, a_scales, dit::mx_scale_bytes(M, K))) ||
        overlaps(out, ob, w_codes, (size_t)N * K / 2) || overlaps(out, ob, w_scales, dit::mx_scale_bytes(N, K)))
        return fail(DIT_ERR_INVALID_ARG, "out overlaps an input");
    return DIT_OK;
}

dit_status_t dit_mxfp4_gemm(const void* a_codes, const void* a_scales, const void* w_codes, const void* w_scales,
                            void* out, int M, int N, int K, void* stream) {
    if (!a_codes || !a_scales || !w_codes || !w_scales || !out)
        return fail(DIT_ERR_INVALID_ARG, "codes, scales and out must be non-NULL");
    dit_status_t st = check_gemm(a_codes, a_scales, w_codes, w_scales, out, M, N, K);
    if (st != DIT_OK) return st;
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_mxfp4_gemm(a_codes, a_scales, w_codes, w_scales, out, M, N, K,
                                           static_cast<hipStream_t>(stream)),
                    "mxfp4_gemm_kernel");
}

dit_status_t dit_mxfp4_linear(const void* x, const void* w_codes, const void* w_scales, void* out, int M, int N,
                              int K, void* stream) {
    if (!x || !w_codes || !w_scales || !out) return fail(DIT_ERR_INVALID_ARG, "x, w_codes, w_scales and out must be non-NULL");
    dit_status_t st = check_gemm(nullptr, nullptr, w_codes, w_scales, out, M, N, K);
    if (st != DIT_OK) return st;
    if (!aligned16(x)) return fail(DIT_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if (overlaps(out, (size_t)M * N * 2, x, (size_t)M * K * 2)) return fail(DIT_ERR_INVALID_ARG, "out overlaps x");
    if ((st = check_device()) != DIT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t cb = ((size_t)M * K / 2 + 255) & ~(size_t)255, sb = dit::mx_scale_bytes(M, K);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, cb + sb, s) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DIT_ERR_OUT_OF_MEMORY, "could not allocate %zu bytes for the quantised activations", cb + sb);
    }
    void* codes = ws;
    void* scales = static_cast<char*>(ws) + cb;
    hipError_t e = dit::launch_mxfp4_quantize(x, codes, scales, M, K, s);
    if (e == hipSuccess) e = dit::launch_mxfp4_gemm(codes, scales, w_codes, w_scales, out, M, N, K, s);
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e == hipSuccess) e = ef;
    return launched(e, "mxfp4 linear");
}

// ---------------------------------------------------------------- DBCache reuse decision

size_t dit_dbcache_workspace_bytes(void) { return dit::residual_diff_workspace_bytes(); }

dit_status_t dit_dbcache_residual_diff(const void* prev, const void* cur, int64_t n, double threshold, void* ws,
                                       size_t ws_bytes, double* diff, int32_t* reuse, void* stream) {
    if (n < 0) return fail(DIT_ERR_INVALID_ARG, "n must be >= 0 (got %lld)", (long long)n);
    if (!ws || !diff || (n > 0 && (!prev || !cur)))
        return fail(DIT_ERR_INVALID_ARG, "ws, diff and (for n > 0) prev and cur must be non-NULL");
    if (n > ((int64_t)1 << 40)) return fail(DIT_ERR_UNSUPPORTED, "n must be at most 2^40 (got %lld)", (long long)n);
    const size_t need = dit::residual_diff_workspace_bytes();
    if (ws_bytes < need) return fail(DIT_ERR_INVALID_ARG, "workspace of %zu bytes is below the %zu needed", ws_bytes, need);
    if (!aligned16(prev) || !aligned16(cur) || !aligned16(ws))
        return fail(DIT_ERR_INVALID_ARG, "prev, cur and ws must be 16-byte aligned");
    if (!aligned(diff, 8) || (reuse && !aligned(reuse, 4)))
        return fail(DIT_ERR_INVALID_ARG, "diff must be 8-byte and reuse 4-byte aligned");
    const size_t nb = (size_t)n * 2;
    if (overlaps(ws, need, prev, nb) || overlaps(ws, need, cur, nb) || overlaps(ws, need, diff, 8) ||
        (reuse && overlaps(ws, need, reuse, 4)))
        return fail(DIT_ERR_INVALID_ARG, "the workspace overlaps an input or an output");
    if (overlaps(diff, 8, prev, nb) || overlaps(diff, 8, cur, nb) ||
        (reuse && (overlaps(reuse, 4, prev, nb) || overlaps(reuse, 4, cur, nb) || overlaps(reuse, 4, diff, 8))))
        return fail(DIT_ERR_INVALID_ARG, "diff or reuse overlaps an input or the other output");
    dit_status_t st;
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_residual_diff(prev, cur, n, threshold, ws, diff, reuse, static_cast<hipStream_t>(stream)),
                    "residual_diff kernels");
}

dit_status_t dit_dbcache_residual_diff_noalloc(const void* prev, const void* cur, int64_t n, double threshold,
                                               double* diff, int32_t* reuse, void* stream) {
    if (n < 0) return fail(DIT_ERR_INVALID_ARG, "n must be >= 0 (got %lld)", (long long)n);
    if (!diff || (n > 0 && (!prev || !cur)))
        return fail(DIT_ERR_INVALID_ARG, "diff and (for n > 0) prev and cur must be non-NULL");
    if (n > ((int64_t)1 << 40)) return fail(DIT_ERR_UNSUPPORTED, "n must be at most 2^40 (got %lld)", (long long)n);
    const size_t need = dit::residual_diff_workspace_bytes();
    if (need > dit::residual_diff_scratch_bytes())
        return fail(DIT_ERR_UNSUPPORTED, "the partials need %zu bytes, the static scratch holds %zu", need,
                    dit::residual_diff_scratch_bytes());
    if (!aligned16(prev) || !aligned16(cur)) return fail(DIT_ERR_INVALID_ARG, "prev and cur must be 16-byte aligned");
    if (!aligned(diff, 8) || (reuse && !aligned(reuse, 4)))
        return fail(DIT_ERR_INVALID_ARG, "diff must be 8-byte and reuse 4-byte aligned");
    const size_t nb = (size_t)n * 2;
    if (overlaps(diff, 8, prev, nb) || overlaps(diff, 8, cur, nb) ||
        (reuse && (overlaps(reuse, 4, prev, nb) || overlaps(reuse, 4, cur, nb) || overlaps(reuse, 4, diff, 8))))
        return fail(DIT_ERR_INVALID_ARG, "diff or reuse overlaps an input or the other output");
    dit_status_t st;
    if ((st = check_device()) != DIT_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(DIT_ERR_NO_DEVICE, "hipGetDevice failed");
    void* scratch = nullptr;
    const hipError_t e = dit::residual_diff_scratch(dev, &scratch);
    if (e != hipSuccess)
        return fail(DIT_ERR_LAUNCH, "address of the static scratch on device %d: %s", dev, hipGetErrorString(e));
    return launched(dit::launch_residual_diff(prev, cur, n, threshold, scratch, diff, reuse,
                                              static_cast<hipStream_t>(stream)),
                    "residual_diff kernels (static scratch)");
}

// ---------------------------------------------------------------- clock probe

dit_status_t dit_clock_probe(void* out, size_t out_bytes, int blocks, int iters, void* stream) {
    if (!out) return fail(DIT_ERR_INVALID_ARG, "out must be non-NULL");
    if (blocks < 1 || blocks > 65535) return fail(DIT_ERR_INVALID_ARG, "blocks must be in [1, 65535] (got %d)", blocks);
    if (iters < 1 || iters > (1 << 24)) return fail(DIT_ERR_INVALID_ARG, "iters must be in [1, 2^24] (got %d)", iters);
    if (out_bytes < (size_t)blocks * 4 * 24)
        return fail(DIT_ERR_INVALID_ARG, "out holds %zu bytes, %zu needed", out_bytes, (size_t)blocks * 4 * 24);
    if (!aligned(out, 8)) return fail(DIT_ERR_INVALID_ARG, "out must be 8-byte aligned");
    dit_status_t st;
    if ((st = check_device()) != DIT_OK) return st;
    return launched(dit::launch_clock_probe(blocks, iters, out, static_cast<hipStream_t>(stream)), "clock_probe_kernel");
}

dit_status_t dit_wall_clock_khz(int* khz) {
    if (!khz) return fail(DIT_ERR_INVALID_ARG, "khz must be non-NULL");
    dit_status_t st;
    if ((st = check_device()) != DIT_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(DIT_ERR_LAUNCH, "could not read the wall clock rate");
    }
    return ok();
}
