// dbcache.hip - the reuse decision of DBCache step caching.
//
// The AMD RDNA 4 xDiT blog (section on skipping transformer work when the
// model takes enough steps) turns on DBCache with a residual diff threshold:
// after the first Fn transformer blocks of a denoising step, the residual
// those blocks produced is compared with the one of the previous step, and
// when the two are close enough the rest of the step reuses cached work.  The
// page gives the threshold (0.12 in its example) but no formula; the
// difference computed here is the relative L1 distance
//
//     diff = sum_i |cur_i - prev_i| / sum_i |prev_i|,   reuse = diff < threshold,
//
// with diff = +inf (no reuse) when the previous residual is all zero.
//
// Two launches, no atomics and nothing to clear beforehand, so the result is
// bitwise reproducible for a given n and a launch can be captured in a graph:
//   residual_diff_partials  a grid of up to 32 blocks per CU streams both
//       residuals once in 16-byte loads (interleaved across the whole grid,
//       so consecutive lanes read consecutive chunks); each 8-element chunk
//       is summed in fp32 and folded into fp64 thread sums, which each block
//       reduces in a fixed order to one (num, den) pair.  Measured on the
//       16896 x 3072 residual, many short-lived blocks (about three chunks
//       per thread) beat fewer blocks that each keep several loads in flight.
//   residual_diff_finish    one block loads every pair at once (up to 32 per
//       thread), adds them in a fixed order and writes diff and the decision.
//
// Roofline: HBM bound.  Algorithmic bytes per element: 2 x 2 B read (bf16).
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "gfx950.h"

namespace dit {

constexpr int RD_THREADS = 256;
constexpr int RD_FINISH_PER_THREAD = 32;
constexpr int RD_MAX_BLOCKS = RD_THREADS * RD_FINISH_PER_THREAD;  // 32 blocks per CU
static_assert(RD_MAX_BLOCKS == MI355X_CUS * 32, "grid cap: 32 blocks per CU");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// |cur - prev| and |prev| of the 8 bf16 values in one 16-byte chunk, summed in fp32.
__device__ __forceinline__ void chunk_sums(const u32x4& p, const u32x4& c, float& num, float& den) {
    const uint32_t pw[4] = {p.x, p.y, p.z, p.w}, cw[4] = {c.x, c.y, c.z, c.w};
    float n = 0.f, d = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p0 = bf16_lo(pw[i]), p1 = bf16_hi(pw[i]);
        n += fabsf(bf16_lo(cw[i]) - p0) + fabsf(bf16_hi(cw[i]) - p1);
        d += fabsf(p0) + fabsf(p1);
    }
    num = n;
    den = d;
}

// Block-wide sum of two doubles in a fixed order (wave butterflies, then the
// waves' results in wave order).  Result valid in thread 0.
__device__ __forceinline__ void block_sum2(double& a, double& b) {
    __shared__ double red[2][RD_THREADS / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = a;
        red[1][wave] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a = red[0][0];
        b = red[1][0];
#pragma unroll
        for (int w = 1; w < RD_THREADS / 64; ++w) {
            a += red[0][w];
            b += red[1][w];
        }
    }
}

__global__ __launch_bounds__(RD_THREADS) void residual_diff_partials(const u32x4* __restrict__ prev,
                                                                    const u32x4* __restrict__ cur, int64_t n,
                                                                    double2* __restrict__ partials) {
    const int64_t nvec = n >> 3;
    const int64_t stride = (int64_t)gridDim.x * RD_THREADS;
    double num = 0.0, den = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x; i < nvec; i += stride) {
        float cn, cd;
        chunk_sums(__builtin_nontemporal_load(prev + i), __builtin_nontemporal_load(cur + i), cn, cd);
        num += cn;
        den += cd;
    }
    // the last n % 8 elements: one thread each, in block 0
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
        const uint16_t* p16 = reinterpret_cast<const uint16_t*>(prev);
        const uint16_t* c16 = reinterpret_cast<const uint16_t*>(cur);
        const int64_t i = (nvec << 3) + threadIdx.x;
        const float pv = __uint_as_float((uint32_t)p16[i] << 16), cv = __uint_as_float((uint32_t)c16[i] << 16);
        num += fabsf(cv - pv);
        den += fabsf(pv);
    }
    block_sum2(num, den);
    if (threadIdx.x == 0) partials[blockIdx.x] = make_double2(num, den);
}

__global__ __launch_bounds__(RD_THREADS) void residual_diff_finish(const double2* __restrict__ partials, int nparts,
                                                                  double threshold, double* __restrict__ diff,
                                                                  int32_t* __restrict__ reuse) {
    double2 v[RD_FINISH_PER_THREAD];
#pragma unroll
    for (int k = 0; k < RD_FINISH_PER_THREAD; ++k) {
        const int i = threadIdx.x + k * RD_THREADS;
        v[k] = i < nparts ? partials[i] : make_double2(0.0, 0.0);
    }
    double num = 0.0, den = 0.0;
#pragma unroll
    for (int k = 0; k < RD_FINISH_PER_THREAD; ++k) {
        num += v[k].x;
        den += v[k].y;
    }
    block_sum2(num, den);
    if (threadIdx.x == 0) {
        const double d = den == 0.0 ? (double)INFINITY : num / den;
        diff[0] = d;
        if (reuse) reuse[0] = d < threshold ? 1 : 0;
    }
}

int residual_diff_blocks(int64_t n) {
    const int64_t want = (n / 8 + RD_THREADS - 1) / RD_THREADS;
    return (int)std::max<int64_t>(1, std::min<int64_t>(want, RD_MAX_BLOCKS));
}

size_t residual_diff_workspace_bytes() { return (size_t)RD_MAX_BLOCKS * sizeof(double2); }

// Scratch of the allocation-free entry point: room for the (num, den) pair of
// every workgroup the partials launch can have (128 KiB).  Each GPU the
// library runs on holds its own copy until the process ends; calls on one GPU
// share it, so overlapping calls there race.  Nothing in it needs clearing:
// the finish kernel reads only the pairs the partials kernel of the same call
// wrote.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address comes from residual_diff_scratch().
static __device__ __align__(256) double2 scratch[RD_MAX_BLOCKS];

size_t residual_diff_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on device `dev`, which must be the current
// device: looked up once per device with hipGetSymbolAddress and kept.
hipError_t residual_diff_scratch(int dev, void** ptr) {
    constexpr int kDevices = 64;
    static std::mutex mu;
    static void* addr[kDevices];
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_residual_diff(const void* prev, const void* cur, int64_t n, double threshold, void* ws,
                                double* diff, int32_t* reuse, hipStream_t stream) {
    const int blocks = residual_diff_blocks(n);
    double2* partials = static_cast<double2*>(ws);
    residual_diff_partials<<<blocks, RD_THREADS, 0, stream>>>(static_cast<const u32x4*>(prev),
                                                             static_cast<const u32x4*>(cur), n, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    residual_diff_finish<<<1, RD_THREADS, 0, stream>>>(partials, blocks, threshold, diff, reuse);
    return hipGetLastError();
}

}  // namespace dit
