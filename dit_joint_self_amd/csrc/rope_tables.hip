// rope_tables.hip - cos/sin tables of multi-axis RoPE, evaluated in fp64.
//
// The DiT pages (AMD RDNA 4 xDiT blog; xDiT paper abstract) describe attention
// over text tokens and a grid of latent patches but never write the position
// embedding out.  The reading implemented here: the head's D dims split into
// consecutive per-axis blocks; local pair i of axis a has frequency
// theta^(-2 i / d_a); the angle at token s is pos[s][a] times that frequency.
// One thread per (token, pair); fp64 angle, cos and sin, rounded to fp32.
// HBM bound and tiny (2 x S x D/2 fp32 written); not on the timed path.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

struct AxisSpec {
    int n_axes;
    int half_dim;      // D / 2 pairs per token
    int first_pair[4]; // global pair index where axis a starts
    int dim[4];        // axes_dim[a]
};

__global__ __launch_bounds__(256) void rope_tables_kernel(const int32_t* __restrict__ pos, int S,
                                                          AxisSpec ax, double log2_theta,
                                                          float* __restrict__ cos_t,
                                                          float* __restrict__ sin_t) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)S * ax.half_dim) return;
    const int64_t s = idx / ax.half_dim;
    const int j = (int)(idx - s * ax.half_dim);
    int a = 0;
#pragma unroll
    for (int t = 1; t < 4; ++t)
        if (t < ax.n_axes && j >= ax.first_pair[t]) a = t;
    const int i = j - ax.first_pair[a];
    const double freq = exp2(-(2.0 * i / ax.dim[a]) * log2_theta);
    const double ang = (double)pos[s * ax.n_axes + a] * freq;
    double sn, cs;
    sincos(ang, &sn, &cs);
    cos_t[idx] = (float)cs;
    sin_t[idx] = (float)sn;
}

hipError_t launch_rope_tables(const int32_t* pos, int S, int n_axes, const int32_t* axes_dim,
                              double theta, float* cos_t, float* sin_t, hipStream_t stream) {
    AxisSpec ax{};
    ax.n_axes = n_axes;
    int pairs = 0;
    for (int a = 0; a < n_axes; ++a) {
        ax.first_pair[a] = pairs;
        ax.dim[a] = axes_dim[a];
        pairs += axes_dim[a] / 2;
    }
    ax.half_dim = pairs;
    const int64_t n = (int64_t)S * pairs;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    rope_tables_kernel<<<blocks, 256, 0, stream>>>(pos, S, ax, log2(theta), cos_t, sin_t);
    return hipGetLastError();
}

}  // namespace dit
