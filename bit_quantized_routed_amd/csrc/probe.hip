// Machine ceilings for the benchmark (see moe_probe.h): a streaming
// HBM read and a bf16 MFMA loop, measured on the box the kernels run on.
#include "common.h"
#include "probe.h"

namespace moe {

namespace {

constexpr int PR_THREADS = 512;
constexpr int PR_DEPTH = 4;        // 16-byte loads in flight per thread

// NT: non-temporal loads (streamed data marked for early eviction)
template <bool NT>
__global__ __launch_bounds__(PR_THREADS) void probe_stream_kernel(const u32x4 *p, size_t n, u32x4 *sink)
{
    const size_t T = (size_t)gridDim.x * PR_THREADS, g = (size_t)blockIdx.x * PR_THREADS + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t b = g; b < n; b += T * PR_DEPTH) {
        u32x4 v[PR_DEPTH];
#pragma unroll
        for (int j = 0; j < PR_DEPTH; ++j) {
            const size_t i = b + (size_t)j * T;
            const size_t ic = i < n ? i : n - 1;
            v[j] = NT ? __builtin_nontemporal_load(&p[ic]) : p[ic];
            if (i >= n) v[j] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < PR_DEPTH; ++j) acc ^= v[j];
    }
    sink[g] = acc;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// SHAPE 0: v_mfma_f32_16x16x32_bf16 (16384 flop); 1: v_mfma_f32_32x32x16_bf16 (32768 flop)
template <int SHAPE>
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *sink)
{
    // operands depend on the thread so nothing folds; eight independent
    // accumulators keep the matrix pipe busy
    const int t = threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(1.0f + 0.001f * (float)((t + i) & 7));
        b[i] = (__bf16)(1.0f - 0.001f * (float)((t * 3 + i) & 7));
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = mfma16x16x32(a, b, c[j]);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    } else {
        f32x16 c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) c[j][v] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) s += c[j][v];
    }
    sink[(size_t)blockIdx.x * 256 + t] = s;
}

}  // namespace

hipError_t launch_probe_stream(const void *buf, size_t bytes, int grid, int nontemporal, void *sink, hipStream_t s)
{
    if (nontemporal) probe_stream_kernel<true><<<grid, PR_THREADS, 0, s>>>((const u32x4 *)buf, bytes / 16, (u32x4 *)sink);
    else probe_stream_kernel<false><<<grid, PR_THREADS, 0, s>>>((const u32x4 *)buf, bytes / 16, (u32x4 *)sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int shape, int grid, int iters, float *sink, hipStream_t s)
{
    if (shape == 0) probe_mfma_kernel<0><<<grid, 256, 0, s>>>(iters, sink);
    else probe_mfma_kernel<1><<<grid, 256, 0, s>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace moe
