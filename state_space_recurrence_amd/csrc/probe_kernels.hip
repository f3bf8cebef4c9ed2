// probe_kernels.hip -- HBM streaming probes: the practical read and copy
// bandwidth of the device, measured with the same 16-byte non-temporal
// accesses the state-streaming kernels use.  Used to put the kernels'
// achieved bandwidth next to what the memory system sustains in practice.
#include "device_common.h"
#include "kernels.h"

namespace rssm {

namespace {

// Each thread keeps kProbeLoads independent 16-byte loads in flight per
// iteration (a workgroup reads kProbeLoads contiguous 4 KB pieces), so the
// probe is not limited by the latency of one outstanding load per thread.
constexpr int kProbeLoads = 8;

__global__ void __launch_bounds__(256) probe_read_kernel(const float *src, size_t n4, float *sink) {
    const size_t step = (size_t)gridDim.x * blockDim.x * kProbeLoads;
    float acc = 0.f;
    for (size_t base = (size_t)blockIdx.x * blockDim.x * kProbeLoads + threadIdx.x; base < n4; base += step) {
        float4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const size_t j = base + (size_t)u * blockDim.x;
            v[u] = j < n4 ? stream_load4(src + 4 * j) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;   // keeps the loads live
}

__global__ void __launch_bounds__(256) probe_copy_kernel(const float *src, float *dst, size_t n4) {
    const size_t step = (size_t)gridDim.x * blockDim.x * kProbeLoads;
    for (size_t base = (size_t)blockIdx.x * blockDim.x * kProbeLoads + threadIdx.x; base < n4; base += step) {
        float4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const size_t j = base + (size_t)u * blockDim.x;
            if (j < n4) v[u] = stream_load4(src + 4 * j);
        }
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) {
            const size_t j = base + (size_t)u * blockDim.x;
            if (j < n4) stream_store4(dst + 4 * j, v[u]);
        }
    }
}

// The replay step's own access shape: one wave per 32 KB block (a head),
// each lane reading 32 x 16 bytes in two halves of 16 loads, the workgroup's
// blocks consecutive.  Blocks past the end of the buffer are skipped.
__global__ void __launch_bounds__(256) probe_head_read_kernel(const float *src, size_t nblocks, float *sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float acc = 0.f;
    for (size_t blk = (size_t)blockIdx.x * 4 + wave; blk < nblocks; blk += (size_t)gridDim.x * 4) {
        const float *h = src + blk * (kP * kN) + 4 * lane;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = stream_load4(h + (size_t)(half * 16 + u) * 256);
#pragma unroll
            for (int u = 0; u < 16; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
        }
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_probe(int mode, const float *src, float *dst, size_t bytes, int grid, hipStream_t stream) {
    const size_t n4 = bytes / 16;
    if (mode == 0)
        hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, stream, src, n4, dst);
    else if (mode == 1)
        hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(256), 0, stream, src, dst, n4);
    else
        hipLaunchKernelGGL(probe_head_read_kernel, dim3(grid), dim3(256), 0, stream, src,
                           bytes / (kP * kN * 4), dst);
    return hipGetLastError();
}

}  // namespace rssm
