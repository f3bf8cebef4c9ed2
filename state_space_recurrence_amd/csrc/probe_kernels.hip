// probe_kernels.hip -- HBM streaming probes: the practical read and copy
// bandwidth of the device, measured with the same 16-byte non-temporal
// accesses the state-streaming kernels use.  Used to put the kernels'
// achieved bandwidth next to what the memory system sustains in practice.
#include "device_common.h"
#include "kernels.h"

namespace rssm {

namespace {

__global__ void __launch_bounds__(256) probe_read_kernel(const float *src, size_t n4, float *sink) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    float acc = 0.f;
    for (; i < n4; i += stride) {
        const float4 v = stream_load4(src + 4 * i);
        acc += (v.x + v.y) + (v.z + v.w);
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;   // keeps the loads live
}

__global__ void __launch_bounds__(256) probe_copy_kernel(const float *src, float *dst, size_t n4) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n4; i += stride) stream_store4(dst + 4 * i, stream_load4(src + 4 * i));
}

}  // namespace

hipError_t launch_probe(int mode, const float *src, float *dst, size_t bytes, int grid, hipStream_t stream) {
    const size_t n4 = bytes / 16;
    if (mode == 0)
        hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, stream, src, n4, dst);
    else
        hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(256), 0, stream, src, dst, n4);
    return hipGetLastError();
}

}  // namespace rssm
