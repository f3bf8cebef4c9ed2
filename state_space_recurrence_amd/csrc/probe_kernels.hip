// probe_kernels.hip -- HBM streaming probes: the practical read and copy
// bandwidth of the device, measured with the same 16-byte non-temporal
// accesses the state-streaming kernels use.  Used to put the kernels'
// achieved bandwidth next to what the memory system sustains in practice.
// Also the self-check of the device conversions the low-precision commit
// relies on.
#include "device_common.h"
#include "kernels.h"
#include "quant.h"

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

// For every fp32 bit pattern in [begin, end), NaNs skipped: (0) gfx950's
// f32 -> E2M1 conversion at unit scale against the threshold encoding at
// scale 1 (the commit takes FP4 codes from the conversion of |v| / s
// bracketed from both sides, which is exact only if the conversion is the
// round-to-nearest-even, saturating, sign-keeping encoding everywhere);
// (1) for |v| <= 0x7F7F0000, bf16 stochastic rounding by integer addition
// against the selecting form, with a draw hashed from the pattern.  Each
// thread adds its mismatch counts to counts[0..1] only when nonzero.
__global__ void __launch_bounds__(256) conversion_check_kernel(uint64_t begin, uint64_t end,
                                                               unsigned long long *counts) {
    const Fp4Thresholds t = fp4_thresholds(1.0f);
    unsigned long long bad_fp4 = 0, bad_sr = 0, bad_e4m3 = 0;
    const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = begin + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < end; i += step) {
        const uint32_t bits = (uint32_t)i;
        const uint32_t mag = bits & 0x7FFFFFFFu;
        const float v = __uint_as_float(bits);
        uint32_t w = bits * 0x9E3779B1u;   // a draw hashed from the pattern
        w ^= w >> 15;
        w *= 0x85EBCA77u;
        w ^= w >> 13;
        const uint32_t r16 = w & 0xFFFFu;
        // E4M3 stochastic rounding, NaNs included, with the draw and its complement
        bad_e4m3 += (e4m3_sr(v, r16) != e4m3_sr_grid(v, r16)) + (e4m3_sr(v, r16 ^ 0xFFFFu) != e4m3_sr_grid(v, r16 ^ 0xFFFFu));
        if (mag > 0x7F800000u) continue;
        const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
        bad_fp4 += hw != fp4_encode(v, t, false);
        if (mag <= 0x7F7F0000u) bad_sr += ((bits + (r16 ^ 0xFFFFu)) >> 16) != bf16_sr(v, r16);
    }
    if (bad_fp4) atomicAdd(&counts[0], bad_fp4);
    if (bad_sr) atomicAdd(&counts[1], bad_sr);
    if (bad_e4m3) atomicAdd(&counts[2], bad_e4m3);
}

}  // namespace

hipError_t launch_conversion_check(uint64_t begin, uint64_t end, unsigned long long *counts, hipStream_t stream) {
    if (end <= begin) return hipSuccess;
    const uint64_t n = end - begin;
    const uint64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(conversion_check_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                       stream, begin, end, counts);
    return hipGetLastError();
}

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
