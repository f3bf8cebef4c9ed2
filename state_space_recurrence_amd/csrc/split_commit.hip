// split_commit.hip -- checkpoint loading for the low-precision state modes
// (article section 4).  Their accepts and flushes list the committing slots
// for the commit pass of split_step.hip.
#include "split_common.h"

namespace rssm {

namespace {

// Quantise an fp32 state into the mode's formats with stream index intv[b].
template <int MODE>
__global__ void __launch_bounds__(256) split_load_kernel(ReplayParams a) {
    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const uint32_t interval = (uint32_t)a.intv[s.b];
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;     // destination (state slot)
    const size_t srow = ((size_t)s.row * a.H + s.h) * kP + s.hf;   // source (call row)
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
        float4 st[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m)
            st[m] = stream_load4(a.src + (srow + 2 * chunk_index(q, m)) * kN + 4 * s.c);
#pragma unroll
        for (int m = 0; m < kPerChunk; m += 2) {
            quantize_store_rows<MODE>(a, hrow + 2 * chunk_index(q, m), hrow + 2 * chunk_index(q, m + 1), s.c,
                                      s.lane, st[m], st[m + 1], interval);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

#define RSSM_MODE_SWITCH(MODEVAR, CALL)                                  \
    switch (MODEVAR) {                                                    \
        case kSplitBF16: { constexpr int M_ = kSplitBF16; CALL; break; } \
        case kSplitE4M3: { constexpr int M_ = kSplitE4M3; CALL; break; } \
        case kSharedFP4: { constexpr int M_ = kSharedFP4; CALL; break; } \
        case kLowBF16: { constexpr int M_ = kLowBF16; CALL; break; }     \
        case kLowE4M3: { constexpr int M_ = kLowE4M3; CALL; break; }     \
        default: return hipErrorInvalidValue;                             \
    }

hipError_t split_load_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_load_kernel<M_>), g, b, 0, st, p));
    return hipGetLastError();
}

#undef RSSM_MODE_SWITCH

}  // namespace

hipError_t launch_split_load(const ReplayParams &p, int mode, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    return split_load_t(p, mode, grid, block, stream);
}

}  // namespace rssm
