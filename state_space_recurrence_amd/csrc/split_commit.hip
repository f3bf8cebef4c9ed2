// split_commit.hip -- accept / flush commits and checkpoint loading for the
// low-precision state modes (article sections 3 and 4).
#include "split_common.h"

namespace rssm {

namespace {

template <typename TIn, int KMAX, bool ACCEPT, int MODE>
__global__ void __launch_bounds__(256) split_commit_kernel(ReplayParams a) {
    __shared__ CommitSmem<KMAX> sm;
    __shared__ float sB[KMAX][kN];
    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    bool commit;
    int seen;
    const int K = commit_count<ACCEPT>(a, s, &commit, &seen);
    if (commit) {
        const uint32_t interval = (uint32_t)a.intv[s.b] + 1u;   // read only where a commit needs it
        const size_t GN = (size_t)a.G * kN;
        const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
        stage_B<TIn, KMAX>(sB, bb, bb, GN, K, K);
        typename io<TIn>::raw4 unused[KMAX];
        const float lam = commit_prologue<TIn, KMAX, false>(a, s, K, sm.l, sm.w, sm.cs, unused);
        commit_head<KMAX, MODE>(a, s, lam, sm.cs[s.wave], sB, interval);
    }
    publish_position(a, s.b, commit ? 0 : K, commit, seen);
}

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

template <typename TIn, int KMAX>
hipError_t split_commit_t(const ReplayParams &p, int mode, bool accept, dim3 g, dim3 b, hipStream_t st) {
    if (accept) {
        RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_commit_kernel<TIn, KMAX, true, M_>), g, b, 0, st, p));
    } else {
        RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_commit_kernel<TIn, KMAX, false, M_>), g, b, 0, st, p));
    }
    return hipGetLastError();
}

hipError_t split_load_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_load_kernel<M_>), g, b, 0, st, p));
    return hipGetLastError();
}

#undef RSSM_MODE_SWITCH

}  // namespace

hipError_t launch_split_commit(const ReplayParams &p, bool in_bf16, int mode, bool accept, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    if (p.Lcap <= 16) return in_bf16 ? split_commit_t<uint16_t, 16>(p, mode, accept, grid, block, stream)
                                     : split_commit_t<float, 16>(p, mode, accept, grid, block, stream);
    return in_bf16 ? split_commit_t<uint16_t, 32>(p, mode, accept, grid, block, stream)
                   : split_commit_t<float, 32>(p, mode, accept, grid, block, stream);
}

hipError_t launch_split_load(const ReplayParams &p, int mode, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    return split_load_t(p, mode, grid, block, stream);
}

}  // namespace rssm
