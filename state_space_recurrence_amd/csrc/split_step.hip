// split_step.hip -- standard decode step with the low-precision state modes
// (precision split, article section 4); the mode pieces are in split_common.h.
#include "split_common.h"

namespace rssm {

namespace {

// Four waves per SIMD (six for split E4M3): the non-commit steps (all but one
// per interval) are latency-bound and gain more from the occupancy than the
// commit path, which holds the most registers, loses to the values the limit
// moves out (split E4M3 at six waves: +6% although its commit path spills).
template <typename TIn, int KMAX, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MODE == kSplitE4M3 ? 6 : 4))) split_step_kernel(ReplayParams a) {
    using MT = ModeTraits<MODE>;
    constexpr int UB = MT::ubits;
    __shared__ StepSmem<TIn, KMAX> sm;

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const int prow = MT::fp4_out ? fp4_prow(s.lane) : s.prow;
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;

    // output-source rows are requested first; the prologue runs under them
    Fp4Rows o;
    typename Raw4<UB>::T raw[kNB][kPerChunk];   // update-source chunks (low modes)
    if constexpr (MT::fp4_out) {
        fp4_rows_load(a, s, o);
    } else {
#pragma unroll
        for (int q = 0; q < kNB; ++q)
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) raw[q][m] = load_row4<UB>(a, hrow + 2 * chunk_index(q, m), s.c);
    }

    const StepIn in = step_inputs<TIn>(a, s, a.L - 1);
    // stream index of this step's commit, read on commit steps only: the
    // value is uniform, and loaded unconditionally the wave waited for it
    // right here, one memory latency ahead of the prologue's loads
    const uint32_t interval = in.commit ? (uint32_t)a.intv[s.b] + 1u : 0u;
    float lam, ybuf;
    step_prologue<TIn, KMAX>(a, s, in, prow, sm, &lam, &ybuf);

    if constexpr (MT::fp4_out) {
        float c8[1][8], y0[1];
        load_c8<TIn>(static_cast<const TIn *>(in.Cin), s.lane & 15, c8[0]);
        fp4_rows_dot<1>(o, c8, s.lane, y0);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + prow] = lam * y0[0] + ybuf;
        if (in.commit) commit_head<KMAX, MODE>(a, s, lam, sm.cs[s.wave], sm.u.B, interval);
    } else {
        const float4 C4 = io<TIn>::load4(static_cast<const TIn *>(in.Cin) + 4 * s.c);
        float r[kChunks];
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            float4 st[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) st[m] = decode_row4<UB>(raw[q % kNB][m]);
            if (q + kNB < kChunks) {
#pragma unroll
                for (int m = 0; m < kPerChunk; ++m)
                    raw[q % kNB][m] = load_row4<UB>(a, hrow + 2 * chunk_index(q + kNB, m), s.c);
            }
            float v[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(st[m], C4);
            r[q] = chunk_reduce8(v, s.lane);
            if (in.commit) commit_chunk_q<KMAX, MODE>(a, s, st, q, lam, sm.cs[s.wave], sm.u.B, interval);
        }
        const float y0 = chunk_combine4(r, s.lane);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + prow] = lam * y0 + ybuf;
    }

    if (!in.commit) step_append<TIn>(a, s, in);
    publish_position(a, s.b, in.commit ? 0 : in.K, in.commit, in.seen);
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
hipError_t split_step_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_step_kernel<TIn, KMAX, M_>), g, b, 0, st, p));
    return hipGetLastError();
}

#undef RSSM_MODE_SWITCH

}  // namespace

hipError_t launch_split_step(const ReplayParams &p, bool in_bf16, int mode, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    if (p.Lcap <= 16) return in_bf16 ? split_step_t<uint16_t, 16>(p, mode, grid, block, stream)
                                     : split_step_t<float, 16>(p, mode, grid, block, stream);
    return in_bf16 ? split_step_t<uint16_t, 32>(p, mode, grid, block, stream)
                   : split_step_t<float, 32>(p, mode, grid, block, stream);
}

}  // namespace rssm
