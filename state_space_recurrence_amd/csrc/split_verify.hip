// split_verify.hip -- speculative verify with the low-precision state modes
// (article sections 3 and 4): outputs of T drafts from the output source,
// no state written.
#include "split_common.h"

namespace rssm {

namespace {

template <typename TIn, int KMAX, int T, int MODE>
__global__ void __launch_bounds__(256) split_verify_kernel(ReplayParams a) {
    using MT = ModeTraits<MODE>;
    constexpr int UB = MT::ubits;
    __shared__ VerifySmemF<TIn, KMAX, KMAX, T> sm;
    __shared__ __align__(16) TIn sC[T][kN];   // the drafts' C, for row-per-lane output dots

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const int prow = MT::fp4_out ? s.lane : s.prow;   // FP4 output copy: a whole row per lane
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;

    // the position first (the prologue's first need), then the output-source
    // rows, then the prologue's loads, whose data the prologue waits for
    const int pos_in = a.pos[s.b];
    Fp4Row o;
    typename Raw4<UB>::T raw[32];
    if constexpr (MT::fp4_out) {
        fp4_row_load(a, s, o);
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) raw[i] = load_row4<UB>(a, hrow + 2 * i, s.c);
    }
    const VerifyIn in = verify_inputs<TIn, T>(a, s, a.L - 1, pos_in);
    VerifyPre<TIn, KMAX, KMAX, T> pre;
    verify_preload<TIn, KMAX, KMAX, T>(a, s, in, pre);
    if constexpr (MT::fp4_out) {   // staged ahead of the prologue, whose barriers publish it
        constexpr int per = 16 / (int)sizeof(TIn);   // elements per 16-byte piece
        for (int q = threadIdx.x; q < T * kN / per; q += blockDim.x) {
            const int t = q / (kN / per), c = per * (q - t * (kN / per));
            store16(&sC[t][c], load16(static_cast<const TIn *>(in.Cin) + (size_t)t * in.GN + c));
        }
    }
    float ybuf[T], lam[T];
    verify_finish<TIn, KMAX, KMAX, T>(a, s, in, pre, sm, prow, ybuf, lam);

    float y0[T];
    if constexpr (MT::fp4_out && sizeof(TIn) == 2) {
        fp4_row_dots<T>(o, sC, y0);
    } else if constexpr (MT::fp4_out) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            Fp4Row ot = o;   // decoded afresh per draft (holding 128 widened values would cost 64 VGPRs)
            if (T > 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    asm volatile("" : "+v"(ot.code[i].x), "+v"(ot.code[i].y), "+v"(ot.code[i].z), "+v"(ot.code[i].w));
            }
            y0[t] = fp4_row_dot(ot, sC[t]);
        }
    } else {
        float4 C4[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            C4[t] = io<TIn>::load4(static_cast<const TIn *>(in.Cin) + (size_t)t * in.GN + 4 * s.c);
        rows4_dot<UB, T>(raw, C4, s.lane, y0);
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
        a.y[((size_t)s.row * T + t) * in.HP + (size_t)s.h * kP + prow] = lam[t] * y0[t] + ybuf[t];
    verify_append<TIn, T>(a, s, in);
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

template <typename TIn, int KMAX, int T>
hipError_t split_verify_tt(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_verify_kernel<TIn, KMAX, T, M_>), g, b, 0, st, p));
    return hipGetLastError();
}

#undef RSSM_MODE_SWITCH

template <typename TIn, int KMAX>
hipError_t split_verify_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    switch (p.T) {
        case 1: return split_verify_tt<TIn, KMAX, 1>(p, mode, g, b, st);
        case 2: return split_verify_tt<TIn, KMAX, 2>(p, mode, g, b, st);
        case 3: return split_verify_tt<TIn, KMAX, 3>(p, mode, g, b, st);
        case 4: return split_verify_tt<TIn, KMAX, 4>(p, mode, g, b, st);
        case 5: return split_verify_tt<TIn, KMAX, 5>(p, mode, g, b, st);
        case 6: return split_verify_tt<TIn, KMAX, 6>(p, mode, g, b, st);
        case 7: return split_verify_tt<TIn, KMAX, 7>(p, mode, g, b, st);
        case 8: return split_verify_tt<TIn, KMAX, 8>(p, mode, g, b, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_verify(const ReplayParams &p, bool in_bf16, int mode, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    // entries per instance: 16, 24 (the 20-entry buffer of L = 16 with 4
    // drafts: 30.8 KB of LDS against 39.8 KB at 32, five workgroups per CU
    // instead of four) or 32
    if (p.Lcap <= 16) return in_bf16 ? split_verify_t<uint16_t, 16>(p, mode, grid, block, stream)
                                     : split_verify_t<float, 16>(p, mode, grid, block, stream);
    if (p.Lcap <= 24) return in_bf16 ? split_verify_t<uint16_t, 24>(p, mode, grid, block, stream)
                                     : split_verify_t<float, 24>(p, mode, grid, block, stream);
    return in_bf16 ? split_verify_t<uint16_t, 32>(p, mode, grid, block, stream)
                   : split_verify_t<float, 32>(p, mode, grid, block, stream);
}

}  // namespace rssm
