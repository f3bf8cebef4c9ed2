// split_step.hip -- standard decode step with the low-precision state modes
// (precision split, article section 4); the mode pieces are in split_common.h.
//
// A step runs as two launches.  The step kernel computes every row's output
// from the output source and appends the token to the buffer -- also the
// token that closes the interval, so a slot that reaches L entries is left
// at pos == L and listed in the commit list.  The commit kernel then rewrites
// the listed slots' state (update checkpoint by stochastic rounding, FP4
// copy) from the update source and the L buffered entries, one workgroup per
// head with each wave taking a quarter of the head's rows, and publishes
// pos = 0, intv + 1.  Keeping the commit out of the step kernel keeps the
// step's registers and LDS small (no spills, more waves per SIMD on the
// latency-bound steps), and spreads each interval's commit work over the
// whole chip whether the slots commit together (lock-step phases) or a few
// on every step (staggered phases).
#include "split_common.h"

namespace rssm {

namespace {

// Last-arriving workgroup of slot b publishes its new position; when the
// step closed the interval (new_pos == L) it lists the slot for the commit
// kernel.  Duplicate rows are flagged as in publish_position.
__device__ __forceinline__ void publish_step(const ReplayParams &a, int b, int new_pos, int seen) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = atomicAdd(&a.work[b], 1);
        if (old >= a.wg_per_slot) atomicOr(a.err, kErrDup);
        if (old == a.wg_per_slot - 1) {
            if (a.pos[b] != seen) atomicOr(a.err, kErrDup);
            a.work[b] = 0;
            a.pos[b] = new_pos;
            if (new_pos == a.L) {
                const int i = atomicAdd(&a.clist[0], 1);
                if (i < a.nslots) a.clist[kListHead + i] = b;
                else atomicOr(a.err, kErrDup);   // more listings than slots: rows repeated a slot
            }
        }
    }
}

// Waves per SIMD: the step is latency-bound, so as many as the registers
// allow without spilling (six for bf16 inputs at 16 entries).
template <typename TIn>
constexpr int step_waves(int kmax) { return sizeof(TIn) == 2 ? (kmax == 16 ? 6 : 5) : (kmax == 16 ? 5 : 4); }

template <typename TIn, int KMAX, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(step_waves<TIn>(KMAX))))
split_step_kernel(ReplayParams a) {
    using MT = ModeTraits<MODE>;
    constexpr int UB = MT::ubits;
    __shared__ StepSmemNoCommit<TIn, KMAX> sm;

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

    StepIn in = step_inputs<TIn>(a, s, a.L - 1);
    in.commit = false;   // the interval-closing commit is the commit kernel's
    float lam, ybuf;
    step_prologue<TIn, KMAX>(a, s, in, prow, sm, &lam, &ybuf);

    if constexpr (MT::fp4_out) {
        float c8[1][8], y0[1];
        load_c8<TIn>(static_cast<const TIn *>(in.Cin), s.lane & 15, c8[0]);
        fp4_rows_dot<1>(o, c8, s.lane, y0);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + prow] = lam * y0[0] + ybuf;
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
        }
        const float y0 = chunk_combine4(r, s.lane);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + prow] = lam * y0 + ybuf;
    }

    step_append<TIn>(a, s, in);   // entry k, including the interval's last (k = L - 1)
    publish_step(a, s.b, in.K, in.seen);
}

// Commit pass over the listed slots: item = (listed slot, head), one
// workgroup per item, wave w rewrites the head's chunk w (rows 2(w + 4m) + hf).
// The workgroups loop over the items; the last slot to finish empties the
// list.
template <int KMAX>
struct ListCommitSmem {
    float B[KMAX][kN];      // the head's group's B entries, zero past K
    float cs[kP * KMAX];    // the head's commit coefficients (cs_index layout)
};

// Arrival of one head of listed slot b (list index li of n): the slot's last
// head publishes the commit (pos = 0, intv + 1) and counts the slot done in
// its group of list indices (li mod kListGroups); the last slot of a group
// counts the group, and the last group empties the list.  Items are assigned
// to workgroups statically, so a workgroup that still reads the list has
// items of its own pending and the list cannot have been emptied under it.
__device__ __forceinline__ void publish_listed(const ReplayParams &a, int b, int seen, int li, int n) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = atomicAdd(&a.work[b], 1);
        if (old >= a.wg_per_slot) atomicOr(a.err, kErrDup);
        if (old == a.wg_per_slot - 1) {
            if (a.pos[b] != seen) atomicOr(a.err, kErrDup);
            a.work[b] = 0;
            a.pos[b] = 0;
            a.intv[b] += 1;
            const int grp = li % kListGroups;
            const int ngrp = n < kListGroups ? n : kListGroups;
            const int members = (n - grp + kListGroups - 1) / kListGroups;
            if (atomicAdd(&a.clist[1 + grp], 1) == members - 1) {
                a.clist[1 + grp] = 0;
                if (atomicAdd(&a.clist[1 + kListGroups], 1) == ngrp - 1) {
                    a.clist[1 + kListGroups] = 0;
                    a.clist[0] = 0;
                }
            }
        }
    }
}

template <typename TIn, int KMAX, int MODE>
__global__ void __launch_bounds__(256) split_commit_list_kernel(ReplayParams a) {
    constexpr int UB = ModeTraits<MODE>::ubits;
    __shared__ ListCommitSmem<KMAX> sm;
    const int nlisted = a.clist[0];
    if (nlisted == 0) return;   // most steps: nothing closed an interval
    const int items = nlisted * a.H;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        Slot s;
        s.b = a.clist[kListHead + it / a.H];
        s.h = it - (it / a.H) * a.H;
        s.row = s.b;
        s.tile = s.h;
        s.wave = wave;
        s.lane = lane;
        s.hpg = a.H / a.G;
        s.g = s.h / s.hpg;
        s.c = lane & 31;
        s.hf = lane >> 5;
        s.prow = 2 * s.c + s.hf;
        int K = a.pos[s.b];
        const int seen = K;
        if (K < 1 || K > KMAX) {   // a listed slot holds L entries
            if (threadIdx.x == 0) atomicOr(a.err, kErrPos);
            K = K < 1 ? 1 : KMAX;
        }
        const uint32_t interval = (uint32_t)a.intv[s.b] + 1u;
        const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * HP + (size_t)s.h * kP;
        const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
        const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;
        // this wave's source rows first, the coefficients under them
        const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;
        typename Raw4<UB>::T raw[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) raw[m] = load_row4<UB>(a, hrow + 2 * chunk_index(wave, m), s.c);
        __syncthreads();   // the previous item's LDS reads are done
        stage_B<TIn, KMAX>(sm.B, bb, bb, GN, K, K);
        // l_i = A dt_i in lane i; Lambda_K and w_j = dt_j exp(sum_{j<i<K} l_i)
        // with the sums grown in ascending i (the commit arithmetic of every
        // other commit path)
        const float dl = lane < K ? io<TIn>::load1(db + (size_t)lane * a.H) : 0.f;
        const float l = a.A[s.h] * dl;
        float tot = 0.f, suf = 0.f;
        for (int i = 0; i < K; ++i) {
            const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
            tot += li;
            if (i > lane) suf += li;
        }
        const float wj = lane < K ? dl * expf(suf) : 0.f;
        const float lam = expf(tot);
        // coefficients w_j x_j[r] of all 64 rows, entries j = wave (mod 4)
        {
            const int i = s.prow >> 1;
#pragma unroll
            for (int j0 = 0; j0 < KMAX; j0 += 4) {
                const int j = j0 + wave;
                const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
                const int jj = j < K ? j : K - 1;
                const float cf = w * io<TIn>::load1(xb + (size_t)jj * HP + s.prow);
                sm.cs[cs_index<KMAX>(s.hf, i & 3, j, i >> 2)] = (j < K) ? cf : 0.f;
            }
        }
        __syncthreads();
        float4 st[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) st[m] = decode_row4<UB>(raw[m]);
        commit_chunk_q<KMAX, MODE>(a, s, st, wave, lam, sm.cs, sm.B, interval);
        publish_listed(a, s.b, seen, it / a.H, nlisted);
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
hipError_t split_step_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_step_kernel<TIn, KMAX, M_>), g, b, 0, st, p));
    return hipGetLastError();
}

template <typename TIn, int KMAX>
hipError_t split_commit_list_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_commit_list_kernel<TIn, KMAX, M_>), g, b, 0, st, p));
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

// Workgroups of the commit pass: enough for every head of the call's slots,
// at most four per CU of the chip (they loop over the items).
constexpr int kCommitListGrid = 1024;

hipError_t launch_split_commit_list(const ReplayParams &p0, bool in_bf16, int mode, hipStream_t stream) {
    if (p0.batch == 0) return hipSuccess;
    ReplayParams p = p0;
    p.wg_per_slot = p.H;   // one arrival per head of a committed slot
    const long heads = (long)p.batch * p.H;
    dim3 grid((unsigned)(heads < kCommitListGrid ? heads : kCommitListGrid)), block(256);
    if (p.L <= 16) return in_bf16 ? split_commit_list_t<uint16_t, 16>(p, mode, grid, block, stream)
                                   : split_commit_list_t<float, 16>(p, mode, grid, block, stream);
    return in_bf16 ? split_commit_list_t<uint16_t, 32>(p, mode, grid, block, stream)
                   : split_commit_list_t<float, 32>(p, mode, grid, block, stream);
}

}  // namespace rssm
