// split_step.hip -- standard decode step with the low-precision state modes
// (precision split, article section 4); the mode pieces are in split_common.h.
//
// A step runs as two launches.  The step kernel computes every row's output
// from the output source and appends the token to the buffer -- also the
// token that closes the interval, so a slot that reaches L entries is left
// at pos == L and listed in the commit list.  The commit kernel then rewrites
// the listed slots' state (update checkpoint by stochastic rounding, FP4
// copy) from the update source and the L buffered entries, one wave per
// head, and publishes pos = 0, intv + 1.  Keeping the commit out of the step kernel keeps the
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

    // the position first (the prologue's first need), then the output-source
    // rows; the prologue runs under them
    const int pos_in = a.pos[s.b];
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

    StepIn in = step_inputs<TIn>(a, s, a.L - 1, pos_in);
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

// Commit pass over the listed slots: item = (listed slot, head), one wave
// per item rewriting the head's 64 rows as four 16-row quarters on the
// matrix cores (lane layout of mfma_update), with no LDS and no barrier.
// Per item the wave loads its A operands (the group's B entries, the same
// for all quarters), the x rows of all quarters and the entries' steps
// once, computes the interval's weights once, and streams the quarters'
// source blocks with the next quarter's loads in flight under the current
// quarter's arithmetic.  Waves loop over the items, and an item's loads are
// issued before the previous item's arrival is counted, so the wait for
// that atomic (and for the stores before it) overlaps them.  The last wave
// of a slot publishes it; the last slot to finish empties the list.

// Arrival of one wave of listed slot b (list index li of n), counted by its
// lane 0 with the value `old` its atomicAdd on the slot's counter returned:
// the slot's last wave publishes the commit (pos = 0, intv + 1) and counts
// the slot done in its group of list indices (li mod kListGroups); the last
// slot of a group counts the group, and the last group empties the list.
// Items are assigned to waves statically and a wave reads the list entry of
// its next item before its current item arrives, so the list cannot be
// emptied under a wave that still reads it.
__device__ __forceinline__ void finish_arrival(const ReplayParams &a, int old, int b, int seen, int li, int n) {
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

// Waves per SIMD of the commit pass: three where the registers allow it
// without spilling (bf16 inputs, up to 16 entries), two otherwise.
template <typename TIn>
constexpr int commit_waves(int kmax) { return sizeof(TIn) == 2 && kmax == 16 ? 3 : 2; }

template <typename TIn, int KMAX, int MODE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(commit_waves<TIn>(KMAX))))
split_commit_list_kernel(ReplayParams a) {
    constexpr int UB = ModeTraits<MODE>::ubits;
    constexpr int NKB = KMAX / 4;
    // the wave's staging tile for the update checkpoint's rows (bf16 or E4M3)
    __shared__ __align__(16) uint8_t stage[16 * (kN * (UB >= 8 ? UB / 8 : 1) + 16)];
    const int nlisted = a.clist[0];
    if (nlisted == 0) return;   // most steps: nothing closed an interval
    const int H = a.H;
    const int items = nlisted * H;
    const int lane = threadIdx.x & 63, pl = lane & 15, g = lane >> 4;
    const size_t HP = (size_t)H * kP, GN = (size_t)a.G * kN;
    const int hpg = H / a.G;
    const int stride = gridDim.x;
    int it = blockIdx.x;
    if (it >= items) return;
    // Slot facts are read ahead: the list entry two items ahead and the
    // position and stream index one item ahead, each issued before the
    // current item's loads so that waiting for them never waits for those.
    // Indices past the end re-read the last item's entries.
    const int *lst = a.clist + kListHead;
    int b = __builtin_amdgcn_readfirstlane(lst[it / H]);
    int pos = __builtin_amdgcn_readfirstlane(a.pos[b]);
    int intv = __builtin_amdgcn_readfirstlane(a.intv[b]);
    int nb = lst[min(it + stride, items - 1) / H];
    int pend_old = 0, pend_b = -1, pend_seen = 0, pend_li = 0;
    for (; it < items; it += stride) {
        const int li = it / H;
        const int h = it - li * H;
        const int nb_u = __builtin_amdgcn_readfirstlane(nb);
        const int npos = a.pos[nb_u], nintv = a.intv[nb_u];
        const int nnb = lst[min(it + 2 * stride, items - 1) / H];
        int K = pos;
        if (K != a.L) {   // a listed slot holds L entries
            if (lane == 0) atomicOr(a.err, kErrPos);
            K = K < 1 ? 1 : (K > a.L ? a.L : K);
        }
        const uint32_t interval = (uint32_t)intv + 1u;
        const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)b * a.Lcap * HP + (size_t)h * kP;
        const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)b * a.Lcap * GN + (size_t)(h / hpg) * kN;
        const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)b * a.Lcap * H + h;
        const size_t hrow0 = ((size_t)b * H + h) * kP;   // the head's first state row
        // loads in the order they are consumed: steps, x rows, quarter 0's
        // source block, A operands
        const float dt_l = io<TIn>::load1(off_bytes(db, (uint32_t)((lane < K ? lane : K - 1) * H * sizeof(TIn))));
        const float Ah = a.A[h];
        int jrow[NKB];   // the lane's entries 4kb + g, clamped into the interval
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) jrow[kb] = 4 * kb + g < K ? 4 * kb + g : K - 1;
        uint32_t xoff[NKB];   // byte offsets of the lane's x_j[pl] from the head's quarter
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) xoff[kb] = (uint32_t)((jrow[kb] * (int)HP + pl) * sizeof(TIn));
        // x rows and source block of a quarter
        auto load_quarter = [&](int q, RawBlock<UB> &raw, float (&xq)[NKB]) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) xq[kb] = io<TIn>::load1(off_bytes(xb + 16 * q, xoff[kb]));
            load_block<UB>(a, BlockAt{hrow0 + 16 * q, pl, g}, raw);
        };
        RawBlock<UB> raw0, raw1;
        float x0[NKB], x1[NKB];
        load_quarter(0, raw0, x0);
        B8<TIn> bo[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            load_b8<TIn>(off_bytes(bb, (uint32_t)((jrow[kb] * (int)GN + 8 * pl) * sizeof(TIn))), bo[kb]);
        // the previous item's arrival (its atomic was issued before these loads)
        if (pend_b >= 0 && lane == 0) finish_arrival(a, pend_old, pend_b, pend_seen, pend_li, nlisted);
        // l_i = A dt_i in lane i; Lambda_K and w_j = dt_j exp(sum_{j<i<K} l_i)
        // with the sums grown in ascending i (the commit arithmetic of every
        // other commit path)
        const float dl = lane < K ? dt_l : 0.f;
        const float l = Ah * dl;
        float tot = 0.f, suf = 0.f;
        for (int i = 0; i < K; ++i) {
            const float li_ = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
            tot += li_;
            if (i > lane) suf += li_;
        }
        const float wj = lane < K ? dl * expf(suf) : 0.f;
        const float lam = expf(tot);
        float w[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) w[kb] = __shfl(wj, 4 * kb + g);
        // one quarter: coefficients w_j x_j[r] of the lane's row for entries
        // j = 4kb + g, the update, the rounding and the stores
        auto commit_quarter = [&](int q, const RawBlock<UB> &raw, const float (&xq)[NKB]) {
            float cf[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) cf[kb] = 4 * kb + g < K ? w[kb] * xq[kb] : 0.f;
            float e[32];
            decode_block<UB>(raw, e);
            mfma_update<TIn, KMAX>(e, lam, cf, bo, g, K);
            quantize_store_block<MODE>(a, BlockAt{hrow0 + 16 * q, pl, g}, e, interval, stage);
        };
        // quarters in pairs, each one's loads in flight under the other's
        // arithmetic (static buffer names: a dynamic index would move the
        // buffers to scratch memory)
#pragma nounroll
        for (int q = 0; q < 4; q += 2) {
            load_quarter(q + 1, raw1, x1);
            commit_quarter(q, raw0, x0);
            __builtin_amdgcn_sched_barrier(0);   // one quarter's arithmetic at a time
            if (q + 2 < 4) load_quarter(q + 2, raw0, x0);
            commit_quarter(q + 1, raw1, x1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // the arrival: an address the compiler cannot prove uniform keeps the
        // atomic a single-lane one whose result is waited for only where the
        // next item uses it
        int zero = 0;
        asm volatile("" : "+v"(zero));
        if (lane == 0) pend_old = atomicAdd(&a.work[b + zero], 1);
        pend_b = b;
        pend_seen = pos;
        pend_li = li;
        b = nb_u;
        pos = __builtin_amdgcn_readfirstlane(npos);
        intv = __builtin_amdgcn_readfirstlane(nintv);
        nb = nnb;
    }
    if (lane == 0) finish_arrival(a, pend_old, pend_b, pend_seen, pend_li, nlisted);
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

// Waves of the commit pass: enough for every item (slot, head) of the call's
// slots, at most sixteen per CU of the chip (they loop over the items).
constexpr int kCommitListGrid = 4096;

hipError_t launch_split_commit_list(const ReplayParams &p0, bool in_bf16, int mode, hipStream_t stream) {
    if (p0.batch == 0) return hipSuccess;
    ReplayParams p = p0;
    p.wg_per_slot = p.H;   // one arrival per wave (one head) of a committed slot
    const long items = (long)p.batch * p.wg_per_slot;
    dim3 grid((unsigned)(items < kCommitListGrid ? items : kCommitListGrid)), block(64);
    if (p.L <= 16) return in_bf16 ? split_commit_list_t<uint16_t, 16>(p, mode, grid, block, stream)
                                   : split_commit_list_t<float, 16>(p, mode, grid, block, stream);
    return in_bf16 ? split_commit_list_t<uint16_t, 32>(p, mode, grid, block, stream)
                   : split_commit_list_t<float, 32>(p, mode, grid, block, stream);
}

}  // namespace rssm
