// split_step.hip -- standard decode step with the low-precision state modes
// (precision split, article section 4); the mode pieces are in split_common.h.
//
// A step runs as two launches.  The step kernel computes every row's output
// from the output source and appends the token to the buffer -- also the
// token that closes the interval: a slot that reaches L entries gets its new
// interval index (intv + 1) at once and is listed with it in the commit
// list.  The commit kernel then moves the call's positions on (pos + 1, or 0
// for a closed interval), and rewrites the listed slots' state (update
// checkpoint by stochastic rounding, FP4 copy) from the update source and
// the L buffered entries, one wave per head (or per half or quarter of a head
// when few slots commit), before any later launch reads it.  Keeping the
// commit out of the step kernel keeps the step's registers and LDS small (no
// spills, more waves per SIMD on the latency-bound steps), and spreads each
// interval's commit work over the whole chip whether the slots commit
// together (lock-step phases) or a few on every step (staggered phases).
// Accepts and flushes of the low-precision formats (article section 3) list
// their committing slots the same way, with each slot's entry count, set the
// positions themselves, and run the same commit pass, which then leaves the
// positions alone.
#include <atomic>
#include "split_common.h"

namespace rssm {

namespace {

// A commit-list entry: the slot with the number of entries it commits, and
// the interval index of the checkpoint the commit writes.
__device__ __forceinline__ int2 list_entry(int b, int K, int iv) {
    return make_int2(b | (K << kListCountShift), iv);
}

// The end of a row's step.  Positions stay as they are during the step
// (every workgroup of the row reads its slot's) and move on in the commit
// pass, which every step launches next, so no workgroup waits for the others
// of its row here.  The row's first workgroup marks the slot (a slot on two
// rows is marked twice, which the commit pass flags) and, when the step
// closes the interval (K == L), publishes the new interval index and lists
// the slot with it in the list the step fills (kListFill, fixed while the
// step runs).  The commit pass reads the entries only after the whole step.
__device__ __forceinline__ void step_arrive(const ReplayParams &a, const Slot &s, int K) {
    if (s.tile != 0 || threadIdx.x != 0) return;
    const int b = s.b;
    atomicAdd(&a.work[b], 1);   // result unused: nothing waits for it
    if (K == a.L) {
        const int e = a.clist[kListFill] & 1;
        const int iv = a.intv[b] + 1;
        a.intv[b] = iv;
        const int i = atomicAdd(&a.clist[e], 1);
        if (i < a.nslots) {
            *reinterpret_cast<int2 *>(a.clist + kListHead + (size_t)e * 2 * a.nslots + 2 * i) = list_entry(b, K, iv);
        } else {
            atomicOr(a.err, kErrDup);   // more listings than slots: rows repeated a slot
        }
    }
}

// Accept / flush (article section 3) for the low-precision formats, one
// thread per call row.  The row's slot holds K = pos + n_keep valid entries
// after an accept (K = pos for a flush), with the same range checks and
// flags as the fp32 accept; a slot that commits (K >= L; any K > 0 for a
// flush) gets its new interval index, is listed with it and K, and its
// position becomes 0, any other slot's becomes K.  The slot is marked like a
// step's; the commit pass that follows rewrites the listed slots from their
// K entries and checks and clears the marks.
template <bool ACCEPT>
__global__ void __launch_bounds__(256) split_accept_list_kernel(ReplayParams a) {
    if (blockIdx.x == 0 && threadIdx.x == 0) a.clist[kListLast] = a.clist[kListFill];
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= a.batch) return;
    const int b = a.slot_idx ? a.slot_idx[r] : r;
    if (b >= a.nslots || b < -1) {
        atomicOr(a.err, kErrSlot);
        return;
    }
    if (b < 0) return;   // padding row
    atomicAdd(&a.work[b], 1);
    // an accept follows a verify (k <= L - 1); a flush folds up to Lcap entries
    const int kmax = ACCEPT ? a.L - 1 : a.Lcap;
    int k = a.pos[b];
    if (k < 0 || k > kmax) {
        atomicOr(a.err, kErrPos);
        k = k < 0 ? 0 : kmax;
    }
    int nk = 0;
    if (ACCEPT) {
        nk = a.n_keep[r];
        if (nk < 0 || nk > a.T) {
            atomicOr(a.err, kErrKeep);
            nk = nk < 0 ? 0 : a.T;
        }
    }
    const int K = k + nk;
    const bool commit = ACCEPT ? K >= a.L : K > 0;
    if (commit) {
        const int e = a.clist[kListFill] & 1;
        const int iv = a.intv[b] + 1;
        a.intv[b] = iv;
        const int i = atomicAdd(&a.clist[e], 1);
        if (i < a.nslots) {
            *reinterpret_cast<int2 *>(a.clist + kListHead + (size_t)e * 2 * a.nslots + 2 * i) = list_entry(b, K, iv);
        } else {
            atomicOr(a.err, kErrDup);
        }
    }
    a.pos[b] = commit ? 0 : K;
}

// The positions of the call's rows after a step (run by the commit pass):
// k + 1, or 0 where the step closed the interval, with k the position the
// step read (clamped as the step did); the slot's mark is checked (one row per
// slot) and cleared.  The workgroup of rank w takes rows 64w + lane, then
// those a grid further on; the pass gives rank 0 to the workgroup with the
// last item, so on a short list these rows go to waves with no item, and
// the item waves' load chains do not wait for them.
template <bool MOVE>
__device__ __forceinline__ void advance_positions(const ReplayParams &a, int rank) {
    const int nthreads = gridDim.x * blockDim.x;
    for (int r = rank * blockDim.x + threadIdx.x; r < a.batch; r += nthreads) {
        const int b = a.slot_idx ? a.slot_idx[r] : r;
        if (b < 0 || b >= a.nslots) continue;   // padding, or flagged by the step
        if (a.work[b] != 1) atomicOr(a.err, kErrDup);
        if (MOVE) {
            int k = a.pos[b];
            k = k < 0 ? 0 : (k > a.L - 1 ? a.L - 1 : k);
            a.pos[b] = k + 1 == a.L ? 0 : k + 1;
        }
        a.work[b] = 0;
    }
}

// Waves per SIMD: the step is latency-bound, so as many as the registers
// allow without spilling.
template <typename TIn>
constexpr int step_waves(int kmax) { return sizeof(TIn) == 2 ? (kmax == 16 ? 6 : 5) : 4; }

template <typename TIn, int KMAX, int MODE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(step_waves<TIn>(KMAX))))
split_step_kernel(ReplayParams a) {
    using MT = ModeTraits<MODE>;
    constexpr int UB = MT::ubits;
    __shared__ StepSmemNoCommit<TIn, KMAX> sm;

    // the list this step fills, for the commit pass (which flips kListFill)
    if (blockIdx.x == 0 && threadIdx.x == 0) a.clist[kListLast] = a.clist[kListFill];
    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const int prow = MT::fp4_out ? s.lane : s.prow;   // FP4 output copy: a whole row per lane
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;

    // the position first (the prologue's first need), then the output-source
    // rows; the prologue runs under them
    const int pos_in = a.pos[s.b];
    Fp4Row o;
    typename Raw4<UB>::T raw[kNB][kPerChunk];   // update-source chunks (low modes)
    if constexpr (MT::fp4_out) {
        fp4_row_load(a, s, o);
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
        const float y0 = fp4_row_dot(o, sm.C);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + prow] = lam * y0 + ybuf;
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
    step_arrive(a, s, in.K);
}

// Commit pass over the listed slots: item = (listed slot, head, part), one
// wave per item rewriting its part of the head's 64 rows, as 16-row quarters
// on the matrix cores (lane layout of mfma_update), with no LDS and no
// barrier.  A part is the whole head when the list is long (every wave then
// has several heads to stream), and a half or a single quarter when it is
// short (a few slots closing their intervals on a step): then one head's
// quarters run on different waves instead of one after the other on a
// single one.  Per item the wave loads its A operands (the group's B
// entries, the same for all quarters), the x rows and the entries' steps
// once, computes the interval's weights once, and streams its quarters'
// source blocks with the next quarter's loads in flight under the current
// quarter's arithmetic.  Waves loop over the items, reading the next item's
// list entry ahead.  The step already published the slots, so the pass
// counts no arrivals: the waves only read the list, and its bookkeeping
// (which list the next step fills, that list's count cleared) is written by
// one wave in words no wave of the pass reads.

// Waves per SIMD of the commit pass: three where the registers allow it
// without spilling (bf16 inputs, up to 16 entries), two otherwise.
template <typename TIn>
constexpr int commit_waves(int kmax) { return sizeof(TIn) == 2 && kmax == 16 ? 3 : 2; }

template <typename TIn, int KMAX, int MODE, bool MOVE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(commit_waves<TIn>(KMAX))))
split_commit_list_kernel(ReplayParams a) {
    constexpr int UB = ModeTraits<MODE>::ubits;
    constexpr int NKB = KMAX / 4;
    // the wave's staging tile for the update checkpoint's rows (bf16 or E4M3)
    __shared__ __align__(16) uint8_t stage[16 * stage_pitch<UB>()];
    const int stride = gridDim.x;
    int it = xcd_remap(blockIdx.x, stride);   // consecutive items (a group's heads) on one XCD's L2
    // counts of both lists, the list the next step fills, the list the last
    // step filled, in one load, in flight while the positions move on
    const int4 hd = *reinterpret_cast<const int4 *>(a.clist);
    advance_positions<MOVE>(a, stride - 1 - it);
    const int e = __builtin_amdgcn_readfirstlane(hd.w) & 1;
    // (a count beyond the slots means rows repeated a slot, flagged by the
    // step; only the entries written are read)
    const int nlisted = min(__builtin_amdgcn_readfirstlane(e ? hd.y : hd.x), a.nslots);
    if (nlisted == 0) return;   // most steps: nothing closed an interval
    if (blockIdx.x == 0 && threadIdx.x == 0) {   // the next step fills the other list, from empty
        a.clist[1 - e] = 0;
        a.clist[kListFill] = 1 - e;
    }
    const int H = a.H;
    // parts per head: as many as keep every item on a wave of its own, one
    // when the heads alone fill the grid (the grid is the resident waves)
    const int parts = nlisted * H * 4 <= stride ? 4 : nlisted * H * 2 <= stride ? 2 : 1;
    const int nq = 4 / parts;          // quarters per item
    const int per_slot = H * parts;    // items per listed slot
    const int items = nlisted * per_slot;
    const int lane = threadIdx.x & 63, pl = lane & 15, g = lane >> 4;
    const size_t HP = (size_t)H * kP, GN = (size_t)a.G * kN;
    const int hpg = H / a.G;
    if (it >= items) return;
    // list entries (slot and entry count, interval index of the new
    // checkpoint); the next item's is read ahead, issued before the current
    // item's loads so that waiting for it never waits for those (past the
    // end: the last entry)
    const int2 *lst = reinterpret_cast<const int2 *>(a.clist + kListHead + (size_t)e * 2 * a.nslots);
    int2 cur = lst[it / per_slot];
    int2 nxt = lst[min(it + stride, items - 1) / per_slot];
    for (; it < items; it += stride) {
        const int li = it / per_slot;
        const int hq = it - li * per_slot;
        const int h = hq / parts;
        const int q0 = (hq - h * parts) * nq;   // the item's first quarter
        const int b = __builtin_amdgcn_readfirstlane(cur.x) & kListSlotMask;
        const int K = (int)((uint32_t)__builtin_amdgcn_readfirstlane(cur.x) >> kListCountShift);   // 1..KMAX
        const uint32_t interval = (uint32_t)__builtin_amdgcn_readfirstlane(cur.y);
        cur = nxt;
        nxt = lst[min(it + 2 * stride, items - 1) / per_slot];
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
        load_quarter(q0, raw0, x0);
        B8<TIn> bo[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            load_b8<TIn>(off_bytes(bb, (uint32_t)((jrow[kb] * (int)GN + 8 * pl) * sizeof(TIn))), bo[kb]);
        // l_i = A dt_i in lane i (zero from K on); Lambda_K and
        // w_j = dt_j exp(sum_{j<i<K} l_i) from one DPP suffix scan: lane i
        // holds sum_{m>=i} l_m, its right neighbour's value is lane i's
        // exclusive suffix and lane 0's the total.  (The stored bytes are the
        // rounding of this pass's own fp32 values, so the summation order
        // only has to keep those values within the parity bound.)
        const float dl = lane < K ? dt_l : 0.f;
        const float R = suffix_sum<KMAX>(Ah * dl, lane);
        const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R), 0));
        const float suf = dpp<kDppWaveShl1>(R);
        const float wj = lane < K ? dl * expf(suf) : 0.f;
        const float lam = expf(tot);
        float w[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) w[kb] = __shfl(wj, 4 * kb + g);
        // one quarter: coefficients w_j x_j[r] of the lane's row for entries
        // j = 4kb + g, the update, the rounding and the stores
        auto commit_quarter = [&](int q, RawBlock<UB> &raw, const float (&xq)[NKB]) {
            float cf[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) cf[kb] = 4 * kb + g < K ? w[kb] * xq[kb] : 0.f;
            float e[32];
            block_to_lanes<UB>(BlockAt{hrow0 + 16 * q, pl, g}, raw, stage);
            decode_block<UB>(raw, e);
            mfma_update<TIn, KMAX>(e, lam, cf, bo, g, K);
            quantize_store_block<MODE>(a, BlockAt{hrow0 + 16 * q, pl, g}, e, interval, stage);
        };
        // quarters in pairs, each one's loads in flight under the other's
        // arithmetic (static buffer names: a dynamic index would move the
        // buffers to scratch memory); an item of one quarter has no pair
        const int q1 = q0 + nq;
#pragma nounroll
        for (int q = q0; q < q1; q += 2) {
            if (q + 1 < q1) load_quarter(q + 1, raw1, x1);
            commit_quarter(q, raw0, x0);
            __builtin_amdgcn_sched_barrier(0);   // one quarter's arithmetic at a time
            if (q + 1 >= q1) break;
            if (q + 2 < q1) load_quarter(q + 2, raw0, x0);
            commit_quarter(q + 1, raw1, x1);
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
hipError_t split_step_t(const ReplayParams &p, int mode, dim3 g, dim3 b, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, hipLaunchKernelGGL((split_step_kernel<TIn, KMAX, M_>), g, b, 0, st, p));
    return hipGetLastError();
}

// Waves of the commit pass: as many as the chip holds at once (they loop
// over the items), and no more than the call's items.  A larger grid only
// queues waves behind the resident ones, and on a short list those late
// waves, each with an item, set the launch's length.  The resident count
// comes from the occupancy query, once per device and kernel.
constexpr int kMaxCommitDevices = 64;

template <typename TIn, int KMAX, int MODE, bool MOVE>
hipError_t split_commit_list_launch(const ReplayParams &p, long items, hipStream_t st) {
    static std::atomic<int> resident[kMaxCommitDevices];   // zero: not queried yet
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxCommitDevices) return hipErrorInvalidDevice;
    int waves = resident[dev].load(std::memory_order_relaxed);
    if (waves == 0) {
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_commit_list_kernel<TIn, KMAX, MODE, MOVE>, 64, 0);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        waves = per_cu * cus > 0 ? per_cu * cus : 1;
        resident[dev].store(waves, std::memory_order_relaxed);
    }
    const dim3 grid((unsigned)(items < waves ? items : waves));
    hipLaunchKernelGGL((split_commit_list_kernel<TIn, KMAX, MODE, MOVE>), grid, dim3(64), 0, st, p);
    return hipGetLastError();
}

template <typename TIn, int KMAX, bool MOVE>
hipError_t split_commit_list_t(const ReplayParams &p, int mode, long items, hipStream_t st) {
    RSSM_MODE_SWITCH(mode, return (split_commit_list_launch<TIn, KMAX, M_, MOVE>(p, items, st)));
    return hipSuccess;
}

// The commit pass over a list; the instance holds up to KMAX entries per
// slot (16 or 32), sized by the most a listed slot can hold.
template <bool MOVE>
hipError_t commit_list_pass(const ReplayParams &p, bool in_bf16, int mode, int kneed, hipStream_t stream) {
    const long items = (long)p.batch * p.H * 4;   // at most (slot, head, quarter) items
    if (kneed <= 16) return in_bf16 ? split_commit_list_t<uint16_t, 16, MOVE>(p, mode, items, stream)
                                    : split_commit_list_t<float, 16, MOVE>(p, mode, items, stream);
    return in_bf16 ? split_commit_list_t<uint16_t, 32, MOVE>(p, mode, items, stream)
                   : split_commit_list_t<float, 32, MOVE>(p, mode, items, stream);
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

hipError_t launch_split_commit_list(const ReplayParams &p, bool in_bf16, int mode, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    return commit_list_pass<true>(p, in_bf16, mode, p.L, stream);   // a step lists slots holding L entries
}

hipError_t launch_split_accept(const ReplayParams &p, bool in_bf16, int mode, bool accept, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    const dim3 grid((unsigned)((p.batch + 255) / 256)), block(256);
    if (accept) hipLaunchKernelGGL((split_accept_list_kernel<true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((split_accept_list_kernel<false>), grid, block, 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return commit_list_pass<false>(p, in_bf16, mode, p.Lcap, stream);   // a listed slot holds up to Lcap
}

}  // namespace rssm
