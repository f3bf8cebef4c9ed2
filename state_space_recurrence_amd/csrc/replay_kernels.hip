// replay_kernels.hip -- ReplaySSM decode kernels for gfx950, fp32 checkpoint.
//
// Method ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer",
// sections 1-3): a slot's SSM state is a checkpoint S0 from the start of the
// current interval plus the inputs (x, B, dt) of the k tokens since then.
// With l_i = A dt_i, Lambda_K = exp(sum_{i<K} l_i) and
// w_Kj = dt_j exp(sum_{j<i<K} l_i) (entries j = 0..K-1):
//     y    = Lambda_K (S0 . C) + sum_j w_Kj (B_j . C) x_j + D x_{K-1}
//     S_K  = Lambda_K S0 + sum_j w_Kj x_j (outer) B_j
//
// Work split: one workgroup = `hpw` (<= 4) heads of one slot that share a
// B/C group; one wave64 per head.  Each wave streams its head's 32 KB of
// checkpoint exactly once, in 4 chunks of 8 x 16-byte loads per lane (see
// device_common.h), with up to kNB chunks in flight; everything that does
// not depend on the checkpoint (decays, weights, the Gram row B_j . C, the
// buffer part of the output and the commit coefficients) is computed while
// the first chunks are in flight.  When the interval closes, each chunk's
// rows are rewritten in place right after they are consumed, so a commit
// step reads the checkpoint once and writes it once.
//
// Decays are formed as exp of segment sums of A dt (never as ratios of
// prefix products, which underflow to 0/0 over an interval).
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "replay_common.h"

namespace rssm {

namespace {

// ------------------------------------------------------------------------
// Standard decode step with fused interval commit.
// ------------------------------------------------------------------------
// Commit steps stage the group's B entries in LDS instead of holding KMAX raw
// slices per lane in registers (a commit happens once per interval; the
// registers are held on every step).  With them out of the register budget
// the 16-entry kernel runs three waves per SIMD (measured +5% over two waves
// with B in registers).
// The 64-entry instance keeps no coefficient table and its B entries as
// stored (StepSmemX): three workgroups per CU with bf16 inputs instead of one.
template <typename TIn>
constexpr int step64_waves() { return sizeof(TIn) == 2 ? 3 : 1; }

template <typename TIn, int KMAX>
using StepLds = typename std::conditional<KMAX == 64, StepSmemX<TIn, KMAX>, StepSmem<TIn, KMAX>>::type;

template <typename TIn, int KMAX>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(KMAX == 16 ? 3 : (KMAX == 64 ? step64_waves<TIn>() : 1))))
replay_step_kernel(ReplayParams a) {
    using SM = StepLds<TIn, KMAX>;
    __shared__ SM sm;

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const HeadState sp = head_state(a.ckpt, s, a.H);

    float4 buf[kNB][kPerChunk];
#pragma unroll
    for (int c = 0; c < kNB; ++c) load_chunk(buf[c], sp, c);

    const StepIn in = step_inputs<TIn>(a, s, a.kmax);
    const float4 C4 = io<TIn>::load4(static_cast<const TIn *>(in.Cin) + 4 * s.c);
    float lam, ybuf, wj = 0.f;
    step_prologue<TIn, KMAX>(a, s, in, s.prow, sm, &lam, &ybuf, &wj);

    float r[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        float4 (&cur)[kPerChunk] = buf[c % kNB];
        float v[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4);
        r[c] = chunk_reduce8(v, s.lane);
        if (in.commit) {
            if constexpr (SM::kCoefFromX)
                commit_chunk_x<TIn, KMAX>(cur, c, lam, wj, sm.u.X[s.wave], sm.u.B, s.hf, in.K, sp);
            else
                commit_chunk_lds<KMAX>(cur, c, lam, sm.cs[s.wave], sm.u.B, s.hf, (in.K + 3) & ~3, sp);
        }
        if (c + kNB < kChunks) load_chunk(cur, sp, c + kNB);
    }
    const float y0 = chunk_combine4(r, s.lane);
    a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + s.prow] = lam * y0 + ybuf;

    if (!in.commit) step_append<TIn>(a, s, in);
    publish_position(a, s.b, in.commit ? 0 : in.K, in.commit, in.seen);
}

// ------------------------------------------------------------------------
// Small-batch step: one workgroup per head, its 4 waves each stream one
// chunk (16 rows) of the head's checkpoint, so a batch-1 step spreads over
// H workgroups x 4 waves instead of H/4 workgroups.  Same arithmetic per row
// as replay_step_kernel (bit-identical results).
// ------------------------------------------------------------------------
template <typename TIn, int KMAX>
__global__ void __launch_bounds__(256) replay_step_rows_kernel(ReplayParams a) {
    __shared__ StepSmem<TIn, KMAX> sm;
    __shared__ float s_r[kChunks][kWave];

    Slot s;
    {
        const int wg = xcd_remap(blockIdx.x, gridDim.x);
        s.row = wg / a.H;
        s.tile = wg - s.row * a.H;
        s.b = slot_of_row(a, s.row);
        s.h = s.tile;
        s.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // = the chunk this wave streams (uniform)
        s.lane = threadIdx.x & 63;
        s.hpg = a.H / a.G;
        s.g = s.h / s.hpg;
        s.c = s.lane & 31;
        s.hf = s.lane >> 5;
        s.prow = 2 * s.c + s.hf;
    }
    if (s.b < 0) return;   // padding row
    const int q = s.wave;
    const HeadState sp = head_state(a.ckpt, s, a.H);
    float4 cur[kPerChunk];
    load_chunk(cur, sp, q);

    const StepIn in = step_inputs<TIn>(a, s, a.kmax);
    const float4 C4 = io<TIn>::load4(static_cast<const TIn *>(in.Cin) + 4 * s.c);
    float lam, ybuf;
    step_prologue<TIn, KMAX>(a, s, in, s.prow, sm, &lam, &ybuf);

    float v[kPerChunk];
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4);
    s_r[q][s.lane] = chunk_reduce8(v, s.lane);
    if (in.commit) commit_chunk_lds<KMAX>(cur, q, lam, sm.cs[s.wave], sm.u.B, s.hf, (in.K + 3) & ~3, sp);
    __syncthreads();
    if (q == 0) {
        float r[kChunks];
#pragma unroll
        for (int c = 0; c < kChunks; ++c) r[c] = s_r[c][s.lane];
        const float y0 = chunk_combine4(r, s.lane);
        a.y[(size_t)s.row * in.HP + (size_t)s.h * kP + s.prow] = lam * y0 + ybuf;
        if (!in.commit) step_append<TIn>(a, s, in);
    }
    publish_position(a, s.b, in.commit ? 0 : in.K, in.commit, in.seen);
}

// ------------------------------------------------------------------------
// Speculative verify: outputs of T draft positions, no state written.
// ------------------------------------------------------------------------
// The verify of one workgroup's heads (slot position k < L).
template <typename TIn, int KMAX, int T>
__device__ __forceinline__ void verify_body(const ReplayParams &a, const Slot &s, const VerifyIn &in,
                                            VerifySmemF<TIn, KMAX, KMAX, T> &sm) {
    const HeadState sp = head_state(a.ckpt, s, a.H);

    // prologue loads first (they retire before the checkpoint chunks)
    VerifyPre<TIn, KMAX, KMAX, T> pre;
    verify_preload<TIn, KMAX, KMAX, T>(a, s, in, pre);
    __builtin_amdgcn_sched_barrier(0);
    // chunks in the order 0, 2, 1, 3: the first butterfly stage of the
    // combine pairs chunk 0 with 2 and 1 with 3, so each pair closes as soon
    // as its second chunk is reduced
    float4 buf[kNB][kPerChunk];
    load_chunk(buf[0], sp, 0);
    load_chunk(buf[1], sp, 2);
    __builtin_amdgcn_sched_barrier(0);

    float ybuf[T], lam[T];
    verify_finish<TIn, KMAX, KMAX, T>(a, s, in, pre, sm, s.prow, ybuf, lam);
#pragma unroll
    for (int t = 0; t < T; ++t)   // uniform: keep it in a scalar register
        lam[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lam[t])));
    float4 C4[T];
#pragma unroll
    for (int t = 0; t < T; ++t) C4[t] = *reinterpret_cast<const float4 *>(&sm.G[in.KL + t][4 * s.c]);

    const bool up2 = (s.lane & 2) != 0;
    float r0[T], p02[T], p13[T];
    chunk_dots_1<T>(buf[0], C4, s.lane, r0);
    load_chunk(buf[0], sp, 1);
    {
        float r2[T];
        chunk_dots_1<T>(buf[1], C4, s.lane, r2);
#pragma unroll
        for (int t = 0; t < T; ++t) p02[t] = combine_pair(r0[t], r2[t], up2);
    }
    load_chunk(buf[1], sp, 3);
    chunk_dots_1<T>(buf[0], C4, s.lane, r0);   // chunk 1
    {
        float r3[T];
        chunk_dots_1<T>(buf[1], C4, s.lane, r3);
#pragma unroll
        for (int t = 0; t < T; ++t) p13[t] = combine_pair(r0[t], r3[t], up2);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float y0 = combine_last(p02[t], p13[t], (s.lane & 1) != 0);
        a.y[((size_t)s.row * T + t) * in.HP + (size_t)s.h * kP + s.prow] = lam[t] * y0 + ybuf[t];
    }
    verify_append<TIn, T>(a, s, in);
}

template <typename TIn, int KMAX, int T>
__global__ void __launch_bounds__(256) replay_verify_kernel(ReplayParams a) {
    __shared__ VerifySmemF<TIn, KMAX, KMAX, T> sm;

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const VerifyIn in = verify_inputs<TIn, T>(a, s, a.kmax);
    if (in.k >= a.L) return;   // layers with deferred commits use replay_verify_fold_kernel
    verify_body<TIn, KMAX, T>(a, s, in, sm);
}

// Verify on a slot a deferred accept left at pos >= L: fold the pos entries
// into the checkpoint while streaming it, then the drafts are entries
// 0..T-1 of the next interval (their outputs from the folded rows).  A
// commit: pos = 0, intv+1.
template <typename TIn, int KMAX, int T>
__device__ __forceinline__ void fold_body(const ReplayParams &a, const Slot &s, VerifyIn in,
                                          FoldSmem<TIn, KMAX, T> &sm) {
    const HeadState sp = head_state(a.ckpt, s, a.H);
    float4 buf[kNB][kPerChunk];   // chunks in the order 0, 2, 1, 3 (as in the verify kernel)
    load_chunk(buf[0], sp, 0);
    load_chunk(buf[1], sp, 2);

    float ybuf[T], lamt[T];
    float lam = fold_prologue<TIn, KMAX, T>(a, s, in.k, in, sm, ybuf, lamt);
    lam = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lam)));
#pragma unroll
    for (int t = 0; t < T; ++t)
        lamt[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, lamt[t])));
    float4 C4[T];   // the drafts' C rows, staged by the prologue (rows KL.. with KL = T)
#pragma unroll
    for (int t = 0; t < T; ++t) C4[t] = *reinterpret_cast<const float4 *>(&sm.v.G[T + t][4 * s.c]);
    const int Kr = (in.k + 3) & ~3;
    const bool up2 = (s.lane & 2) != 0;
    float r0[T], p02[T], p13[T];
    commit_chunk_lds<KMAX>(buf[0], 0, lam, sm.cs[s.wave], sm.B, s.hf, Kr, sp);
    chunk_dots_1<T>(buf[0], C4, s.lane, r0);
    load_chunk(buf[0], sp, 1);
    {
        float r2[T];
        commit_chunk_lds<KMAX>(buf[1], 2, lam, sm.cs[s.wave], sm.B, s.hf, Kr, sp);
        chunk_dots_1<T>(buf[1], C4, s.lane, r2);
#pragma unroll
        for (int t = 0; t < T; ++t) p02[t] = combine_pair(r0[t], r2[t], up2);
    }
    load_chunk(buf[1], sp, 3);
    commit_chunk_lds<KMAX>(buf[0], 1, lam, sm.cs[s.wave], sm.B, s.hf, Kr, sp);
    chunk_dots_1<T>(buf[0], C4, s.lane, r0);
    {
        float r3[T];
        commit_chunk_lds<KMAX>(buf[1], 3, lam, sm.cs[s.wave], sm.B, s.hf, Kr, sp);
        chunk_dots_1<T>(buf[1], C4, s.lane, r3);
#pragma unroll
        for (int t = 0; t < T; ++t) p13[t] = combine_pair(r0[t], r3[t], up2);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float y0 = combine_last(p02[t], p13[t], (s.lane & 1) != 0);
        a.y[((size_t)s.row * T + t) * in.HP + (size_t)s.h * kP + s.prow] = lamt[t] * y0 + ybuf[t];
    }
    in.k = 0;
    verify_append<TIn, T, false>(a, s, in);
    publish_fold<TIn>(a, s.b, 0, reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.row * T * in.GN, T, in.seen);
}

// Verify for layers that declare deferred commits: each workgroup folds or
// verifies by its slot's position, in one launch (no second pass over the
// grid for the folding slots, and the folding workgroups share the chip
// with the verifying ones).  The LDS is either pass's layout.
template <typename TIn, int KMAX, int FK, int T>
union VerifyFoldSmem {
    VerifySmemF<TIn, KMAX, KMAX, T> v;
    FoldSmem<TIn, FK, T> f;
};

template <typename TIn, int KMAX, int FK, int T>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FK <= 24 ? 3 : 1)))
replay_verify_fold_kernel(ReplayParams a) {
    __shared__ VerifyFoldSmem<TIn, KMAX, FK, T> sm;

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const VerifyIn in = verify_inputs<TIn, T>(a, s, a.kmax);
    if (in.k >= a.L)
        fold_body<TIn, FK, T>(a, s, in, sm.f);
    else
        verify_body<TIn, KMAX, T>(a, s, in, sm.v);
}

// ------------------------------------------------------------------------
// Accept (pos += n_keep, commit when the count reaches L) and flush
// (commit every slot holding buffered tokens).
// ------------------------------------------------------------------------
template <typename TIn, int KMAX, bool ACCEPT>
__global__ void __launch_bounds__(256) replay_commit_kernel(ReplayParams a) {
    __shared__ CommitSmem<KMAX> sm;
    __shared__ float sB[KMAX][kN];

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    bool commit;
    int seen;
    const int K = commit_count<ACCEPT>(a, s, &commit, &seen);
    if (commit) {
        const HeadState sp = head_state(a.ckpt, s, a.H);
        float4 buf[kNB][kPerChunk];
#pragma unroll
        for (int c = 0; c < kNB; ++c) load_chunk(buf[c], sp, c);
        const size_t GN = (size_t)a.G * kN;
        const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
        stage_B<TIn, KMAX>(sB, bb, bb, GN, K, K);
        typename io<TIn>::raw4 unused[KMAX];
        const float lam = commit_prologue<TIn, KMAX, false>(a, s, K, sm.l, sm.w, sm.cs, unused);
        const int Kr = (K + 3) & ~3;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            float4 (&cur)[kPerChunk] = buf[c % kNB];
            commit_chunk_lds<KMAX>(cur, c, lam, sm.cs[s.wave], sB, s.hf, Kr, sp);
            if (c + kNB < kChunks) load_chunk(cur, sp, c + kNB);
        }
    }
    publish_position(a, s.b, commit ? 0 : K, commit, seen);
}

// Deferred accept: pos += n_keep only; a slot reaching L keeps its entries
// until the next step, verify or flush on it folds them.
__global__ void defer_accept_kernel(ReplayParams a) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.batch) return;
    int b = row;
    if (a.slot_idx) {
        b = a.slot_idx[row];
        if (b >= a.nslots || b < -1) atomicOr(a.err, kErrSlot);
        if (b < 0 || b >= a.nslots) return;
    }
    int k = a.pos[b];
    if (k < 0 || k > a.L - 1) {
        atomicOr(a.err, kErrPos);
        k = k < 0 ? 0 : a.L - 1;
    }
    int nk = a.n_keep[row];
    if (nk < 0 || nk > a.T) {
        atomicOr(a.err, kErrKeep);
        nk = nk < 0 ? 0 : a.T;
    }
    a.pos[b] = k + nk;
}

__global__ void zero_pos_kernel(ReplayParams a) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= a.batch) return;
    const int b = a.slot_idx ? a.slot_idx[row] : row;
    if (b >= 0 && b < a.nslots) a.pos[b] = 0;
}

// ckpt[slot_idx[row]] <- src[row] for every mapped row (fp32 checkpoint); one
// workgroup per (row, head), 16-byte non-temporal copies.
__global__ void __launch_bounds__(256) load_f32_kernel(ReplayParams a) {
    const int row = blockIdx.x / a.H, h = blockIdx.x - row * a.H;
    const int b = a.slot_idx ? a.slot_idx[row] : row;
    if (b < 0 || b >= a.nslots) {
        if (threadIdx.x == 0 && (b < -1 || b >= a.nslots)) atomicOr(a.err, kErrSlot);
        return;
    }
    const float *src = a.src + ((size_t)row * a.H + h) * kP * kN;
    float *dst = a.ckpt + ((size_t)b * a.H + h) * kP * kN;
#pragma unroll
    for (int i = 0; i < kP * kN / 4 / 256; ++i) {
        const int e = 4 * (threadIdx.x + 256 * i);
        stream_store4(dst + e, stream_load4(src + e));
    }
}

}  // namespace

// ---------------------------------------------------------------- launchers --

// Below this many head-tile workgroups the chip is under-filled and the
// per-head row split is used instead.
constexpr int kRowSplitBelow = 512;

// Buffer entries a kernel instance handles: 16, 32 or 64.
#define RSSM_KMAX_DISPATCH(N, CALL)                  \
    do {                                             \
        if ((N) <= 16) { constexpr int KM_ = 16; CALL; } \
        else if ((N) <= 32) { constexpr int KM_ = 32; CALL; } \
        else { constexpr int KM_ = 64; CALL; }       \
    } while (0)

hipError_t launch_replay_step(const ReplayParams &p0, bool in_bf16, hipStream_t stream) {
    if (p0.batch == 0) return hipSuccess;
    const int kneed = p0.kmax + 1;   // a step folds up to kmax + 1 entries
    if (p0.batch * p0.wg_per_slot < kRowSplitBelow) {
        ReplayParams p = p0;
        p.hpw = 1;
        p.wg_per_slot = p.H;
        dim3 grid(p.batch * p.H), block(256);
        RSSM_KMAX_DISPATCH(kneed, {
            if (in_bf16) hipLaunchKernelGGL((replay_step_rows_kernel<uint16_t, KM_>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((replay_step_rows_kernel<float, KM_>), grid, block, 0, stream, p);
        });
        return hipGetLastError();
    }
    const ReplayParams &p = p0;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    RSSM_KMAX_DISPATCH(kneed, {
        if (in_bf16) hipLaunchKernelGGL((replay_step_kernel<uint16_t, KM_>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((replay_step_kernel<float, KM_>), grid, block, 0, stream, p);
    });
    return hipGetLastError();
}

// The fold pass folds up to Lcap entries; its LDS (commit coefficients and B
// per entry) is sized by FK = Lcap rounded up to 16, 24 or 32, which decides
// how many of its workgroups fit on a CU (three at 24: a 20-entry buffer).
template <typename TIn, int KMAX, int FK>
static void launch_verify_t(const ReplayParams &p, dim3 grid, dim3 block, hipStream_t stream) {
    switch (p.T) {
#define RSSM_VERIFY_CASE(TT)                                                                            \
    case TT:                                                                                            \
        if (p.kmax >= p.L)                                                                              \
            hipLaunchKernelGGL((replay_verify_fold_kernel<TIn, KMAX, FK, TT>), grid, block, 0, stream, p);  \
        else                                                                                            \
            hipLaunchKernelGGL((replay_verify_kernel<TIn, KMAX, TT>), grid, block, 0, stream, p);       \
        break;
        RSSM_VERIFY_CASE(1)
        RSSM_VERIFY_CASE(2)
        RSSM_VERIFY_CASE(3)
        RSSM_VERIFY_CASE(4)
        RSSM_VERIFY_CASE(5)
        RSSM_VERIFY_CASE(6)
        RSSM_VERIFY_CASE(7)
        RSSM_VERIFY_CASE(8)
#undef RSSM_VERIFY_CASE
        default: break;
    }
}

hipError_t launch_replay_verify(const ReplayParams &p, bool in_bf16, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    if (p.Lcap <= 16) {
        if (in_bf16) launch_verify_t<uint16_t, 16, 16>(p, grid, block, stream);
        else launch_verify_t<float, 16, 16>(p, grid, block, stream);
    } else if (p.Lcap <= 24) {
        if (in_bf16) launch_verify_t<uint16_t, 32, 24>(p, grid, block, stream);
        else launch_verify_t<float, 32, 24>(p, grid, block, stream);
    } else {
        if (in_bf16) launch_verify_t<uint16_t, 32, 32>(p, grid, block, stream);
        else launch_verify_t<float, 32, 32>(p, grid, block, stream);
    }
    return hipGetLastError();
}

// Entries a commit can fold: 16, 24, 32 or 64 (24 covers a 20-entry buffer:
// its coefficients and B take 37 KB of LDS, four workgroups per CU).
#define RSSM_COMMIT_KMAX_DISPATCH(N, CALL)             \
    do {                                               \
        if ((N) <= 16) { constexpr int KM_ = 16; CALL; } \
        else if ((N) <= 24) { constexpr int KM_ = 24; CALL; } \
        else if ((N) <= 32) { constexpr int KM_ = 32; CALL; } \
        else { constexpr int KM_ = 64; CALL; }         \
    } while (0)

hipError_t launch_replay_commit(const ReplayParams &p, bool in_bf16, bool accept, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    RSSM_COMMIT_KMAX_DISPATCH(p.Lcap, {
        if (in_bf16) {
            if (accept) hipLaunchKernelGGL((replay_commit_kernel<uint16_t, KM_, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((replay_commit_kernel<uint16_t, KM_, false>), grid, block, 0, stream, p);
        } else {
            if (accept) hipLaunchKernelGGL((replay_commit_kernel<float, KM_, true>), grid, block, 0, stream, p);
            else hipLaunchKernelGGL((replay_commit_kernel<float, KM_, false>), grid, block, 0, stream, p);
        }
    });
    return hipGetLastError();
}

hipError_t launch_defer_accept(const ReplayParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(defer_accept_kernel, dim3((p.batch + 255) / 256), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_zero_pos(const ReplayParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_pos_kernel, dim3((p.batch + 255) / 256), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_load_f32(const ReplayParams &p, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    hipLaunchKernelGGL(load_f32_kernel, dim3(p.batch * p.H), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ------------------------------------------------ no-allocation scratch --
// Per-slot arrival counters and the low-precision step's commit list for
// callers that cannot allocate (or bring) them: a file-scope device array,
// one copy per device, held until the process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) int32_t scratch[kNoAllocMaxSlots + list_words(kNoAllocMaxSlots)];

namespace {

__global__ void zero_i32_kernel(int32_t *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_work(int32_t **work, int32_t **clist, hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        // the counters must start at zero (every complete call leaves them so)
        hipLaunchKernelGGL(zero_i32_kernel, dim3(64), dim3(256), 0, stream, static_cast<int32_t *>(ptr),
                           (int)(kNoAllocMaxSlots + list_words(kNoAllocMaxSlots)));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<int32_t *>(ptr);
    }
    *work = g_scratch[dev];
    *clist = g_scratch[dev] + kNoAllocMaxSlots;
    return hipSuccess;
}

}  // namespace rssm
