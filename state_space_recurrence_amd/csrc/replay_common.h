// replay_common.h -- pieces shared by the fp32 and the low-precision replay
// kernels: workgroup -> (slot, head) mapping, position publication, the
// per-chunk commit of fp32 rows and the LDS layout of commit coefficients.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace rssm {
namespace {

constexpr int kMaxHpw = 4;
constexpr int kNB = 2;   // checkpoint chunks in flight per wave

struct Slot {
    int b;     // state slot (checkpoint, buffers, pos, intv); < 0: padding row, nothing to do
    int row;   // call row (inputs x, B, C, dt, n_keep and outputs y)
    int tile, wave, lane, h, g, c, hf, prow, hpg;
};

// State slot of call row `row`: slot_idx[row], or `row` without a map.  Rows
// mapped outside 0..nslots-1 are flagged and treated as padding.
__device__ __forceinline__ int slot_of_row(const ReplayParams &a, int row) {
    if (!a.slot_idx) return row;
    const int b = a.slot_idx[row];
    if (b >= a.nslots || b < -1) {
        if (threadIdx.x == 0) atomicOr(a.err, kErrSlot);
        return -1;
    }
    return b;
}

// Slot, head tile and lane roles of logical workgroup `wg`.
__device__ __forceinline__ Slot slot_at(const ReplayParams &a, int wg) {
    Slot s;
    s.row = wg / a.wg_per_slot;
    s.tile = wg - s.row * a.wg_per_slot;
    s.b = slot_of_row(a, s.row);
    s.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: head math in scalar registers
    s.lane = threadIdx.x & 63;
    s.h = s.tile * a.hpw + s.wave;
    s.hpg = a.H / a.G;
    s.g = (s.tile * a.hpw) / s.hpg;
    s.c = s.lane & 31;
    s.hf = s.lane >> 5;
    s.prow = 2 * s.c + s.hf;
    return s;
}

__device__ __forceinline__ Slot slot_of(const ReplayParams &a) {
    return slot_at(a, xcd_remap(blockIdx.x, gridDim.x));
}

// Head (b,h) of an fp32 state (64 x 128, 32 KB) as a buffer resource: the
// head's base address is wave-uniform and sits in scalar registers, the lane
// adds one 32-bit byte offset vo (row hf, columns 4c..4c+3) and each row
// access a constant offset (value index i adds i * 2 rows).  Loads carry the
// row offset in the scalar offset operand, so the 32 row loads of a lane
// share a single address register; the hardware range check does not cover
// that operand, and vo + row offset <= 32 KB - 16 holds by construction
// (0 <= vo <= 1008, row offsets 0..31744).  Stores (commits only) put the
// row offset into the vector operand (see buffer_stream_store4).
struct HeadState {
    __amdgpu_buffer_rsrc_t r;
    int vo;
};

__device__ __forceinline__ HeadState head_state(float *base, const Slot &s, int H) {
    float *hb = base + (size_t)(s.b * H + s.h) * kP * kN;
    const uint64_t u = reinterpret_cast<uint64_t>(hb);   // uniform; pinned to scalar registers
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u), hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    HeadState hs;
    hs.r = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0, kP * kN * 4,
                                             kBufferRsrcWord3);
    hs.vo = (s.hf * kN + 4 * s.c) * 4;
    return hs;
}

__device__ __forceinline__ int row_offset(int c, int m) { return chunk_index(c, m) * 2 * kN * 4; }

__device__ __forceinline__ void load_chunk(float4 (&buf)[kPerChunk], const HeadState &hs, int c) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) buf[m] = buffer_stream_load4(hs.r, hs.vo, row_offset(c, m));
}

__device__ __forceinline__ void store_chunk(const HeadState &hs, int c, const float4 (&st)[kPerChunk]) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) buffer_stream_store4(hs.r, hs.vo + row_offset(c, m), st[m]);
}

// Last-arriving workgroup of slot b publishes the slot's new position (and
// interval count).  Every workgroup of the slot read pos[b] (as `seen`, or
// -1 where the caller checks it otherwise) before arriving.  Two rows of one
// call on the same slot are a race the caller must avoid; it shows up as more
// than wg_per_slot arrivals before a reset, or as a position that changed
// between a workgroup's read and its publication, and is flagged (kErrDup).
__device__ __forceinline__ void publish_position(const ReplayParams &a, int b, int new_pos,
                                                 bool committed, int seen) {
    __syncthreads();
    if (threadIdx.x == 0) {
        int old = atomicAdd(&a.work[b], 1);
        if (old >= a.wg_per_slot) atomicOr(a.err, kErrDup);
        if (old == a.wg_per_slot - 1) {
            if (seen >= 0 && a.pos[b] != seen) atomicOr(a.err, kErrDup);
            a.work[b] = 0;
            a.pos[b] = new_pos;
            if (committed) a.intv[b] += 1;
        }
    }
}

// Commit coefficients cs = w_j x_j[r] live in LDS as [hf][c][j][m] for row
// r = 2(c + 4m) + hf, so the 8 coefficients one chunk needs for entry j are
// two contiguous 16-byte reads (the same address across a half-wave).
template <int KMAX>
__device__ __forceinline__ int cs_index(int hf, int c, int j, int m) {
    return ((hf * kChunks + c) * KMAX + j) * kPerChunk + m;
}

// Stage the group's B entries 0..KMAX-1 of a commit into LDS as fp32 (the
// workgroup's heads share one group): entries j < nbuf from the buffer, entry
// nbuf (when < K) from the current input, entries >= K zero.  Visible after
// the next __syncthreads.
// Four pieces per thread are requested together (entries past K re-read
// entry K - 1 and are zeroed afterwards), so the staging waits for one
// memory latency, not one per piece.
template <typename TIn, int KMAX>
__device__ __forceinline__ void stage_B(float (*sB)[kN], const TIn *bb, const TIn *Bin, size_t GN, int nbuf,
                                        int K) {
    constexpr int total = KMAX * kN / 4;
    for (int q0 = threadIdx.x; q0 < total; q0 += 4 * blockDim.x) {
        typename io<TIn>::raw4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int q = q0 + u * blockDim.x;
            q = q < total ? q : total - 1;
            int j = q / (kN / 4);
            const int n = 4 * (q - j * (kN / 4));
            j = j < K ? j : K - 1;
            r[u] = io<TIn>::load_raw4((j < nbuf ? bb + (size_t)j * GN : Bin) + n);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * blockDim.x;
            if (q < total) {
                const int j = q / (kN / 4), n = 4 * (q - j * (kN / 4));
                const float4 v = io<TIn>::widen(r[u]);
                *reinterpret_cast<float4 *>(&sB[j][n]) = j < K ? v : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }
}

// stage_B keeping the entries as stored (TIn), zero past K.
template <typename TIn, int KMAX>
__device__ __forceinline__ void stage_B_raw(TIn (*sB)[kN], const TIn *bb, const TIn *Bin, size_t GN, int nbuf,
                                            int K) {
    constexpr int total = KMAX * kN / 4;
    for (int q0 = threadIdx.x; q0 < total; q0 += 4 * blockDim.x) {
        typename io<TIn>::raw4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int q = q0 + u * blockDim.x;
            q = q < total ? q : total - 1;
            int j = q / (kN / 4);
            const int n = 4 * (q - j * (kN / 4));
            j = j < K ? j : K - 1;
            r[u] = io<TIn>::load_raw4((j < nbuf ? bb + (size_t)j * GN : Bin) + n);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u * blockDim.x;
            if (q < total) {
                const int j = q / (kN / 4), n = 4 * (q - j * (kN / 4));
                *reinterpret_cast<typename io<TIn>::raw4 *>(&sB[j][n]) = j < K ? r[u] : typename io<TIn>::raw4{};
            }
        }
    }
}

// x rows of one head (64 elements each) are fetched with 16-byte loads:
// xt_elems elements per lane, xt_rows rows per wave-wide load.
template <typename TIn>
constexpr int xt_elems() { return 16 / (int)sizeof(TIn); }
template <typename TIn>
constexpr int xt_rows() { return kWave * xt_elems<TIn>() / kP; }
template <typename TIn, int XR>
constexpr int xt_loads() { return (XR + xt_rows<TIn>() - 1) / xt_rows<TIn>(); }

__device__ __forceinline__ uint4 load16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void store16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

// ------------------------------------------------------------------------
// Standard-step prologue: everything that does not read the checkpoint.
// ------------------------------------------------------------------------
template <typename TIn, int KMAX>
struct __align__(16) StepSmem {
    static constexpr bool kCommit = true;
    static constexpr bool kCoefFromX = false;
    float gram[KMAX];              // B_j . C  (one group per workgroup)
    float cs[kMaxHpw][kP * KMAX];  // commit coefficients w_j x_j[r] (cs_index layout)
    union {
        TIn X[kMaxHpw][KMAX][kP];  // prologue, per head: x rows of the K entries as stored (rows >= K unset)
        float B[KMAX][kN];         // commit steps, after the prologue: the group's B entries, zero past K
    } u;
};

// The 64-entry step: no coefficient table (it alone would be 64 KB for four
// heads).  Commit steps form the coefficients w_j x_j[r] as they use them,
// from the x rows, which therefore stay in LDS next to the B entries, and
// keep the B entries as stored: 48 KB per workgroup with bf16 inputs
// instead of 96 KB, so three workgroups fit on a CU.
template <typename TIn, int KMAX>
struct __align__(16) StepSmemX {
    static constexpr bool kCommit = true;
    static constexpr bool kCoefFromX = true;
    float gram[KMAX];
    struct {
        TIn X[kMaxHpw][KMAX][kP];
        TIn B[KMAX][kN];   // as stored (widened where the commit reads them), zero past K
    } u;
};

// The same for steps that never commit (the low-precision step, whose
// interval-closing commits run in a kernel of their own): no coefficient
// table, so the workgroup's LDS is a third of StepSmem's.
template <typename TIn, int KMAX>
struct __align__(16) StepSmemNoCommit {
    static constexpr bool kCommit = false;
    float gram[KMAX];
    float cy[kMaxHpw][KMAX];   // per head: w_j g_j, read back as broadcasts
    union {
        TIn X[kMaxHpw][KMAX][kP];
    } u;
    TIn C[kN];   // the group's C of the current token (for row-per-lane output dots)
};

struct StepIn {
    int k, K;
    int seen;   // pos[b] as read (before clamping)
    bool commit;
    size_t HP, GN;
    const void *xin, *Bin, *Cin, *dtin, *xb, *bb, *db;   // typed by the caller
};

// The slot's input / buffer pointers (everything of StepIn but the position).
template <typename TIn>
__device__ __forceinline__ StepIn step_pointers(const ReplayParams &a, const Slot &s) {
    StepIn in;
    in.HP = (size_t)a.H * kP;
    in.GN = (size_t)a.G * kN;
    in.xin = reinterpret_cast<const TIn *>(a.x) + (size_t)s.row * in.HP + (size_t)s.h * kP;
    in.Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.row * in.GN + (size_t)s.g * kN;
    in.Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)s.row * in.GN + (size_t)s.g * kN;
    in.dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)s.row * a.H + s.h;
    in.xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * in.HP + (size_t)s.h * kP;
    in.bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * in.GN + (size_t)s.g * kN;
    in.db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;
    return in;
}

// Sets the position k as read: clamped into 0..kmax, flagged otherwise.
// kmax is L-1, or Lcap where deferred accepts can leave k >= L entries: the
// step then replays and commits all k+1.
__device__ __forceinline__ void step_position(StepIn &in, const ReplayParams &a, int kmax, int k) {
    in.seen = k;
    if (k < 0 || k > kmax) {
        if (threadIdx.x == 0) atomicOr(a.err, kErrPos);
        k = k < 0 ? 0 : kmax;
    }
    in.k = k;
    in.K = k + 1;
    in.commit = (in.K >= a.L);   // > L only after a deferred accept
}

// Pointers and position in one.
template <typename TIn>
__device__ __forceinline__ StepIn step_inputs(const ReplayParams &a, const Slot &s, int kmax, int k) {
    StepIn in = step_pointers<TIn>(a, s);
    step_position(in, a, kmax, k);
    return in;
}

template <typename TIn>
__device__ __forceinline__ StepIn step_inputs(const ReplayParams &a, const Slot &s, int kmax) {
    return step_inputs<TIn>(a, s, kmax, a.pos[s.b]);
}

// After the Gram row and the x rows are in LDS (behind a barrier): with
// l_i = A dt_i in lane i, Lambda_K = exp(sum_{i<K} l_i) in *lam, and each
// lane's suffix sum_{lane < i < K} l_i grown in ascending i through lane
// broadcasts (no LDS round trips); the buffer part of the output
// sum_j w_j g_j x_j[prow] + D x_k[prow] in *ybuf.  Returns w_j in lane j
// (zero for j >= K).
template <typename TIn, int KMAX, typename SM>
__device__ __forceinline__ float step_replay_terms(const Slot &s, int k, int K, float l, float d, float Dh, int prow,
                                                   SM &sm, float *lam, float *ybuf) {
    if constexpr (!SM::kCommit) {
        // A step that never commits uses its weights for the output alone, so
        // the sums need not follow the commit's ascending order: a DPP suffix
        // scan gives every lane sum_{i >= lane} l_i at once (l_i = 0 for
        // i >= K), its right neighbour's value is the exclusive suffix, lane
        // 0's the total.  w_j g_j goes to LDS and returns as broadcasts; the
        // x rows in LDS up to K rounded up to 4 hold finite values (entries
        // past K repeat entry K-1) and meet zero weights there, so the sum
        // needs no selects.
        const float R = suffix_sum<KMAX>(l, s.lane);
        const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, R), 0));
        const float suf = dpp<kDppWaveShl1>(R);
        *lam = expf(tot);
        const float wj = s.lane < K ? d * expf(suf) : 0.f;
        if (s.lane < KMAX) sm.cy[s.wave][s.lane] = s.lane < K ? wj * sm.gram[s.lane] : 0.f;
        const TIn *xrow = &sm.u.X[s.wave][0][prow];
        const float *cy = sm.cy[s.wave];
        float yb = Dh * io<TIn>::load1(xrow + k * kP);
        for (int j0 = 0; j0 < K; j0 += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) yb = fmaf(cy[j0 + u], io<TIn>::load1(xrow + (j0 + u) * kP), yb);
        }
        *ybuf = yb;
        return wj;
    }
    float tot = 0.f, suf = 0.f;
    for (int i = 0; i < K; ++i) {
        const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
        tot += li;
        if (i > s.lane) suf += li;
    }
    *lam = expf(tot);
    const float wj = s.lane < K ? d * expf(suf) : 0.f;               // w_j in lane j, zero for j >= K
    const float cyj = s.lane < K ? wj * sm.gram[s.lane < KMAX ? s.lane : 0] : 0.f;   // w_j g_j

    const TIn *xrow = &sm.u.X[s.wave][0][prow];   // x_j[prow] at xrow[j * kP]
    float yb = Dh * io<TIn>::load1(xrow + k * kP);
    for (int j0 = 0; j0 < K; j0 += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + u;
            const float cj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cyj), j));
            const float term = cj * io<TIn>::load1(xrow + j * kP);
            yb += (j < K) ? term : 0.f;   // select: entries beyond K never leak (even NaN)
        }
    }
    *ybuf = yb;
    return wj;
}

// Decay prep, Gram row, replay weights and the buffer part of the output for
// row `prow` of this lane; on commit steps also the commit coefficients
// (sm.cs) and the group's B entries (sm.u.B, fp32).  Returns Lambda_K in
// *lam and sum_j w_j g_j x_j[prow] + D x[prow] in *ybuf.  The head's x rows
// arrive with a few 16-byte loads and are read back per row from LDS, so the
// prologue holds few registers next to the checkpoint chunks in flight.
template <typename TIn, int KMAX, typename SM>
__device__ __forceinline__ void step_prologue(const ReplayParams &a, const Slot &s, const StepIn &in,
                                              int prow, SM &sm, float *lam, float *ybuf, float *wj_out = nullptr) {
    const int k = in.k, K = in.K;
    const TIn *xin = static_cast<const TIn *>(in.xin);
    const TIn *Bin = static_cast<const TIn *>(in.Bin);
    const TIn *Cin = static_cast<const TIn *>(in.Cin);
    const TIn *xb = static_cast<const TIn *>(in.xb);
    const TIn *bb = static_cast<const TIn *>(in.bb);
    const TIn *db = static_cast<const TIn *>(in.db);

    // x rows of entries 0..K-1 (entry k is the current token)
    const int lpr = kP / xt_elems<TIn>();
    const int r0 = s.lane / lpr, col = xt_elems<TIn>() * (s.lane % lpr);
    uint4 xw[xt_loads<TIn, KMAX>()];
#pragma unroll
    for (int i = 0; i < xt_loads<TIn, KMAX>(); ++i) {
        if (i * xt_rows<TIn>() < K) {   // uniform: loads past the last row are skipped
            int j = i * xt_rows<TIn>() + r0;
            j = j < K ? j : K - 1;      // lanes past it repeat the last row
            xw[i] = load16(j < k ? xb + (size_t)j * in.HP + col : xin + col);
        }
    }
    const float Ah = a.A[s.h], Dh = a.D[s.h];
    // dt of entry `lane`: every lane loads (lanes past the last entry repeat
    // it) and the value is widened and masked at its use, so no branch around
    // the load makes the wave wait for it on the spot.
    const int jd = s.lane < K ? s.lane : K - 1;
    const TIn draw = *((jd < k) ? db + (size_t)jd * a.H : static_cast<const TIn *>(in.dtin));
    {   // Gram row g_j = B_j . C, 16 lanes x 8 elements per dot; the first
        // pass's operands are requested unconditionally with the other
        // prologue loads (a group past the last entry re-reads it)
        const int t16 = threadIdx.x & 15, grp = threadIdx.x >> 4, ngrp = blockDim.x >> 4;
        const typename io<TIn>::raw4 rc0 = io<TIn>::load_raw4(Cin + 8 * t16), rc1 = io<TIn>::load_raw4(Cin + 8 * t16 + 4);
        const int j0 = grp < K ? grp : K - 1;
        const TIn *pb0 = (j0 < k) ? bb + (size_t)j0 * in.GN : Bin;
        const typename io<TIn>::raw4 rb0 = io<TIn>::load_raw4(pb0 + 8 * t16), rb1 = io<TIn>::load_raw4(pb0 + 8 * t16 + 4);
        const float4 c0 = io<TIn>::widen(rc0), c1 = io<TIn>::widen(rc1);
        if constexpr (!SM::kCommit) {   // C into LDS for row-per-lane output dots (16 lanes hold all of it)
            if (grp == 0) {
                *reinterpret_cast<typename io<TIn>::raw4 *>(&sm.C[8 * t16]) = rc0;
                *reinterpret_cast<typename io<TIn>::raw4 *>(&sm.C[8 * t16 + 4]) = rc1;
            }
        }
        {   // computed by every group (keeps the loads ahead), stored where grp < K
            const float acc = row16_sum(dot4(io<TIn>::widen(rb0), c0) + dot4(io<TIn>::widen(rb1), c1));
            if (grp < K && t16 == 0) sm.gram[grp] = acc;
        }
        for (int j = grp + ngrp; j < K; j += ngrp) {
            const TIn *pb = (j < k) ? bb + (size_t)j * in.GN : Bin;
            const float4 b0 = io<TIn>::load4(pb + 8 * t16), b1 = io<TIn>::load4(pb + 8 * t16 + 4);
            const float acc = row16_sum(dot4(b0, c0) + dot4(b1, c1));
            if (t16 == 0) sm.gram[j] = acc;
        }
    }
    const float d = s.lane < K ? io<TIn>::load1(&draw) : 0.f;
#pragma unroll
    for (int i = 0; i < xt_loads<TIn, KMAX>(); ++i) {
        const int j = i * xt_rows<TIn>() + r0;
        // steps that never commit also keep the repeated rows past K (the
        // output sum reads up to K rounded up to 4)
        if (i * xt_rows<TIn>() < K && (!SM::kCommit || j < K)) store16(&sm.u.X[s.wave][j][col], xw[i]);
    }
    __syncthreads();
    const float wj = step_replay_terms<TIn, KMAX>(s, k, K, Ah * d, d, Dh, prow, sm, lam, ybuf);
    if (wj_out) *wj_out = wj;
    const TIn *xrow = &sm.u.X[s.wave][0][prow];   // x_j[prow] at xrow[j * kP]
    if constexpr (SM::kCommit) {
        if (in.commit) {
            if constexpr (!SM::kCoefFromX) {
                // row prow of the commit coefficients; any lane -> row bijection fills them all
                const int i = prow >> 1, hf = prow & 1;
#pragma unroll
                for (int j = 0; j < KMAX; ++j) {
                    const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
                    const float cf = w * io<TIn>::load1(xrow + j * kP);
                    sm.cs[s.wave][cs_index<KMAX>(hf, i & 3, j, i >> 2)] = (j < K) ? cf : 0.f;
                }
                __syncthreads();   // every head is done with its x rows; B takes their place
            }
            if constexpr (SM::kCoefFromX)
                stage_B_raw<TIn, KMAX>(sm.u.B, bb, Bin, in.GN, k, K);
            else
                stage_B<TIn, KMAX>(sm.u.B, bb, Bin, in.GN, k, K);
        }
        __syncthreads();
    }
    // (a step that never commits writes no LDS after the barrier above: its
    // waves go on without waiting for each other)
}

// Append the current token at buffer entry k (x and dt per head; B once per
// group, by the group's first workgroup).
template <typename TIn>
__device__ __forceinline__ void step_append(const ReplayParams &a, const Slot &s, const StepIn &in) {
    const TIn *xin = static_cast<const TIn *>(in.xin);
    const TIn *Bin = static_cast<const TIn *>(in.Bin);
    const bool dt_lane = s.lane == 0;
    const bool b_wave = s.wave == 0 && (s.tile * a.hpw) % s.hpg == 0;   // the group's first workgroup
    // every value is read before anything is written (the buffers could alias
    // the inputs as far as the compiler knows, which would otherwise make each
    // copy wait for its load on the spot)
    const TIn xv = xin[s.lane];
    TIn dv{}, b0{}, b1{};
    if (dt_lane) dv = *static_cast<const TIn *>(in.dtin);
    if (b_wave) {
        b0 = Bin[s.lane];
        b1 = Bin[s.lane + 64];
    }
    TIn *xw = reinterpret_cast<TIn *>(a.xbuf) + ((size_t)s.b * a.Lcap + in.k) * in.HP + (size_t)s.h * kP;
    xw[s.lane] = xv;
    if (dt_lane) reinterpret_cast<TIn *>(a.dtbuf)[((size_t)s.b * a.Lcap + in.k) * a.H + s.h] = dv;
    if (b_wave) {
        TIn *bw = reinterpret_cast<TIn *>(a.bbuf) + ((size_t)s.b * a.Lcap + in.k) * in.GN + (size_t)s.g * kN;
        bw[s.lane] = b0;
        bw[s.lane + 64] = b1;
    }
}


// ------------------------------------------------------------------------
// Speculative-verify prologue.
// ------------------------------------------------------------------------

struct VerifyIn {
    int k, KL;
    int seen;   // pos[b] as read (before clamping)
    size_t HP, GN;
    const void *xin, *Bin, *Cin, *dtin, *xb, *bb, *db;
};

template <typename TIn, int T>
__device__ __forceinline__ VerifyIn verify_inputs(const ReplayParams &a, const Slot &s, int kmax, int k) {
    VerifyIn in;
    in.seen = k;
    if (k < 0 || k > kmax) {
        if (threadIdx.x == 0) atomicOr(a.err, kErrPos);
        k = k < 0 ? 0 : kmax;
    }
    in.k = k;
    in.KL = k + T;   // entries once all drafts are appended
    in.HP = (size_t)a.H * kP;
    in.GN = (size_t)a.G * kN;
    // token-axis inputs [B,T,...]
    in.xin = reinterpret_cast<const TIn *>(a.x) + (size_t)s.row * T * in.HP + (size_t)s.h * kP;
    in.Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.row * T * in.GN + (size_t)s.g * kN;
    in.Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)s.row * T * in.GN + (size_t)s.g * kN;
    in.dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)s.row * T * a.H + s.h;
    in.xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * in.HP + (size_t)s.h * kP;
    in.bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * in.GN + (size_t)s.g * kN;
    in.db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;
    return in;
}

template <typename TIn, int T>
__device__ __forceinline__ VerifyIn verify_inputs(const ReplayParams &a, const Slot &s, int kmax) {
    return verify_inputs<TIn, T>(a, s, kmax, a.pos[s.b]);
}

// ---- Split form of the verify prologue for the verify kernel.  Loads
// retire in issue order, so a wave waiting for a load issued after the
// checkpoint chunks also waits for those chunks: verify_preload issues every
// prologue load (the head's x rows, dt, A, D and the Gram operands B_j / C_t as
// raw pieces) before the kernel starts the checkpoint stream, and
// verify_finish consumes them through LDS: Gram rows, per-wave decay sums
// (lane broadcasts), then the buffer part of the outputs from the staged x
// rows and replay coefficients.  The raw pieces occupy few registers while
// the first chunks are in flight, which keeps the kernel at four waves per
// SIMD.  Per draft t (entries j < k + t + 1): w_tj = dt_j exp(sum of l_i over
// j < i <= k + t) and Lambda_t = exp(sum of l_i over i <= k + t), sums grown
// in ascending i; ybuf[t] = D x_t[prow] + sum_j w_tj (B_j . C_t) x_j[prow].
template <int KMAX, int T>
constexpr int stage_pieces() { return (KMAX + T) * (kN / 4); }
template <int KMAX, int T>
constexpr int stage_iters() { return (stage_pieces<KMAX, T>() + 255) / 256; }

// XR: rows of the x tile (>= k + T, a multiple of 4).
template <typename TIn, int KMAX, int XR, int T>
struct VerifyPre {
    uint4 xw[xt_loads<TIn, XR>()];   // x rows j < KL: entry j < k from the buffer, else draft j - k
    TIn draw;                        // dt of entry min(lane, KL - 1) as stored (widened in verify_finish)
    float Ah, Dh;                    // the head's A and D
    typename io<TIn>::raw4 g[stage_iters<KMAX, T>()];   // Gram operand pieces
};

template <typename TIn, int KMAX, int XR, int T>
struct __align__(16) VerifySmemF {
    float G[KMAX + T][kN];        // rows 0..KL-1: B_j; rows KL..KL+T-1: C_t (fp32)
    float gram[T][KMAX];
    float cy[kMaxHpw][T][XR];     // per head: w_tj (B_j . C_t), zero for j > k + t
    TIn X[kMaxHpw][XR][kP];       // per head: x rows as stored (rows >= KL unset)
};

// Gram operand piece q (4 elements): row q/32 of the staged rows.
template <typename TIn>
__device__ __forceinline__ const TIn *stage_src(const VerifyIn &in, int q) {
    const int row = q >> 5, col = 4 * (q & 31);
    const TIn *bb = static_cast<const TIn *>(in.bb), *Bin = static_cast<const TIn *>(in.Bin);
    const TIn *Cin = static_cast<const TIn *>(in.Cin);
    const TIn *p = row < in.k ? bb + (size_t)row * in.GN
                 : row < in.KL ? Bin + (size_t)(row - in.k) * in.GN
                 : Cin + (size_t)(row - in.KL) * in.GN;
    return p + col;
}

template <typename TIn, int KMAX, int XR, int T>
__device__ __forceinline__ void verify_preload(const ReplayParams &a, const Slot &s, const VerifyIn &in,
                                               VerifyPre<TIn, KMAX, XR, T> &pre) {
    static_assert(XR % 4 == 0 && XR <= KMAX, "x tile rows");
    const int k = in.k;
    const TIn *xin = static_cast<const TIn *>(in.xin);
    const TIn *xb = static_cast<const TIn *>(in.xb);
    const int lpr = kP / xt_elems<TIn>();
    const int r0 = s.lane / lpr, col = xt_elems<TIn>() * (s.lane % lpr);
#pragma unroll
    for (int i = 0; i < xt_loads<TIn, XR>(); ++i) {
        if (i * xt_rows<TIn>() < in.KL) {   // uniform: loads past the last row are skipped
            int j = i * xt_rows<TIn>() + r0;
            j = j < in.KL ? j : in.KL - 1;   // lanes past it repeat the last row
            const TIn *px = (j < k) ? xb + (size_t)j * in.HP + col : xin + (size_t)(j - k) * in.HP + col;
            pre.xw[i] = load16(px);
        }
    }
    pre.Ah = a.A[s.h];
    pre.Dh = a.D[s.h];
    {   // every lane loads (no branch around the load): lanes past the last entry repeat it
        const int j = s.lane < in.KL ? s.lane : in.KL - 1;
        const TIn *pd = (j < k) ? static_cast<const TIn *>(in.db) + (size_t)j * a.H
                                : static_cast<const TIn *>(in.dtin) + (size_t)(j - k) * a.H;
        pre.draw = *pd;
    }
    const int nq = (in.KL + T) * (kN / 4);
#pragma unroll
    for (int i = 0; i < stage_iters<KMAX, T>(); ++i) {
        const int q = threadIdx.x + i * blockDim.x;
        if (q < nq) pre.g[i] = io<TIn>::load_raw4(stage_src<TIn>(in, q));
    }
}

// Returns ybuf[t] = sum_{j < k+t+1} w_tj (B_j . C_t) x_j[prow] + D x_t[prow]
// and lam[t] = Lambda_t (uniform across the wave).  The C_t rows stay in
// sm.G[KL + t] for the caller.
template <typename TIn, int KMAX, int XR, int T>
__device__ __forceinline__ void verify_finish(const ReplayParams &a, const Slot &s, const VerifyIn &in,
                                              const VerifyPre<TIn, KMAX, XR, T> &pre,
                                              VerifySmemF<TIn, KMAX, XR, T> &sm, int prow, float (&ybuf)[T],
                                              float (&lam)[T]) {
    const int k = in.k, KL = in.KL;
    const int nq = (KL + T) * (kN / 4);
#pragma unroll
    for (int i = 0; i < stage_iters<KMAX, T>(); ++i) {
        const int q = threadIdx.x + i * blockDim.x;
        if (q < nq) *reinterpret_cast<float4 *>(&sm.G[q >> 5][4 * (q & 31)]) = io<TIn>::widen(pre.g[i]);
    }
    // workgroups narrower than 256 threads stage the remaining pieces directly
    for (int q = threadIdx.x + stage_iters<KMAX, T>() * blockDim.x; q < nq; q += blockDim.x)
        *reinterpret_cast<float4 *>(&sm.G[q >> 5][4 * (q & 31)]) = io<TIn>::load4(stage_src<TIn>(in, q));
    {
        const int lpr = kP / xt_elems<TIn>();
        const int r0 = s.lane / lpr, col = xt_elems<TIn>() * (s.lane % lpr);
#pragma unroll
        for (int i = 0; i < xt_loads<TIn, XR>(); ++i) {
            const int j = i * xt_rows<TIn>() + r0;
            if (i * xt_rows<TIn>() < KL && j < KL) store16(&sm.X[s.wave][j][col], pre.xw[i]);
        }
    }
    __syncthreads();
    {   // Gram g[t][j] = B_j . C_t, 16 lanes x 8 elements per dot
        const int t16 = threadIdx.x & 15, grp = threadIdx.x >> 4, ngrp = blockDim.x >> 4;
        for (int dd = grp; dd < T * KL; dd += ngrp) {
            const int t = dd / KL, j = dd - t * KL;
            const float4 b0 = *reinterpret_cast<const float4 *>(&sm.G[j][8 * t16]);
            const float4 b1 = *reinterpret_cast<const float4 *>(&sm.G[j][8 * t16 + 4]);
            const float4 c0 = *reinterpret_cast<const float4 *>(&sm.G[KL + t][8 * t16]);
            const float4 c1 = *reinterpret_cast<const float4 *>(&sm.G[KL + t][8 * t16 + 4]);
            const float acc = row16_sum(dot4(b0, c0) + dot4(b1, c1));
            if (t16 == 0) sm.gram[t][j] = acc;
        }
    }
    __syncthreads();

    // Per wave (head): l_i = A dt_i lives in lane i.  Suffix sums
    // sum_{lane < i <= k+t} l_i and prefix sums sum_{i <= k+t} l_i grow in
    // ascending i, one entry per step, as the sequential loops add them.
    const float Dh = pre.Dh;
    const float d = s.lane < KL ? io<TIn>::load1(&pre.draw) : 0.f;   // dt of entry `lane`, 0 past the last
    const float l = pre.Ah * d;
    float suf = 0.f, tot = 0.f;
    for (int i = 0; i <= k; ++i) {
        const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
        tot += li;
        if (i > s.lane) suf += li;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        if (t > 0) {
            const int i = k + t;
            const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
            tot += li;
            if (i > s.lane) suf += li;
        }
        lam[t] = expf(tot);
        const float cy = (s.lane < k + t + 1) ? d * expf(suf) * sm.gram[t][s.lane < KMAX ? s.lane : 0] : 0.f;
        if (s.lane < XR) sm.cy[s.wave][t][s.lane] = cy;
    }
    __syncthreads();
    // buffer part: x rows (broadcast across rows of the tile) times the
    // coefficients (LDS broadcasts), entries in ascending order
    float acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = Dh * io<TIn>::load1(&sm.X[s.wave][k + t][prow]);
    for (int j0 = 0; j0 < KL; j0 += 4) {
        float xj[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xj[u] = io<TIn>::load1(&sm.X[s.wave][j0 + u][prow]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float4 c4 = *reinterpret_cast<const float4 *>(&sm.cy[s.wave][t][j0]);
            const float cf[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float term = cf[u] * xj[u];
                acc[t] += (j0 + u < k + t + 1) ? term : 0.f;   // later drafts never reach output t
            }
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) ybuf[t] = acc[t];
}

// Append the T drafts at entries k .. k+T-1 (the position is not advanced).
// WRITE_B = false leaves the group's B entries to publish_fold.
template <typename TIn, int T, bool WRITE_B = true>
__device__ __forceinline__ void verify_append(const ReplayParams &a, const Slot &s, const VerifyIn &in) {
    const TIn *xin = static_cast<const TIn *>(in.xin);
    const TIn *Bin = static_cast<const TIn *>(in.Bin);
    const TIn *dtin = static_cast<const TIn *>(in.dtin);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        TIn *xw = reinterpret_cast<TIn *>(a.xbuf) + ((size_t)s.b * a.Lcap + in.k + t) * in.HP + (size_t)s.h * kP;
        io<TIn>::copy1(xw + s.lane, xin + (size_t)t * in.HP + s.lane);
    }
    if (s.lane < T) {
        TIn *dw = reinterpret_cast<TIn *>(a.dtbuf) + ((size_t)s.b * a.Lcap + in.k + s.lane) * a.H + s.h;
        io<TIn>::copy1(dw, dtin + (size_t)s.lane * a.H);
    }
    if (WRITE_B && s.wave == 0 && (s.tile * a.hpw) % s.hpg == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            TIn *bw = reinterpret_cast<TIn *>(a.bbuf) + ((size_t)s.b * a.Lcap + in.k + t) * in.GN + (size_t)s.g * kN;
            io<TIn>::copy1(bw + s.lane, Bin + (size_t)t * in.GN + s.lane);
            io<TIn>::copy1(bw + s.lane + 64, Bin + (size_t)t * in.GN + s.lane + 64);
        }
    }
}

// ------------------------------------------------------------------------
// Accept / flush prologue: how many entries to fold and whether to commit.
// ------------------------------------------------------------------------
template <int KMAX>
struct CommitSmem {
    float l[kMaxHpw][KMAX];
    float w[kMaxHpw][KMAX];
    float cs[kMaxHpw][kP * KMAX];
};

template <bool ACCEPT>
__device__ __forceinline__ int commit_count(const ReplayParams &a, const Slot &s, bool *commit, int *seen) {
    // an accept follows a verify (k <= L-1); a flush also folds the up to
    // Lcap entries a deferred accept can leave
    const int kmax = ACCEPT ? a.L - 1 : a.Lcap;
    int k = a.pos[s.b];
    *seen = k;
    if (k < 0 || k > kmax) {
        if (threadIdx.x == 0) atomicOr(a.err, kErrPos);
        k = k < 0 ? 0 : kmax;
    }
    int nk = 0;
    if (ACCEPT) {
        nk = a.n_keep[s.row];
        if (nk < 0 || nk > a.T) {
            if (threadIdx.x == 0) atomicOr(a.err, kErrKeep);
            nk = nk < 0 ? 0 : a.T;
        }
    }
    const int K = k + nk;
    *commit = ACCEPT ? (K >= a.L) : (K > 0);
    return K;
}

// Lambda_K, commit coefficients (LDS) and this lane's B_j slices for folding
// all K buffered entries (K >= 1).  l_i = A dt_i lives in lane i; the prefix
// sum (Lambda_K) and each lane's suffix sum sum_{lane < i < K} l_i grow in
// ascending i through lane broadcasts (no LDS round trips).  sl / sw are
// unused (kept for the callers' shared-memory layouts).
template <typename TIn, int KMAX, bool LOAD_BJ = true>
__device__ __forceinline__ float commit_prologue(const ReplayParams &a, const Slot &s, int K,
                                                 float (*sl)[KMAX], float (*sw)[KMAX],
                                                 float (*scs)[kP * KMAX],
                                                 typename io<TIn>::raw4 (&Bj)[KMAX]) {
    (void)sl;
    (void)sw;
    const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
    const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * HP + (size_t)s.h * kP;
    const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
    const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;
    const float Ah = a.A[s.h];

    float xv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int jj = j < K ? j : K - 1;
        xv[j] = io<TIn>::load1(xb + (size_t)jj * HP + s.prow);
        if (LOAD_BJ) Bj[j] = io<TIn>::load_raw4(bb + (size_t)jj * GN + 4 * s.c);
    }
    const float dl = s.lane < K ? io<TIn>::load1(db + (size_t)s.lane * a.H) : 0.f;
    const float l = Ah * dl;
    float tot = 0.f, suf = 0.f;
    for (int i = 0; i < K; ++i) {
        const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), i));
        tot += li;
        if (i > s.lane) suf += li;
    }
    const float wj = s.lane < K ? dl * expf(suf) : 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
        const float cf = w * xv[j];
        scs[s.wave][cs_index<KMAX>(s.hf, s.c & 3, j, s.c >> 2)] = (j < K) ? cf : 0.f;
    }
    __syncthreads();
    return expf(tot);
}

// Rewrite the 8 rows of chunk c in place, S_new[r] = lam S0[r] + sum_j
// cs[r][j] B_j[4c..4c+3], with the group's B entries staged in LDS (sB, zero past
// K) and the entry loop cut at Kr = K rounded up to 4, so a short fold does
// not pay for KMAX entries.  `col` = 4c, laundered per chunk by the caller's
// asm so the B_j reads are redone per chunk instead of held in registers.
template <int KMAX>
__device__ __forceinline__ void commit_chunk_lds(float4 (&st)[kPerChunk], int c, float lam, const float *cs,
                                                 const float (*sB)[kN], int hf, int Kr, const HeadState &dst) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) {
        st[m].x *= lam; st[m].y *= lam; st[m].z *= lam; st[m].w *= lam;
    }
    int col = 4 * (threadIdx.x & 31);
    asm volatile("" : "+v"(col));
    for (int j0 = 0; j0 < Kr; j0 += 4) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = j0 + jj;
            const float4 b = *reinterpret_cast<const float4 *>(&sB[j][col]);
            const float *cp = cs + cs_index<KMAX>(hf, c, j, 0);
            const float4 c0 = *reinterpret_cast<const float4 *>(cp);
            const float4 c1 = *reinterpret_cast<const float4 *>(cp + 4);
            const float cf[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) {
                st[m].x += cf[m] * b.x;
                st[m].y += cf[m] * b.y;
                st[m].z += cf[m] * b.z;
                st[m].w += cf[m] * b.w;
            }
        }
    }
    store_chunk(dst, c, st);
}

// commit_chunk_lds with the coefficients formed as they are used: w_j (lane
// j of wj) times x_j[r] from the head's x rows in LDS (sX[j][r]; entries
// from K on are unset there and masked), the same products as the table
// the other commit paths fill, so the results are bit-identical.
template <typename TIn, int KMAX>
__device__ __forceinline__ void commit_chunk_x(float4 (&st)[kPerChunk], int c, float lam, float wj,
                                               const TIn (*sX)[kP], const TIn (*sB)[kN], int hf, int K,
                                               const HeadState &dst) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) {
        st[m].x *= lam; st[m].y *= lam; st[m].z *= lam; st[m].w *= lam;
    }
    int col = 4 * (threadIdx.x & 31);
    asm volatile("" : "+v"(col));
    const int Kr = (K + 3) & ~3;
    for (int j0 = 0; j0 < Kr; j0 += 4) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int j = j0 + jj;
            const float4 b = io<TIn>::widen(*reinterpret_cast<const typename io<TIn>::raw4 *>(&sB[j][col]));
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
            float cf[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) {
                const float prod = w * io<TIn>::load1(&sX[j][2 * chunk_index(c, m) + hf]);
                cf[m] = (j < K) ? prod : 0.f;
            }
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) {
                st[m].x += cf[m] * b.x;
                st[m].y += cf[m] * b.y;
                st[m].z += cf[m] * b.z;
                st[m].w += cf[m] * b.w;
            }
        }
    }
    store_chunk(dst, c, st);
}

// Partial sums of row pairs of one chunk against T vectors, reduce-scattered
// so that lane (c, hf) ends with its share of row 2c+hf (see chunk_combine4).
template <int T>
__device__ __forceinline__ void chunk_dots(const float4 (&cur)[kPerChunk], const float4 (&C4)[T], int lane,
                                           float (&r)[T][kChunks], int c) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float v[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4[t]);
        r[t][c] = chunk_reduce8(v, lane);
    }
}

// Dots of one chunk's 8 rows with the T vectors C4[t], each reduced over
// the lane's half-wave down to the chunk value of the lane's row.
template <int T>
__device__ __forceinline__ void chunk_dots_1(const float4 (&cur)[kPerChunk], const float4 (&C4)[T], int lane,
                                             float (&out)[T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float v[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4[t]);
        out[t] = chunk_reduce8(v, lane);
    }
}

// The two stages of chunk_combine4 taken one pair at a time: combine_pair
// closes lane bit 1 for chunks (0, 2) or (1, 3), combine_last closes lane
// bit 0 on the two pair values.  Same additions as chunk_combine4.
__device__ __forceinline__ float combine_pair(float ra, float rb, bool up) {
    const float lo = ra + dpp<kDppQuadRev>(ra);
    const float hi = rb + dpp<kDppQuadRev>(rb);
    return up ? hi : lo;
}
__device__ __forceinline__ float combine_last(float p0, float p1, bool up) {
    const float lo = p0 + dpp<kDppQuadSwap1>(p0);
    const float hi = p1 + dpp<kDppQuadSwap1>(p1);
    return up ? hi : lo;
}

// ------------------------------------------------------------------------
// Deferred fold.  replayssm_accept_deferred only advances pos, so a slot can
// hold K = pos >= L accepted entries; the next verify on the slot folds them
// into the checkpoint in the pass that streams it anyway (each chunk:
// S_new = Lambda_K S0 + sum_j w_j x_j (x) B_j, stored, then the dots of the
// drafts against S_new), and the drafts become entries 0..T-1 of the next
// interval.  Same per-element arithmetic as a commit followed by a verify
// at pos 0, so results are bit-identical to the eager accept.
// ------------------------------------------------------------------------
template <int T>
constexpr int fold_xrows() { return (T + 3) & ~3; }   // the drafts' x rows, rounded to 4

template <typename TIn, int KMAX, int T>
struct FoldSmem {
    float cs[kMaxHpw][kP * KMAX];   // commit coefficients (cs_index layout)
    float B[KMAX][kN];              // the group's B entries, zero past K
    VerifySmemF<TIn, fold_xrows<T>(), fold_xrows<T>(), T> v;   // the drafts (entries 0..T-1): Gram operands, x rows
};

// Commit coefficients of the K buffered entries, then the replay
// coefficients, Lambda_t (lam) and buffer part of the outputs of T tokens at
// positions 0..T-1 (token inputs as laid out for verify).  Returns Lambda_K.
template <typename TIn, int KMAX, int T>
__device__ __forceinline__ float fold_prologue(const ReplayParams &a, const Slot &s, int K, const VerifyIn &in,
                                               FoldSmem<TIn, KMAX, T> &sm, float (&ybuf)[T], float (&lam)[T]) {
    VerifyIn v = in;
    v.k = 0;
    v.KL = T;
    constexpr int FX = fold_xrows<T>();
    VerifyPre<TIn, FX, FX, T> pre;
    verify_preload<TIn, FX, FX, T>(a, s, v, pre);
    stage_B<TIn, KMAX>(sm.B, static_cast<const TIn *>(in.bb), static_cast<const TIn *>(in.bb), in.GN, K, K);
    typename io<TIn>::raw4 unused[KMAX];
    const float lamK = commit_prologue<TIn, KMAX, false>(a, s, K, nullptr, nullptr, sm.cs, unused);
    verify_finish<TIn, FX, FX, T>(a, s, v, pre, sm.v, s.prow, ybuf, lam);
    return lamK;
}

// End of a fold: the last-arriving workgroup of slot b publishes the commit
// (pos = new_pos, intv + 1) and only then writes the B entries 0..T-1 of all
// the slot's groups.  Every workgroup of the slot reads B entries 0..K-1 of
// its group for the fold; a workgroup writing entry 0 earlier would race
// with the others' reads, while the last arrival knows they are all done.
// Bin: the slot's [T,G,N] input B (contiguous, as are entries 0..T-1).
template <typename TIn>
__device__ __forceinline__ void publish_fold(const ReplayParams &a, int b, int new_pos, const TIn *Bin, int T,
                                             int seen) {
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = atomicAdd(&a.work[b], 1);
        if (old >= a.wg_per_slot) atomicOr(a.err, kErrDup);
        last = old == a.wg_per_slot - 1;
        if (last) {
            if (a.pos[b] != seen) atomicOr(a.err, kErrDup);
            a.work[b] = 0;
            a.pos[b] = new_pos;
            a.intv[b] += 1;
        }
    }
    __syncthreads();
    if (last) {
        const size_t GN = (size_t)a.G * kN;
        TIn *dst = reinterpret_cast<TIn *>(a.bbuf) + (size_t)b * a.Lcap * GN;
        for (size_t i = threadIdx.x; i < (size_t)T * GN; i += blockDim.x) io<TIn>::copy1(dst + i, Bin + i);
    }
}

}  // namespace
}  // namespace rssm
