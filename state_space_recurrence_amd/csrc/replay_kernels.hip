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
#include "device_common.h"
#include "kernels.h"

namespace rssm {

namespace {

constexpr int kMaxHpw = 4;
constexpr int kNB = 2;   // checkpoint chunks in flight per wave

struct Slot {
    int b, tile, wave, lane, h, g, c, hf, prow, hpg;
};

__device__ __forceinline__ Slot slot_of(const ReplayParams &a) {
    Slot s;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    s.b = wg / a.wg_per_slot;
    s.tile = wg - s.b * a.wg_per_slot;
    s.wave = threadIdx.x >> 6;
    s.lane = threadIdx.x & 63;
    s.h = s.tile * a.hpw + s.wave;
    s.hpg = a.H / a.G;
    s.g = (s.tile * a.hpw) / s.hpg;
    s.c = s.lane & 31;
    s.hf = s.lane >> 5;
    s.prow = 2 * s.c + s.hf;
    return s;
}

// Lane base pointer into head (b,h) of an fp32 state: row hf, columns 4c..;
// value index i adds i * 2 rows.
__device__ __forceinline__ float *state_ptr(float *base, const Slot &s, int H) {
    return base + ((size_t)(s.b * H + s.h) * kP + s.hf) * kN + 4 * s.c;
}

__device__ __forceinline__ void load_chunk(float4 (&buf)[kPerChunk], const float *p, int c) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m)
        buf[m] = stream_load4(p + (size_t)chunk_index(c, m) * 2 * kN);
}

// Last-arriving workgroup of slot b publishes the slot's new position (and
// interval count).  Every workgroup of the slot read pos[b] before arriving.
__device__ __forceinline__ void publish_position(const ReplayParams &a, int b, int new_pos,
                                                 bool committed) {
    __syncthreads();
    if (threadIdx.x == 0) {
        int old = atomicAdd(&a.work[b], 1);
        if (old == a.wg_per_slot - 1) {
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

// Rewrite the 8 rows of chunk c in place:
//   S_new[r] = lam * S0[r] + sum_j cs[r][j] * B_j[4c..4c+3]
// (cs zero for j >= K).  Entry-outer order keeps one widened B_j slice and
// 8 coefficients live at a time.
template <typename TIn, int KMAX>
__device__ __forceinline__ void commit_chunk(float4 (&st)[kPerChunk], int c, float lam,
                                             const float *cs, const typename io<TIn>::raw4 (&Bj)[KMAX],
                                             int hf, float *dst) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) {
        st[m].x *= lam; st[m].y *= lam; st[m].z *= lam; st[m].w *= lam;
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const float4 b = io<TIn>::widen_here(Bj[j]);
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
        if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // bound hoisted LDS reads
    }
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m)
        stream_store4(dst + (size_t)chunk_index(c, m) * 2 * kN, st[m]);
}

// ------------------------------------------------------------------------
// Standard decode step with fused interval commit.
// ------------------------------------------------------------------------
template <typename TIn, int KMAX>
__global__ void __launch_bounds__(256) replay_step_kernel(ReplayParams a) {
    __shared__ float s_l[kMaxHpw][KMAX];
    __shared__ float s_dt[kMaxHpw][KMAX];
    __shared__ float s_gram[KMAX];
    __shared__ float s_w[kMaxHpw][KMAX];
    __shared__ float s_cy[kMaxHpw][KMAX];
    __shared__ float s_cs[kMaxHpw][kP * KMAX];

    const Slot s = slot_of(a);
    float *sp = state_ptr(a.ckpt, s, a.H);

    float4 buf[kNB][kPerChunk];
#pragma unroll
    for (int c = 0; c < kNB; ++c) load_chunk(buf[c], sp, c);

    int k = a.pos[s.b];
    if (k < 0 || k > a.L - 1) {
        if (threadIdx.x == 0) atomicOr(&a.work[a.batch], kErrPos);
        k = k < 0 ? 0 : a.L - 1;
    }
    const int K = k + 1;
    const bool commit = (K == a.L);

    const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
    const TIn *xin = reinterpret_cast<const TIn *>(a.x) + (size_t)s.b * HP + (size_t)s.h * kP;
    const TIn *Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.b * GN + (size_t)s.g * kN;
    const TIn *Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)s.b * GN + (size_t)s.g * kN;
    const TIn *dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)s.b * a.H + s.h;
    const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * HP + (size_t)s.h * kP;
    const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
    const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;

    // x_j[prow] of every entry (entry k is the current token)
    float xv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const TIn *px = (j < k) ? xb + (size_t)j * HP + s.prow : xin + s.prow;
        xv[j] = io<TIn>::load1(px);
    }
    const float xcur = io<TIn>::load1(xin + s.prow);
    const float4 C4 = io<TIn>::load4(Cin + 4 * s.c);
    const float Ah = a.A[s.h], Dh = a.D[s.h];

    if (s.lane < K) {
        const TIn *pd = (s.lane < k) ? db + (size_t)s.lane * a.H : dtin;
        float d = io<TIn>::load1(pd);
        s_dt[s.wave][s.lane] = d;
        s_l[s.wave][s.lane] = Ah * d;
    }
    {   // Gram row g_j = B_j . C, 16 lanes x 8 elements per dot
        const int t16 = threadIdx.x & 15, grp = threadIdx.x >> 4, ngrp = blockDim.x >> 4;
        const float4 c0 = io<TIn>::load4(Cin + 8 * t16), c1 = io<TIn>::load4(Cin + 8 * t16 + 4);
        for (int j = grp; j < K; j += ngrp) {
            const TIn *pb = (j < k) ? bb + (size_t)j * GN : Bin;
            float4 b0 = io<TIn>::load4(pb + 8 * t16), b1 = io<TIn>::load4(pb + 8 * t16 + 4);
            float acc = row16_sum(dot4(b0, c0) + dot4(b1, c1));
            if (t16 == 0) s_gram[j] = acc;
        }
    }
    __syncthreads();

    float tot = 0.f;
    for (int i = 0; i < K; ++i) tot += s_l[s.wave][i];
    const float lam = expf(tot);
    if (s.lane < KMAX) {
        float wj = 0.f, cy = 0.f;
        if (s.lane < K) {
            float suf = 0.f;
            for (int i = s.lane + 1; i < K; ++i) suf += s_l[s.wave][i];
            wj = s_dt[s.wave][s.lane] * expf(suf);
            cy = wj * s_gram[s.lane];
        }
        s_w[s.wave][s.lane] = wj;
        s_cy[s.wave][s.lane] = cy;
    }
    __syncthreads();

    // the part of y that does not read the checkpoint
    float ybuf = Dh * xcur;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const float term = s_cy[s.wave][j] * xv[j];
        ybuf += (j < K) ? term : 0.f;   // select: entries beyond K never leak (even NaN)
    }
    typename io<TIn>::raw4 Bj[KMAX];
    if (commit) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const float cf = s_w[s.wave][j] * xv[j];
            s_cs[s.wave][cs_index<KMAX>(s.hf, s.c & 3, j, s.c >> 2)] = (j < K) ? cf : 0.f;
            const TIn *pb = (j < k) ? bb + (size_t)j * GN : Bin;
            Bj[j] = io<TIn>::load_raw4(pb + 4 * s.c);
        }
    }
    __syncthreads();

    float r[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        float4 (&cur)[kPerChunk] = buf[c % kNB];
        float v[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4);
        r[c] = chunk_reduce8(v, s.lane);
        if (commit) commit_chunk<TIn, KMAX>(cur, c, lam, s_cs[s.wave], Bj, s.hf, sp);
        if (c + kNB < kChunks) load_chunk(cur, sp, c + kNB);
    }
    const float y0 = chunk_combine4(r, s.lane);
    a.y[(size_t)s.b * HP + (size_t)s.h * kP + s.prow] = lam * y0 + ybuf;

    if (!commit) {
        // append the token at entry k
        TIn *xw = reinterpret_cast<TIn *>(a.xbuf) + ((size_t)s.b * a.Lcap + k) * HP + (size_t)s.h * kP;
        io<TIn>::copy1(xw + s.lane, xin + s.lane);
        if (s.lane == 0) {
            TIn *dw = reinterpret_cast<TIn *>(a.dtbuf) + ((size_t)s.b * a.Lcap + k) * a.H + s.h;
            io<TIn>::copy1(dw, dtin);
        }
        if (s.wave == 0 && (s.tile * a.hpw) % s.hpg == 0) {
            TIn *bw = reinterpret_cast<TIn *>(a.bbuf) + ((size_t)s.b * a.Lcap + k) * GN + (size_t)s.g * kN;
            io<TIn>::copy1(bw + s.lane, Bin + s.lane);
            io<TIn>::copy1(bw + s.lane + 64, Bin + s.lane + 64);
        }
    }
    publish_position(a, s.b, commit ? 0 : K, commit);
}

// ------------------------------------------------------------------------
// Speculative verify: outputs of T draft positions, no state written.
// ------------------------------------------------------------------------
template <typename TIn, int KMAX, int T>
__global__ void __launch_bounds__(256) replay_verify_kernel(ReplayParams a) {
    __shared__ float s_l[kMaxHpw][KMAX];
    __shared__ float s_dt[kMaxHpw][KMAX];
    __shared__ float s_gram[T][KMAX];
    __shared__ float s_cy[kMaxHpw][T][KMAX];
    __shared__ float s_lam[kMaxHpw][T];

    const Slot s = slot_of(a);
    float *sp = state_ptr(a.ckpt, s, a.H);
    float4 buf[kNB][kPerChunk];
#pragma unroll
    for (int c = 0; c < kNB; ++c) load_chunk(buf[c], sp, c);

    int k = a.pos[s.b];
    if (k < 0 || k > a.L - 1) {
        if (threadIdx.x == 0) atomicOr(&a.work[a.batch], kErrPos);
        k = k < 0 ? 0 : a.L - 1;
    }
    const int KL = k + T;   // entries once all drafts are appended

    const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
    // token-axis inputs [B,T,...]
    const TIn *xin = reinterpret_cast<const TIn *>(a.x) + (size_t)s.b * T * HP + (size_t)s.h * kP;
    const TIn *Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.b * T * GN + (size_t)s.g * kN;
    const TIn *Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)s.b * T * GN + (size_t)s.g * kN;
    const TIn *dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)s.b * T * a.H + s.h;
    const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * HP + (size_t)s.h * kP;
    const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
    const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;

    float xv[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        int t = j - k;
        t = t < 0 ? 0 : (t > T - 1 ? T - 1 : t);
        const TIn *px = (j < k) ? xb + (size_t)j * HP + s.prow : xin + (size_t)t * HP + s.prow;
        xv[j] = io<TIn>::load1(px);
    }
    float ybuf[T];
    float4 C4[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        ybuf[t] = io<TIn>::load1(xin + (size_t)t * HP + s.prow);
        C4[t] = io<TIn>::load4(Cin + (size_t)t * GN + 4 * s.c);
    }
    const float Ah = a.A[s.h], Dh = a.D[s.h];

    if (s.lane < KL) {
        const TIn *pd = (s.lane < k) ? db + (size_t)s.lane * a.H : dtin + (size_t)(s.lane - k) * a.H;
        float d = io<TIn>::load1(pd);
        s_dt[s.wave][s.lane] = d;
        s_l[s.wave][s.lane] = Ah * d;
    }
    {   // Gram g[t][j] = B_j . C_t for every draft t and entry j < KL
        const int t16 = threadIdx.x & 15, grp = threadIdx.x >> 4, ngrp = blockDim.x >> 4;
        for (int d = grp; d < T * KL; d += ngrp) {
            const int t = d / KL, j = d - t * KL;
            const TIn *pb = (j < k) ? bb + (size_t)j * GN : Bin + (size_t)(j - k) * GN;
            const TIn *pc = Cin + (size_t)t * GN;
            float4 b0 = io<TIn>::load4(pb + 8 * t16), b1 = io<TIn>::load4(pb + 8 * t16 + 4);
            float4 c0 = io<TIn>::load4(pc + 8 * t16), c1 = io<TIn>::load4(pc + 8 * t16 + 4);
            float acc = row16_sum(dot4(b0, c0) + dot4(b1, c1));
            if (t16 == 0) s_gram[t][j] = acc;
        }
    }
    __syncthreads();

    if (s.lane < KMAX) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int Kt = k + t + 1;
            float cy = 0.f;
            if (s.lane < Kt) {
                float suf = 0.f;
                for (int i = s.lane + 1; i < Kt; ++i) suf += s_l[s.wave][i];
                cy = s_dt[s.wave][s.lane] * expf(suf) * s_gram[t][s.lane];
            }
            s_cy[s.wave][t][s.lane] = cy;
        }
    }
    if (s.lane < T) {
        float tot = 0.f;
        for (int i = 0; i < k + s.lane + 1; ++i) tot += s_l[s.wave][i];
        s_lam[s.wave][s.lane] = expf(tot);
    }
    __syncthreads();

    // the parts of the outputs that do not read the checkpoint
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int Kt = k + t + 1;
        float acc = Dh * ybuf[t];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const float term = s_cy[s.wave][t][j] * xv[j];
            acc += (j < Kt) ? term : 0.f;   // later drafts never reach output t
        }
        ybuf[t] = acc;
    }

    float r[T][kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        float4 (&cur)[kPerChunk] = buf[c % kNB];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float v[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(cur[m], C4[t]);
            r[t][c] = chunk_reduce8(v, s.lane);
        }
        if (c + kNB < kChunks) load_chunk(cur, sp, c + kNB);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float y0 = chunk_combine4(r[t], s.lane);
        a.y[((size_t)s.b * T + t) * HP + (size_t)s.h * kP + s.prow] = s_lam[s.wave][t] * y0 + ybuf[t];
    }

    // append the T drafts at entries k .. k+T-1 (position is not advanced)
#pragma unroll
    for (int t = 0; t < T; ++t) {
        TIn *xw = reinterpret_cast<TIn *>(a.xbuf) + ((size_t)s.b * a.Lcap + k + t) * HP + (size_t)s.h * kP;
        io<TIn>::copy1(xw + s.lane, xin + (size_t)t * HP + s.lane);
    }
    if (s.lane < T) {
        TIn *dw = reinterpret_cast<TIn *>(a.dtbuf) + ((size_t)s.b * a.Lcap + k + s.lane) * a.H + s.h;
        io<TIn>::copy1(dw, dtin + (size_t)s.lane * a.H);
    }
    if (s.wave == 0 && (s.tile * a.hpw) % s.hpg == 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            TIn *bw = reinterpret_cast<TIn *>(a.bbuf) + ((size_t)s.b * a.Lcap + k + t) * GN + (size_t)s.g * kN;
            io<TIn>::copy1(bw + s.lane, Bin + (size_t)t * GN + s.lane);
            io<TIn>::copy1(bw + s.lane + 64, Bin + (size_t)t * GN + s.lane + 64);
        }
    }
}

// ------------------------------------------------------------------------
// Accept (pos += n_keep, commit when the count reaches L) and flush
// (commit every slot holding buffered tokens).
// ------------------------------------------------------------------------
template <typename TIn, int KMAX, bool ACCEPT>
__global__ void __launch_bounds__(256) replay_commit_kernel(ReplayParams a) {
    __shared__ float s_l[kMaxHpw][KMAX];
    __shared__ float s_w[kMaxHpw][KMAX];
    __shared__ float s_cs[kMaxHpw][kP * KMAX];

    const Slot s = slot_of(a);
    int k = a.pos[s.b];
    if (k < 0 || k > a.L - 1) {
        if (threadIdx.x == 0) atomicOr(&a.work[a.batch], kErrPos);
        k = k < 0 ? 0 : a.L - 1;
    }
    int nk = 0;
    if (ACCEPT) {
        nk = a.n_keep[s.b];
        if (nk < 0 || nk > a.T) {
            if (threadIdx.x == 0) atomicOr(&a.work[a.batch], kErrKeep);
            nk = nk < 0 ? 0 : a.T;
        }
    }
    const int K = k + nk;
    const bool commit = ACCEPT ? (K >= a.L) : (K > 0);

    if (commit) {
        float *sp = state_ptr(a.ckpt, s, a.H);
        float4 buf[kNB][kPerChunk];
#pragma unroll
        for (int c = 0; c < kNB; ++c) load_chunk(buf[c], sp, c);

        const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
        const TIn *xb = reinterpret_cast<const TIn *>(a.xbuf) + (size_t)s.b * a.Lcap * HP + (size_t)s.h * kP;
        const TIn *bb = reinterpret_cast<const TIn *>(a.bbuf) + (size_t)s.b * a.Lcap * GN + (size_t)s.g * kN;
        const TIn *db = reinterpret_cast<const TIn *>(a.dtbuf) + (size_t)s.b * a.Lcap * a.H + s.h;
        const float Ah = a.A[s.h];

        float xv[KMAX];
        typename io<TIn>::raw4 Bj[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int jj = j < K ? j : K - 1;
            xv[j] = io<TIn>::load1(xb + (size_t)jj * HP + s.prow);
            Bj[j] = io<TIn>::load_raw4(bb + (size_t)jj * GN + 4 * s.c);
        }
        float dl = 0.f;
        if (s.lane < K) {
            float d = io<TIn>::load1(db + (size_t)s.lane * a.H);
            dl = d;
            s_l[s.wave][s.lane] = Ah * d;
        }
        __syncthreads();
        float tot = 0.f;
        for (int i = 0; i < K; ++i) tot += s_l[s.wave][i];
        const float lam = expf(tot);
        if (s.lane < KMAX) {
            float wj = 0.f;
            if (s.lane < K) {
                float suf = 0.f;
                for (int i = s.lane + 1; i < K; ++i) suf += s_l[s.wave][i];
                wj = dl * expf(suf);
            }
            s_w[s.wave][s.lane] = wj;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const float cf = s_w[s.wave][j] * xv[j];
            s_cs[s.wave][cs_index<KMAX>(s.hf, s.c & 3, j, s.c >> 2)] = (j < K) ? cf : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            float4 (&cur)[kPerChunk] = buf[c % kNB];
            commit_chunk<TIn, KMAX>(cur, c, lam, s_cs[s.wave], Bj, s.hf, sp);
            if (c + kNB < kChunks) load_chunk(cur, sp, c + kNB);
        }
    }
    publish_position(a, s.b, commit ? 0 : K, commit);
}

__global__ void zero_pos_kernel(int32_t *pos, int n) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) pos[i] = 0;
}

}  // namespace

// ---------------------------------------------------------------- launchers --

hipError_t launch_replay_step(const ReplayParams &p, bool in_bf16, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    if (p.Lcap <= 16) {
        if (in_bf16) hipLaunchKernelGGL((replay_step_kernel<uint16_t, 16>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((replay_step_kernel<float, 16>), grid, block, 0, stream, p);
    } else {
        if (in_bf16) hipLaunchKernelGGL((replay_step_kernel<uint16_t, 32>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((replay_step_kernel<float, 32>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <typename TIn, int KMAX>
static void launch_verify_t(const ReplayParams &p, dim3 grid, dim3 block, hipStream_t stream) {
    switch (p.T) {
#define RSSM_VERIFY_CASE(TT) \
    case TT: hipLaunchKernelGGL((replay_verify_kernel<TIn, KMAX, TT>), grid, block, 0, stream, p); break;
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
        if (in_bf16) launch_verify_t<uint16_t, 16>(p, grid, block, stream);
        else launch_verify_t<float, 16>(p, grid, block, stream);
    } else {
        if (in_bf16) launch_verify_t<uint16_t, 32>(p, grid, block, stream);
        else launch_verify_t<float, 32>(p, grid, block, stream);
    }
    return hipGetLastError();
}

hipError_t launch_replay_commit(const ReplayParams &p, bool in_bf16, bool accept, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
#define RSSM_COMMIT(TIn, KM)                                                                          \
    do {                                                                                           \
        if (accept) hipLaunchKernelGGL((replay_commit_kernel<TIn, KM, true>), grid, block, 0, stream, p); \
        else hipLaunchKernelGGL((replay_commit_kernel<TIn, KM, false>), grid, block, 0, stream, p);      \
    } while (0)
    if (p.Lcap <= 16) {
        if (in_bf16) RSSM_COMMIT(uint16_t, 16);
        else RSSM_COMMIT(float, 16);
    } else {
        if (in_bf16) RSSM_COMMIT(uint16_t, 32);
        else RSSM_COMMIT(float, 32);
    }
#undef RSSM_COMMIT
    return hipGetLastError();
}

hipError_t launch_zero_pos(int32_t *pos, int batch, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_pos_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, pos, batch);
    return hipGetLastError();
}

}  // namespace rssm
