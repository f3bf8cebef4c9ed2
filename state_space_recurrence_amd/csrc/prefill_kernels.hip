// prefill_kernels.hip -- prompt prefill into the first checkpoint.
//
// The state a slot decodes from summarizes its prompt ("NVIDIA ReplaySSM:
// hybrid model SSM decoding with a state buffer", section 1).  A prompt of
// Tp tokens is run through the recurrence in chunks of kQ = 16 tokens with
// each head's state (64 x 128 fp32, 128 values per lane in the decode
// layout of device_common.h) held in registers for the whole prompt: per
// chunk, the outputs of its tokens are the replayed outputs from the
// chunk-start state (the arithmetic of a decode step at buffer positions
// 0..kQ-1), then the state advances by the chunk's rank-kQ update (the
// arithmetic of the interval commit).  The result is bit-identical to
// decoding the prompt token by token with a 16-token interval and flushing
// at the end, while HBM sees only the prompt inputs, the outputs and one
// read and one write of the state.
//
// With a low-precision state (precision split, section 4) the prompt runs the
// same way in fp32 on chip; the start state is the decoded update source (the
// update checkpoint, or the FP4 copy of the shared mode) and the final state
// is written once, like a commit: the update checkpoint stochastically rounded
// with the stream index of the interval it starts (intv + 1), the FP4 output
// copy quantised from the same fp32 values.
#include "device_common.h"
#include "kernels.h"
#include "replay_common.h"
#include "split_common.h"

namespace rssm {

namespace {

constexpr int kQ = 16;   // tokens per chunk

struct PrefillSmem {
    float B[kQ][kN];              // the chunk's B_j (the workgroup's group), fp32
    float C[kQ][kN];              // the chunk's C_t
    float gram[kQ][kQ];           // gram[t][j] = B_j . C_t, j <= t
    float x[kMaxHpw][kQ][kP];     // x_j[p] per head
    float cy[kMaxHpw][kQ][kQ];    // cy[t][j] = w_tj gram[t][j], j <= t, else 0
    float lam[kMaxHpw][kQ];       // Lambda_t = exp(sum_{i <= t} A dt_i)
    float cs[kMaxHpw][kP * kQ];   // commit coefficients w_j x_j[r] (cs_index<kQ> layout)
};

// st <- lam st + sum_{j < Kr} cs[r][j] B_j[cols], rows and columns of the
// lane's register chunk c (the FMA order of the interval commit).
__device__ __forceinline__ void advance_chunk(float4 (&st)[kPerChunk], int c, float lam, const float *cs,
                                              const float (*sB)[kN], int hf, int Kr) {
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
            const float *cp = cs + cs_index<kQ>(hf, c, j, 0);
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
}

// Rounds and stores the lane's rows of chunk C (a template argument, so the
// state array is indexed statically and stays in registers).
template <int MODE, int C>
__device__ __forceinline__ void quantize_chunk(const ReplayParams &a, const Slot &s, size_t hrow,
                                               const float4 (&st)[kPerChunk], uint32_t interval) {
#pragma unroll
    for (int m = 0; m < kPerChunk; m += 2) {
        quantize_store_rows<MODE>(a, hrow + 2 * chunk_index(C, m), hrow + 2 * chunk_index(C, m + 1), s.c, s.lane,
                                  st[m], st[m + 1], interval);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// MODE: -1 for the fp32 checkpoint, else the SplitMode of a low-precision state.
template <typename TIn, bool OUT, int MODE>
__global__ void __launch_bounds__(256) prefill_kernel(ReplayParams a) {
    __shared__ PrefillSmem sm;

    const Slot s = slot_of(a);
    if (s.b < 0) return;   // padding row
    const int Tp = a.T;
    const HeadState sp = head_state(a.ckpt, s, a.H);
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;   // the lane's first row (low-precision state)
    float4 st[kChunks][kPerChunk];
    if (a.from_zero) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c)
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) st[c][m] = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
        if constexpr (MODE < 0) {
#pragma unroll
            for (int c = 0; c < kChunks; ++c) load_chunk(st[c], sp, c);
        } else {   // the decoded update source, in the same lane layout
            constexpr int UB = ModeTraits<MODE>::ubits;
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
#pragma unroll
                for (int m = 0; m < kPerChunk; ++m)
                    st[c][m] = decode_row4<UB>(load_row4<UB>(a, hrow + 2 * chunk_index(c, m), s.c));
        }
        if (threadIdx.x == 0 && a.pos[s.b] != 0) atomicOr(a.err, kErrPos);   // buffer not empty
    }
    const size_t HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;
    const TIn *xin = reinterpret_cast<const TIn *>(a.x) + (size_t)s.row * Tp * HP + (size_t)s.h * kP;
    const TIn *Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)s.row * Tp * GN + (size_t)s.g * kN;
    const TIn *Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)s.row * Tp * GN + (size_t)s.g * kN;
    const TIn *dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)s.row * Tp * a.H + s.h;
    float *yout = a.y + (size_t)s.row * Tp * HP + (size_t)s.h * kP + s.prow;
    const float Ah = a.A[s.h], Dh = a.D[s.h];
    const int i_row = s.prow >> 1;   // the lane's row 2 i + hf in cs_index terms

    for (int t0 = 0; t0 < Tp; t0 += kQ) {
        const int q = Tp - t0 < kQ ? Tp - t0 : kQ;   // tokens in this chunk
        __syncthreads();   // the previous chunk's LDS reads are done
        const int Kr = (q + 3) & ~3;   // entries the update loop touches; rows q..Kr-1 are zero
        for (int i = threadIdx.x; i < Kr * (kN / 4); i += blockDim.x) {
            const int j = i >> 5, n = 4 * (i & 31);
            float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < q) {
                b = io<TIn>::load4(Bin + (size_t)(t0 + j) * GN + n);
                if (OUT) *reinterpret_cast<float4 *>(&sm.C[j][n]) = io<TIn>::load4(Cin + (size_t)(t0 + j) * GN + n);
            }
            *reinterpret_cast<float4 *>(&sm.B[j][n]) = b;
        }
#pragma unroll
        for (int j = 0; j < kQ; ++j)
            if (j < q) sm.x[s.wave][j][s.lane] = io<TIn>::load1(xin + (size_t)(t0 + j) * HP + s.lane);
        const float d = s.lane < q ? io<TIn>::load1(dtin + (size_t)(t0 + s.lane) * a.H) : 0.f;
        __syncthreads();
        if (OUT) {   // Gram rows of the chunk, 16 lanes x 8 elements per dot
            const int t16 = threadIdx.x & 15, grp = threadIdx.x >> 4, ngrp = blockDim.x >> 4;
            for (int dd = grp; dd < q * q; dd += ngrp) {
                const int t = dd / q, j = dd - t * q;
                if (j > t) continue;
                const float4 b0 = *reinterpret_cast<const float4 *>(&sm.B[j][8 * t16]);
                const float4 b1 = *reinterpret_cast<const float4 *>(&sm.B[j][8 * t16 + 4]);
                const float4 c0 = *reinterpret_cast<const float4 *>(&sm.C[t][8 * t16]);
                const float4 c1 = *reinterpret_cast<const float4 *>(&sm.C[t][8 * t16 + 4]);
                const float acc = row16_sum(dot4(b0, c0) + dot4(b1, c1));
                if (t16 == 0) sm.gram[t][j] = acc;
            }
            __syncthreads();
        }
        // Decays per head: l_i = A dt_i in lane i.  For token t (buffer
        // position t of the chunk): w_tj = dt_j exp(sum_{j < i <= t} l_i) in
        // lane j, Lambda_t = exp(sum_{i <= t} l_i); sums grow in ascending i.
        const float l = Ah * d;
        float suf = 0.f, tot = 0.f, wq = 0.f, lamq = 1.f;
        for (int t = 0; t < q; ++t) {
            const float li = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), t));
            tot += li;
            if (t > s.lane) suf += li;
            const float wt = s.lane <= t ? d * expf(suf) : 0.f;
            lamq = expf(tot);
            wq = wt;
            if (OUT) {
                if (s.lane < kQ) sm.cy[s.wave][t][s.lane] = s.lane <= t ? wt * sm.gram[t][s.lane] : 0.f;
                if (s.lane == 0) sm.lam[s.wave][t] = lamq;
            }
        }
        // commit coefficients of the lane's row: wq_j x_j[prow], j < q (zero past)
#pragma unroll
        for (int j = 0; j < kQ; ++j) {
            const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wq), j));
            const float cf = wj * sm.x[s.wave][j][s.prow];
            sm.cs[s.wave][cs_index<kQ>(s.hf, i_row & 3, j, i_row >> 2)] = j < q ? cf : 0.f;
        }
        __syncthreads();
        if (OUT) {   // y_t = Lambda_t (S . C_t) + sum_{j <= t} cy[t][j] x_j + D x_t, four tokens at a time
            for (int tg = 0; tg < q; tg += 4) {
                float r[4][kChunks];
#pragma unroll
                for (int c = 0; c < kChunks; ++c) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        int t = tg + tt;
                        t = t < q ? t : q - 1;
                        const float4 C4 = *reinterpret_cast<const float4 *>(&sm.C[t][4 * s.c]);
                        float v[kPerChunk];
#pragma unroll
                        for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(st[c][m], C4);
                        r[tt][c] = chunk_reduce8(v, s.lane);
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = tg + tt;
                    const float y0 = chunk_combine4(r[tt], s.lane);
                    if (t < q) {
                        float yb = Dh * sm.x[s.wave][t][s.prow];
#pragma unroll
                        for (int j = 0; j < kQ; ++j) {
                            const float term = sm.cy[s.wave][t][j] * sm.x[s.wave][j][s.prow];
                            yb += (j <= t) ? term : 0.f;
                        }
                        yout[(size_t)(t0 + t) * HP] = sm.lam[s.wave][t] * y0 + yb;
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kChunks; ++c) advance_chunk(st[c], c, lamq, sm.cs[s.wave], sm.B, s.hf, Kr);
    }
    if constexpr (MODE < 0) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) store_chunk(sp, c, st[c]);
    } else {
        // stream index of the interval the written state starts (read before
        // the slot's position and interval count are published)
        const uint32_t interval = (uint32_t)a.intv[s.b] + 1u;
        quantize_chunk<MODE, 0>(a, s, hrow, st[0], interval);
        quantize_chunk<MODE, 1>(a, s, hrow, st[1], interval);
        quantize_chunk<MODE, 2>(a, s, hrow, st[2], interval);
        quantize_chunk<MODE, 3>(a, s, hrow, st[3], interval);
    }
    publish_position(a, s.b, 0, true, -1);
}

}  // namespace

template <int MODE>
static void launch_prefill_m(const ReplayParams &p, bool in_bf16, bool outputs, dim3 grid, dim3 block,
                             hipStream_t stream) {
    if (in_bf16) {
        if (outputs) hipLaunchKernelGGL((prefill_kernel<uint16_t, true, MODE>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_kernel<uint16_t, false, MODE>), grid, block, 0, stream, p);
    } else {
        if (outputs) hipLaunchKernelGGL((prefill_kernel<float, true, MODE>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((prefill_kernel<float, false, MODE>), grid, block, 0, stream, p);
    }
}

hipError_t launch_prefill(const ReplayParams &p, bool in_bf16, bool outputs, int mode, hipStream_t stream) {
    if (p.batch == 0 || p.T == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    switch (mode) {
        case -1: launch_prefill_m<-1>(p, in_bf16, outputs, grid, block, stream); break;
        case kSplitBF16: launch_prefill_m<kSplitBF16>(p, in_bf16, outputs, grid, block, stream); break;
        case kSplitE4M3: launch_prefill_m<kSplitE4M3>(p, in_bf16, outputs, grid, block, stream); break;
        case kSharedFP4: launch_prefill_m<kSharedFP4>(p, in_bf16, outputs, grid, block, stream); break;
        case kLowBF16: launch_prefill_m<kLowBF16>(p, in_bf16, outputs, grid, block, stream); break;
        case kLowE4M3: launch_prefill_m<kLowE4M3>(p, in_bf16, outputs, grid, block, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rssm
