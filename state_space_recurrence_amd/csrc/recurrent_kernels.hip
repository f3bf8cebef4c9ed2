// recurrent_kernels.hip -- the conventional SSM decode update, kept as the
// in-run GPU baseline ("NVIDIA ReplaySSM: hybrid model SSM decoding with a
// state buffer", section 1: the usual scheme reads and writes the whole state
// for every token; section 3: speculative decoding keeps one state copy per
// draft token).  Per head h, group g = h / (H/G), for each token:
//     a = exp(dt A_h);  S <- a S + dt x (outer) B;  y = S . C + D_h x
//
// Same mapping and load width as the replay kernels (one wave64 per head,
// 16-byte coalesced loads and stores, DPP / permlane reduce-scatter), so the
// comparison measures the method, not the tuning.
#include "device_common.h"
#include "kernels.h"

namespace rssm {

namespace {

constexpr int kMaxHpw = 4;

constexpr int kNB = 2;   // state chunks in flight per wave

template <typename TIn, int T, bool POOL>
__global__ void __launch_bounds__(256) recurrent_kernel(RecurrentParams a) {
    // x of each token in the order a lane consumes rows: s_x[w][t][hf][c][m]
    // = x_t[2(c + 4m) + hf] (chunk c of the state stream, see device_common.h)
    __shared__ float s_x[kMaxHpw][T][2][kChunks][kPerChunk];

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / a.wg_per_slot, tile = wg - b * a.wg_per_slot;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = tile * a.hpw + wave;
    const int g = (tile * a.hpw) / (a.H / a.G);
    const int c = lane & 31, hf = lane >> 5, prow = 2 * c + hf;
    const size_t PN = (size_t)kP * kN, HP = (size_t)a.H * kP, GN = (size_t)a.G * kN;

    int cur = 0;
    const float *src;
    if (POOL) {
        cur = a.sel[b];
        cur = cur < 0 ? 0 : (cur > a.Tmax ? a.Tmax : cur);
        src = a.state + (((size_t)b * (a.Tmax + 1) + cur) * a.H + h) * PN;
    } else {
        src = a.state + ((size_t)b * a.H + h) * PN;
    }
    const size_t lane_off = (size_t)hf * kN + 4 * c;
    src += lane_off;

    float4 buf[kNB][kPerChunk];
#pragma unroll
    for (int q = 0; q < kNB; ++q)
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m)
            buf[q][m] = stream_load4(src + (size_t)chunk_index(q, m) * 2 * kN);

    const TIn *xin = reinterpret_cast<const TIn *>(a.x) + (size_t)b * T * HP + (size_t)h * kP;
    const TIn *Bin = reinterpret_cast<const TIn *>(a.Bm) + (size_t)b * T * GN + (size_t)g * kN;
    const TIn *Cin = reinterpret_cast<const TIn *>(a.Cm) + (size_t)b * T * GN + (size_t)g * kN;
    const TIn *dtin = reinterpret_cast<const TIn *>(a.dt) + (size_t)b * T * a.H + h;
    const float Ah = a.A[h], Dh = a.D[h];

    typename io<TIn>::raw4 Braw[T], Craw[T];   // widened at each use
    float dtv[T], at[T], xcur[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float xl = io<TIn>::load1(xin + (size_t)t * HP + lane);
        s_x[wave][t][lane & 1][(lane >> 1) & 3][lane >> 3] = xl;
        xcur[t] = io<TIn>::load1(xin + (size_t)t * HP + prow);
        Braw[t] = io<TIn>::load_raw4(Bin + (size_t)t * GN + 4 * c);
        Craw[t] = io<TIn>::load_raw4(Cin + (size_t)t * GN + 4 * c);
        dtv[t] = io<TIn>::load1(dtin + (size_t)t * a.H);
        at[t] = expf(dtv[t] * Ah);
    }
    __syncthreads();

    float r[T][kChunks];
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
        float4 (&st)[kPerChunk] = buf[q % kNB];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const float *xs = s_x[wave][t][hf][q];
            const float4 x0 = *reinterpret_cast<const float4 *>(xs);
            const float4 x1 = *reinterpret_cast<const float4 *>(xs + 4);
            const float xr[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float4 Bt = io<TIn>::widen_here(Braw[t]), Ct = io<TIn>::widen_here(Craw[t]);
            float v[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) {
                const float cx = dtv[t] * xr[m];
                st[m].x = at[t] * st[m].x + cx * Bt.x;
                st[m].y = at[t] * st[m].y + cx * Bt.y;
                st[m].z = at[t] * st[m].z + cx * Bt.z;
                st[m].w = at[t] * st[m].w + cx * Bt.w;
                v[m] = dot4(st[m], Ct);
            }
            r[t][q] = chunk_reduce8(v, lane);
            if (POOL) {
                const int slot = (cur + 1 + t) % (a.Tmax + 1);
                float *dst = a.state + (((size_t)b * (a.Tmax + 1) + slot) * a.H + h) * PN + lane_off;
#pragma unroll
                for (int m = 0; m < kPerChunk; ++m)
                    stream_store4(dst + (size_t)chunk_index(q, m) * 2 * kN, st[m]);
            }
            __builtin_amdgcn_sched_barrier(0);   // one token's work at a time
        }
        if (!POOL) {
            float *dst = a.state + ((size_t)b * a.H + h) * PN + lane_off;
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m)
                stream_store4(dst + (size_t)chunk_index(q, m) * 2 * kN, st[m]);
        }
        if (q + kNB < kChunks) {
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m)
                st[m] = stream_load4(src + (size_t)chunk_index(q + kNB, m) * 2 * kN);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float y0 = chunk_combine4(r[t], lane);
        a.y[((size_t)b * T + t) * HP + (size_t)h * kP + prow] = y0 + Dh * xcur[t];
    }
}

__global__ void recurrent_accept_kernel(int32_t *sel, const int32_t *n_keep, int batch, int T,
                                        int Tmax) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    int nk = n_keep[b];
    nk = nk < 0 ? 0 : (nk > T ? T : nk);
    if (nk > 0) sel[b] = (sel[b] + nk) % (Tmax + 1);
}

template <typename TIn, bool POOL>
void launch_rec_t(const RecurrentParams &p, dim3 grid, dim3 block, hipStream_t stream) {
    switch (p.T) {
#define RSSM_REC_CASE(TT) \
    case TT: hipLaunchKernelGGL((recurrent_kernel<TIn, TT, POOL>), grid, block, 0, stream, p); break;
        RSSM_REC_CASE(1)
        RSSM_REC_CASE(2)
        RSSM_REC_CASE(3)
        RSSM_REC_CASE(4)
        RSSM_REC_CASE(5)
        RSSM_REC_CASE(6)
        RSSM_REC_CASE(7)
        RSSM_REC_CASE(8)
#undef RSSM_REC_CASE
        default: break;
    }
}

}  // namespace

hipError_t launch_recurrent(const RecurrentParams &p, bool in_bf16, bool pool, hipStream_t stream) {
    if (p.batch == 0) return hipSuccess;
    dim3 grid(p.batch * p.wg_per_slot), block(64 * p.hpw);
    if (pool) {
        if (in_bf16) launch_rec_t<uint16_t, true>(p, grid, block, stream);
        else launch_rec_t<float, true>(p, grid, block, stream);
    } else {
        if (in_bf16) launch_rec_t<uint16_t, false>(p, grid, block, stream);
        else launch_rec_t<float, false>(p, grid, block, stream);
    }
    return hipGetLastError();
}

hipError_t launch_recurrent_accept(int32_t *sel, const int32_t *n_keep, int batch, int T, int Tmax,
                                   hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(recurrent_accept_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, sel,
                       n_keep, batch, T, Tmax);
    return hipGetLastError();
}

}  // namespace rssm
