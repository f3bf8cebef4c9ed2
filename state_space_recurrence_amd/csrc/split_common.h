// split_common.h -- ReplaySSM with low-precision state (precision split):
// formats, row codecs, commit and output-stream pieces shared by the
// split step / verify / commit kernels.
//
// Article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"),
// section 4: low-precision states reduce the bytes read, but rounding errors
// accumulate when the rounded state feeds the next update; ReplaySSM keeps a
// high-precision checkpoint for updates and a separate low-precision copy
// for outputs, so the copy's errors never reach later updates.  Updates are
// stored in 16- or 8-bit floats with stochastic rounding, the output copy in
// a 4-bit float.  Modes (SplitMode in kernels.h):
//   split bf16 / split E4M3 : outputs read the FP4 copy O; a commit reads
//                             the update checkpoint U, forms the new state in
//                             fp32 from it and the buffer, and writes
//                             U' = SR(S_new) and O' = Q4(S_new);
//   shared FP4              : O is the only state (outputs and updates),
//                             O' = Q4(S_new) -- the ablation the article
//                             compares against;
//   low bf16 / low E4M3     : one rounded checkpoint U serves outputs and
//                             updates (no copy).
// Formats, the rounding rules and the random stream are in quant.h.
//
// Lane layouts.  Outputs from O use 8 columns per lane (one dword of codes):
// lane l = 16 rg + cq reads columns 8cq..8cq+7 of rows 4i + rg, i = 0..15,
// and a 16-lane reduce-scatter leaves lane l with row 4cq + rg.  Outputs
// from U and every commit use the fp32 kernels' layout (4 columns 4c..4c+3
// of rows 2i + hf) so that a 32-element scale block is 8 adjacent lanes.
#pragma once

#include "device_common.h"
#include "kernels.h"
#include "quant.h"
#include "replay_common.h"

namespace rssm {

namespace {

template <int MODE> struct ModeTraits;
template <> struct ModeTraits<kSplitBF16> {
    static constexpr bool fp4_out = true, has_u = true, has_o = true;
    static constexpr int ubits = 16;
};
template <> struct ModeTraits<kSplitE4M3> {
    static constexpr bool fp4_out = true, has_u = true, has_o = true;
    static constexpr int ubits = 8;
};
template <> struct ModeTraits<kSharedFP4> {
    static constexpr bool fp4_out = true, has_u = false, has_o = true;
    static constexpr int ubits = 4;
};
template <> struct ModeTraits<kLowBF16> {
    static constexpr bool fp4_out = false, has_u = true, has_o = false;
    static constexpr int ubits = 16;
};
template <> struct ModeTraits<kLowE4M3> {
    static constexpr bool fp4_out = false, has_u = true, has_o = false;
    static constexpr int ubits = 8;
};

// Rows 4i + rg of the output copy for lane l = 16 rg + cq end up as row 4cq + rg.
__device__ __forceinline__ int fp4_prow(int lane) { return 4 * (lane & 15) + (lane >> 4); }

// ----------------------------------------------------------- 4-col rows --
// Raw source values of 4 consecutive elements (columns 4c..4c+3) of a row,
// in the update-source format UB (16: bf16, 8: E4M3, 4: FP4 code16 | scale<<16).
template <int UB> struct Raw4;
template <> struct Raw4<16> { using T = uint2; };
template <> struct Raw4<8> { using T = uint32_t; };
template <> struct Raw4<4> { using T = uint32_t; };

template <int UB>
__device__ __forceinline__ typename Raw4<UB>::T load_row4(const ReplayParams &a, size_t row, int c) {
    if constexpr (UB == 16) {
        return *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.u) + row * kN + 4 * c);
    } else if constexpr (UB == 8) {
        return *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(a.u) + row * kN + 4 * c);
    } else {
        const uint32_t code16 = *reinterpret_cast<const uint16_t *>(a.oq + row * (kN / 2) + 2 * c);
        const uint32_t sc = a.os[row * (kN / 32) + (c >> 3)];
        return code16 | (sc << 16);
    }
}

template <int UB>
__device__ __forceinline__ float4 decode_row4(typename Raw4<UB>::T r) {
    if constexpr (UB == 16) {
        return make_float4(bf16_decode(r.x & 0xFFFFu), bf16_decode(r.x >> 16), bf16_decode(r.y & 0xFFFFu),
                           bf16_decode(r.y >> 16));
    } else if constexpr (UB == 8) {
        return e4m3_decode4(r);
    } else {   // two codes per byte, decoded by the packed FP4 -> f32 conversion (exact, unit scale)
        const float s = e4m3_decode(r >> 16);
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 0);
        const f2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r, 1.0f, 1);
        return make_float4(lo.x * s, lo.y * s, hi.x * s, hi.y * s);
    }
}

// The 16-bit draws of columns 4c..4c+3 of two rows (elements e0 and e1,
// multiples of 4).  Element e draws halfword (e mod 8) of Philox4x32-10 at
// counter (e / 8, interval, layer, 0), key = seed, low halfword of each word
// first -- so lanes 2j and 2j+1 share a counter (8 draws = 8 columns).
// Instead of both computing it, the even lane computes row 0's counter and
// the odd lane row 1's, and they swap the halves the other needs (one
// quad_perm [1,0,3,2] exchange).
__device__ __forceinline__ uint32_t swap_pair_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap1, 0xF, 0xF, false);
}

__device__ __forceinline__ void sr_draws4_pair(uint64_t seed, uint32_t layer, uint32_t interval, uint32_t e0,
                                               uint32_t e1, int lane, uint32_t (&r0)[4], uint32_t (&r1)[4]) {
    const bool odd = lane & 1;
    const Philox4 o = philox4x32_10((odd ? e1 : e0) >> 3, interval, layer, 0, (uint32_t)seed,
                                    (uint32_t)(seed >> 32));
    // an even lane's columns use words x, y of a counter, an odd lane's z, w
    const uint32_t own_a = odd ? o.z : o.x, own_b = odd ? o.w : o.y;
    const uint32_t got_a = swap_pair_u32(odd ? o.x : o.z), got_b = swap_pair_u32(odd ? o.y : o.w);
    const uint32_t wa0 = odd ? got_a : own_a, wb0 = odd ? got_b : own_b;
    const uint32_t wa1 = odd ? own_a : got_a, wb1 = odd ? own_b : got_b;
    r0[0] = wa0 & 0xFFFFu; r0[1] = wa0 >> 16; r0[2] = wb0 & 0xFFFFu; r0[3] = wb0 >> 16;
    r1[0] = wa1 & 0xFFFFu; r1[1] = wa1 >> 16; r1[2] = wb1 & 0xFFFFu; r1[3] = wb1 >> 16;
}

// Rounds and stores one row slice (columns 4c..4c+3 of row `row`) of a new
// state: the update checkpoint by stochastic rounding with the draws `r`
// (stream index of the interval being started), the output copy by FP4
// quantisation (scale over the 8 lanes sharing a 32-element block).  Must be
// called by all 64 lanes together.
template <int MODE>
__device__ __forceinline__ void quantize_store_row(const ReplayParams &a, size_t row, int c, int lane,
                                                   float4 v, const uint32_t (&r)[4]) {
    using MT = ModeTraits<MODE>;
    if (a.dbg) stream_store4(a.dbg + row * kN + 4 * c, v);
    if constexpr (MT::has_u) {
        if constexpr (MT::ubits == 16) {
            uint2 q;
            q.x = bf16_sr(v.x, r[0]) | (bf16_sr(v.y, r[1]) << 16);
            q.y = bf16_sr(v.z, r[2]) | (bf16_sr(v.w, r[3]) << 16);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.u) + row * kN + 4 * c) = q;
        } else {
            const uint32_t q = e4m3_sr(v.x, r[0]) | (e4m3_sr(v.y, r[1]) << 8) | (e4m3_sr(v.z, r[2]) << 16) |
                               (e4m3_sr(v.w, r[3]) << 24);
            *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.u) + row * kN + 4 * c) = q;
        }
    }
    if constexpr (MT::has_o) {
        float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        m = fmaxf(m, dpp<kDppQuadSwap1>(m));
        m = fmaxf(m, dpp<0x4E>(m));                 // quad_perm [2,3,0,1]
        m = fmaxf(m, dpp<kDppRowHalfMirror>(m));    // lanes i <-> 7-i: the two quads of a block
        const uint32_t sc = fp4_scale_code(m);
        const float s = e4m3_decode(sc);
        const Fp4Thresholds t = fp4_thresholds(s);
        const bool z = (sc == 0u);
        const uint32_t code16 = fp4_encode(v.x, t, z) | (fp4_encode(v.y, t, z) << 4) |
                                (fp4_encode(v.z, t, z) << 8) | (fp4_encode(v.w, t, z) << 12);
        *reinterpret_cast<uint16_t *>(a.oq + row * (kN / 2) + 2 * c) = (uint16_t)code16;
        if ((c & 7) == 0) a.os[row * (kN / 32) + (c >> 3)] = (uint8_t)sc;
    }
}

// Two row slices (see quantize_store_row), their draws generated together.
template <int MODE>
__device__ __forceinline__ void quantize_store_rows(const ReplayParams &a, size_t row0, size_t row1, int c, int lane,
                                                    float4 v0, float4 v1, uint32_t interval) {
    uint32_t r0[4] = {0, 0, 0, 0}, r1[4] = {0, 0, 0, 0};
    if constexpr (ModeTraits<MODE>::has_u)
        sr_draws4_pair(a.seed, (uint32_t)a.layer, interval, (uint32_t)(row0 * kN + 4 * c),
                       (uint32_t)(row1 * kN + 4 * c), lane, r0, r1);
    quantize_store_row<MODE>(a, row0, c, lane, v0, r0);
    __builtin_amdgcn_sched_barrier(0);   // the rows' quantisers one after the other
    quantize_store_row<MODE>(a, row1, c, lane, v1, r1);
}

// New state rows of chunk q (rows 2(q + 4m) + hf) from the decoded source
// rows: S_new = lam * U + sum_j cs[r][j] B_j (B_j staged in LDS as fp32),
// then rounded and stored.
template <int KMAX, int MODE>
__device__ __forceinline__ void commit_chunk_q(const ReplayParams &a, const Slot &s, float4 (&st)[kPerChunk],
                                               int q, float lam, const float *cs, const float (*sB)[kN],
                                               uint32_t interval) {
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) {
        st[m].x *= lam; st[m].y *= lam; st[m].z *= lam; st[m].w *= lam;
    }
    // An opaque column offset per chunk: the B_j reads are redone for every
    // chunk instead of being hoisted and held (64 VGPRs) across chunks.
    int col = 4 * s.c;
    asm volatile("" : "+v"(col));
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const float4 b = *reinterpret_cast<const float4 *>(&sB[j][col]);
        const float *cp = cs + cs_index<KMAX>(s.hf, q, j, 0);
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
    // all rows of the chunk are complete before any is rounded (keeps the
    // rounding streams from being interleaved with, and stretching, the FMAs)
#pragma unroll
    for (int m = 0; m < kPerChunk; ++m) asm volatile("" : "+v"(st[m].x), "+v"(st[m].y), "+v"(st[m].z), "+v"(st[m].w));
    if constexpr (ModeTraits<MODE>::has_u) {
#pragma unroll
        for (int m = 0; m < kPerChunk; m += 2) {
            const size_t row0 = ((size_t)s.b * a.H + s.h) * kP + 2 * chunk_index(q, m) + s.hf;
            const size_t row1 = ((size_t)s.b * a.H + s.h) * kP + 2 * chunk_index(q, m + 1) + s.hf;
            quantize_store_rows<MODE>(a, row0, row1, s.c, s.lane, st[m], st[m + 1], interval);
            __builtin_amdgcn_sched_barrier(0);   // one row pair's rounding streams at a time
        }
    } else {   // no stochastic rounding (shared FP4): one row at a time
        const uint32_t none[4] = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) {
            const size_t row = ((size_t)s.b * a.H + s.h) * kP + 2 * chunk_index(q, m) + s.hf;
            quantize_store_row<MODE>(a, row, s.c, s.lane, st[m], none);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// Rewrites the whole head from its source (U, or O for the shared mode),
// streaming the source rows chunk by chunk with kNB chunks in flight.
template <int KMAX, int MODE>
__device__ __forceinline__ void commit_head(const ReplayParams &a, const Slot &s, float lam, const float *cs,
                                            const float (*sB)[kN], uint32_t interval) {
    constexpr int UB = ModeTraits<MODE>::ubits;
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP + s.hf;
    typename Raw4<UB>::T raw[kNB][kPerChunk];
#pragma unroll
    for (int q = 0; q < kNB; ++q)
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) raw[q][m] = load_row4<UB>(a, hrow + 2 * chunk_index(q, m), s.c);
    // The commit body is too large for the chunk loop to be unrolled whole;
    // the inner loop over the kNB buffers is, so every buffer index stays
    // static (a dynamic index would move the buffers to scratch memory).
#pragma nounroll
    for (int q0 = 0; q0 < kChunks; q0 += kNB) {
#pragma unroll
        for (int qq = 0; qq < kNB; ++qq) {
            const int q = q0 + qq;
            float4 st[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) st[m] = decode_row4<UB>(raw[qq][m]);
            if (q + kNB < kChunks) {
#pragma unroll
                for (int m = 0; m < kPerChunk; ++m)
                    raw[qq][m] = load_row4<UB>(a, hrow + 2 * chunk_index(q + kNB, m), s.c);
            }
            commit_chunk_q<KMAX, MODE>(a, s, st, q, lam, cs, sB, interval);
        }
    }
}

// ------------------------------------------------------ output streams --
// Rows of the FP4 output copy in the 8-columns-per-lane layout.
struct Fp4Rows {
    uint32_t code[16];   // 8 codes (one dword) of rows 4i + rg
    uint32_t scale[16];  // E4M3 scale of the lane's 32-element block of those rows
};

__device__ __forceinline__ void fp4_rows_load(const ReplayParams &a, const Slot &s, Fp4Rows &o) {
    const int rg = s.lane >> 4, cq = s.lane & 15;
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const size_t row = hrow + 4 * i + rg;
        o.code[i] = *reinterpret_cast<const uint32_t *>(a.oq + row * (kN / 2) + 4 * cq);
        o.scale[i] = a.os[row * (kN / 32) + (cq >> 2)];
    }
}

template <typename TIn>
__device__ __forceinline__ void load_c8(const TIn *Cin, int cq, float (&c8)[8]) {
    const float4 c0 = io<TIn>::load4(Cin + 8 * cq), c1 = io<TIn>::load4(Cin + 8 * cq + 4);
    c8[0] = c0.x; c8[1] = c0.y; c8[2] = c0.z; c8[3] = c0.w;
    c8[4] = c1.x; c8[5] = c1.y; c8[6] = c1.z; c8[7] = c1.w;
}

// The 8 E2M1 values of a dword of codes (element n in nibble n), decoded by
// gfx950's packed FP4 -> f32 conversion with unit scale (exact; the block's
// E4M3 scale, which is not a power of two, is applied by the caller).
typedef float f2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e2m1_decode8(uint32_t w, float (&d)[8]) {
    const f2v a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f2v b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f2v c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f2v e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    d[0] = a.x; d[1] = a.y; d[2] = b.x; d[3] = b.y; d[4] = c.x; d[5] = c.y; d[6] = e.x; d[7] = e.y;
}

// Reduce-scatter of 16 values over the 16 lanes of a DPP row: lane with low
// bits cq keeps the total of item cq.
__device__ __forceinline__ float reduce_scatter16(float (&v)[16], int lane) {
    rs_stage<kDppRowMirror, 8>(v, (lane & 8) != 0);
    rs_stage<kDppRowHalfMirror, 4>(v, (lane & 4) != 0);
    rs_stage<kDppQuadRev, 2>(v, (lane & 2) != 0);
    rs_stage<kDppQuadSwap1, 1>(v, (lane & 1) != 0);
    return v[0];
}

// y0[t] = deq(O) . C_t for this lane's row 4cq + rg, every draft t.  The
// codes are re-decoded per draft (4 packed conversions per 8 values) rather
// than held decoded across drafts (128 VGPRs).
template <int T>
__device__ __forceinline__ void fp4_rows_dot(const Fp4Rows &o, const float (&c8)[T][8], int lane, float (&y0)[T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t w = o.code[i], sraw = o.scale[i];
            if (T > 1) asm volatile("" : "+v"(w), "+v"(sraw));   // fresh decode per draft
            float d[8];
            e2m1_decode8(w, d);
            float acc = 0.f;
#pragma unroll
            for (int n = 0; n < 8; ++n) acc += d[n] * c8[t][n];
            v[i] = acc * e4m3_decode(sraw);
        }
        y0[t] = reduce_scatter16(v, lane);
    }
}

// y0[t] = deq(U) . C_t for this lane's row 2c + hf, every draft t, from the
// raw rows (4-column layout) -- decoded chunk by chunk.
template <int UB, int T>
__device__ __forceinline__ void rows4_dot(const typename Raw4<UB>::T (&raw)[32], const float4 (&C4)[T], int lane,
                                          float (&y0)[T]) {
    float r[T][kChunks];
#pragma unroll
    for (int q = 0; q < kChunks; ++q) {
        float4 st[kPerChunk];
#pragma unroll
        for (int m = 0; m < kPerChunk; ++m) {
            typename Raw4<UB>::T rw = raw[chunk_index(q, m)];
            if constexpr (UB == 16) asm volatile("" : "+v"(rw.x), "+v"(rw.y));   // decode chunk by chunk
            else asm volatile("" : "+v"(rw));
            st[m] = decode_row4<UB>(rw);
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float v[kPerChunk];
#pragma unroll
            for (int m = 0; m < kPerChunk; ++m) v[m] = dot4(st[m], C4[t]);
            r[t][q] = chunk_reduce8(v, lane);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) y0[t] = chunk_combine4(r[t], lane);
}

}  // namespace
}  // namespace rssm
