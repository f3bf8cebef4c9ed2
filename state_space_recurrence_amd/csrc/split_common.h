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

// ----------------------------------------------------------- 4-col rows --
// Raw source values of 4 consecutive elements (columns 4c..4c+3) of a row,
// in the update-source format UB (16: bf16, 8: E4M3, 4: FP4 code16 | scale<<16).
template <int UB> struct Raw4;
template <> struct Raw4<16> { using T = uint2; };
template <> struct Raw4<8> { using T = uint32_t; };
template <> struct Raw4<4> { using T = uint32_t; };

template <int UB>
__device__ __forceinline__ typename Raw4<UB>::T load_row4(const ReplayParams &a, size_t row, int c) {
    // (the single checkpoint is streamed whole on every step: non-temporal,
    // like the fp32 checkpoint stream)
    if constexpr (UB == 16) {
        typedef unsigned int u2v __attribute__((ext_vector_type(2)));
        const u2v t = __builtin_nontemporal_load(
            reinterpret_cast<const u2v *>(reinterpret_cast<const uint16_t *>(a.u) + row * kN + 4 * c));
        return make_uint2(t.x, t.y);
    } else if constexpr (UB == 8) {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(a.u) + row * kN + 4 * c));
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

__device__ __forceinline__ void sr_draws4_pair(uint64_t seed, uint32_t layer, uint32_t interval, size_t e0,
                                               size_t e1, int lane, uint32_t (&r0)[4], uint32_t (&r1)[4]) {
    const bool odd = lane & 1;
    // the counter is the low word of e / 8 (e itself may pass 2^32 in a large pool)
    const Philox4 o = philox4x32_10((uint32_t)((odd ? e1 : e0) >> 3), interval, layer, 0, (uint32_t)seed,
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
        sr_draws4_pair(a.seed, (uint32_t)a.layer, interval, row0 * kN + 4 * c, row1 * kN + 4 * c, lane, r0, r1);
    quantize_store_row<MODE>(a, row0, c, lane, v0, r0);
    __builtin_amdgcn_sched_barrier(0);   // the rows' quantisers one after the other
    quantize_store_row<MODE>(a, row1, c, lane, v1, r1);
}

// ------------------------------------------------------ output streams --
// A lane's whole row of the FP4 copy (lane = row): 128 codes in four 16-byte
// pieces (piece i = block i, columns 32i..32i+31, element n in nibble n of
// its dword) and the row's four block scales in one dword (byte i = block
// i).  A wave reads the head's 4 KB of codes and 256 B of scales in five
// contiguous wave-wide loads.
struct Fp4Row {
    uint4 code[4];
    uint32_t scale;
};

__device__ __forceinline__ void fp4_row_load(const ReplayParams &a, const Slot &s, Fp4Row &o) {
    const size_t hrow = ((size_t)s.b * a.H + s.h) * kP;
    const __amdgpu_buffer_rsrc_t rc = uniform_rsrc(a.oq + hrow * (kN / 2), kP * (kN / 2));
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(a.os + hrow * (kN / 32), kP * (kN / 32));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o.code[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, s.lane * (kN / 2) + 16 * i, 0, 0));
    o.scale = __builtin_amdgcn_raw_buffer_load_b32(rs, s.lane * (kN / 32), 0, 0);
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// deq(row) . C for a lane's whole row (Fp4Row), C read from LDS: 128 bf16 as
// 64 packed pairs (pair p = columns 2p, 2p+1), the same for every lane.  Per
// block: the codes widened exactly to bf16 meet the pairs in packed bf16 dots
// (exact products), then the block's scale; blocks summed in order.
__device__ __forceinline__ float fp4_row_dot(const Fp4Row &o, const uint16_t *sC) {
    const uint32_t *cp = reinterpret_cast<const uint32_t *>(sC);
    float y = 0.f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const uint32_t w[4] = {o.code[blk].x, o.code[blk].y, o.code[blk].z, o.code[blk].w};
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint4 c = *reinterpret_cast<const uint4 *>(cp + 16 * blk + 4 * d);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 0),
                                                  __builtin_bit_cast(bf16x2, c.x), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 1),
                                                  __builtin_bit_cast(bf16x2, c.y), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 2),
                                                  __builtin_bit_cast(bf16x2, c.z), acc, false);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 3),
                                                  __builtin_bit_cast(bf16x2, c.w), acc, false);
        }
        y += acc * e4m3_decode((o.scale >> (8 * blk)) & 0xFFu);
    }
    return y;
}

// The same for T drafts at once (C of draft t at sC[t]): each pair of codes is
// widened once and meets the T drafts' pairs, so the conversions do not grow
// with T and no widened row is held.  Per draft the same products and sums in
// the same order as fp4_row_dot.
template <int T>
__device__ __forceinline__ void fp4_row_dots(const Fp4Row &o, const uint16_t (*sC)[kN], float (&y)[T]) {
#pragma unroll
    for (int t = 0; t < T; ++t) y[t] = 0.f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const uint32_t w[4] = {o.code[blk].x, o.code[blk].y, o.code[blk].z, o.code[blk].w};
        float acc[T];
#pragma unroll
        for (int t = 0; t < T; ++t) acc[t] = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint4 c[T];
#pragma unroll
            for (int t = 0; t < T; ++t) c[t] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint32_t *>(sC[t]) + 16 * blk + 4 * d);
            const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 0);
            const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 1);
            const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 2);
            const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[d], 1.0f, 3);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                acc[t] = __builtin_amdgcn_fdot2_f32_bf16(v0, __builtin_bit_cast(bf16x2, c[t].x), acc[t], false);
                acc[t] = __builtin_amdgcn_fdot2_f32_bf16(v1, __builtin_bit_cast(bf16x2, c[t].y), acc[t], false);
                acc[t] = __builtin_amdgcn_fdot2_f32_bf16(v2, __builtin_bit_cast(bf16x2, c[t].z), acc[t], false);
                acc[t] = __builtin_amdgcn_fdot2_f32_bf16(v3, __builtin_bit_cast(bf16x2, c[t].w), acc[t], false);
            }
            __builtin_amdgcn_sched_barrier(0);   // one dword of codes (T drafts' C pieces) live at a time
        }
        const float sc = e4m3_decode((o.scale >> (8 * blk)) & 0xFFu);
#pragma unroll
        for (int t = 0; t < T; ++t) y[t] += acc[t] * sc;
    }
}

// The same with fp32 C in LDS (128 floats): codes widened to f32, one fused
// multiply-add per element.
__device__ __forceinline__ float fp4_row_dot(const Fp4Row &o, const float *sC) {
    float y = 0.f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        const uint32_t w[4] = {o.code[blk].x, o.code[blk].y, o.code[blk].z, o.code[blk].w};
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float v[8];
            e2m1_decode8(w[d], v);
            const float4 c0 = *reinterpret_cast<const float4 *>(sC + 32 * blk + 8 * d);
            const float4 c1 = *reinterpret_cast<const float4 *>(sC + 32 * blk + 8 * d + 4);
            acc += v[0] * c0.x + v[1] * c0.y + v[2] * c0.z + v[3] * c0.w;
            acc += v[4] * c1.x + v[5] * c1.y + v[6] * c1.z + v[7] * c1.w;
        }
        y += acc * e4m3_decode((o.scale >> (8 * blk)) & 0xFFu);
    }
    return y;
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


// -------------------------------------------------- matrix-core commit --
// A commit's rank-K update S_new = lam U + sum_j cs[r][j] B_j is a dense
// contraction (per wave: 16 rows x 128 columns x K entries) and runs on the
// matrix cores, v_mfma_f32_16x16x4_f32, with the state transposed (the MFMA
// row index is the state column) so that the accumulators land in the
// layout the quantisers want: lane l = 16 g + pl of a wave holds state row
// pl of the wave's 16 rows, columns 32g .. 32g+31 -- one whole FP4 scale
// block and the 32 draws of four whole Philox counters, so the block scale
// needs no cross-lane step and the draws no exchange.
//   A (16 x 4; lane i + 16k holds A[i][k]):  A[i][k] = B_{4kb+k}[8i + t]
//   B (4 x 16; lane j + 16k holds B[k][j]):  B[k][j] = cs[row j][4kb + k]
//   D (16 x 16; lane j + 16(i/4), register i % 4, holds D[i][j]):
//      state row j, column 8i + t  ->  lane (pl = j, g = i / 4), register
//      v = i % 4 of tile t: column 32g + 8v + t.
// A lane's block is held as e[32], e[i] = column 32g + i (i = 8v + t).

// Raw update-source values of one lane's 32-column block.
template <int UB> struct RawBlock;
template <> struct RawBlock<16> { uint4 q[4]; };               // 32 bf16
template <> struct RawBlock<8> { uint4 q[2]; };                // 32 E4M3
template <> struct RawBlock<4> { uint4 q[1]; uint32_t sc; };   // 32 E2M1 codes + the block's E4M3 scale

// base + byte_off with the offset kept 32-bit, so that a wave-uniform base
// and a per-lane offset address memory as scalar base + vector offset.
template <typename T>
__device__ __forceinline__ T *off_bytes(T *base, uint32_t byte_off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ const T *off_bytes(const T *base, uint32_t byte_off) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

// Where a lane's block lives: the first state row of the wave's 16 rows
// (wave-uniform, so the pointers below are a scalar base plus a 32-bit lane
// offset), the lane's row among them and its column block.
struct BlockAt {
    size_t row0;
    int r, g;
};

// Byte pitch of a row in a wave's LDS staging tile of 16 rows (padded by 16
// bytes: a 16-byte access per lane to one column of all 16 rows, and a row
// written contiguously, each touch every bank once).
template <int UB>
constexpr int stage_pitch() { return kN * (UB >= 8 ? UB / 8 : 1) + 16; }

// Loads the update source of the wave's 16 rows.  For bf16 and E4M3 the
// block is requested coalesced -- load k of lane l is bytes 1024 k + 16 l of
// the 16 contiguous rows, whole cache lines per instruction -- and moved to
// the lane layout by block_to_lanes; requesting each lane's own 32 columns
// directly touches every line of the rows with every instruction (measured
// 14 % slower on the commit's full stream).  The loads are non-temporal: the
// update source is streamed once per interval and would otherwise displace
// the output copies and buffer entries that the next steps read from the
// fabric cache.
template <int UB>
__device__ __forceinline__ void load_block(const ReplayParams &a, const BlockAt &at, RawBlock<UB> &r) {
    if constexpr (UB == 16 || UB == 8) {
        constexpr int eb = UB / 8;   // bytes per element
        const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(a.u) + at.row0 * (kN * eb));
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < 2 * eb; ++k) r.q[k] = stream_load16(p + 64 * k + lane);
    } else {
        r.q[0] = *off_bytes(reinterpret_cast<const uint4 *>(a.oq + at.row0 * (kN / 2)), (uint32_t)(at.r * (kN / 2) + 16 * at.g));
        r.sc = *off_bytes(a.os + at.row0 * (kN / 32), (uint32_t)(at.r * (kN / 32) + at.g));
    }
}

// The coalesced block of load_block into the lane layout (lane: row at.r,
// columns 32 at.g .. 32 at.g + 31) through the wave's LDS tile `stage`.  The
// caller's wave owns the tile; LDS accesses of one wave complete in order, so
// the reads see these writes and earlier reads of the tile are done.
template <int UB>
__device__ __forceinline__ void block_to_lanes(const BlockAt &at, RawBlock<UB> &r, uint8_t *stage) {
    if constexpr (UB == 16 || UB == 8) {
        constexpr int eb = UB / 8, rowb = kN * eb, pitch = stage_pitch<UB>();
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < 2 * eb; ++k) {
            const int i = 1024 * k + 16 * lane;   // byte within the 16 rows
            *reinterpret_cast<uint4 *>(stage + (i / rowb) * pitch + i % rowb) = r.q[k];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int k = 0; k < 2 * eb; ++k)
            r.q[k] = *reinterpret_cast<const uint4 *>(stage + at.r * pitch + 32 * at.g * eb + 16 * k);
        __builtin_amdgcn_wave_barrier();
    }
}

__device__ __forceinline__ void words_of(const uint4 &q, uint32_t (&w)[4]) {
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
}

template <int UB>
__device__ __forceinline__ void decode_block(const RawBlock<UB> &r, float (&e)[32]) {
    if constexpr (UB == 16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t w[4];
            words_of(r.q[k], w);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                e[8 * k + 2 * m] = __uint_as_float(w[m] << 16);
                e[8 * k + 2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
            }
        }
    } else if constexpr (UB == 8) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t w[4];
            words_of(r.q[k], w);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 d = e4m3_decode4(w[m]);
                e[16 * k + 4 * m] = d.x; e[16 * k + 4 * m + 1] = d.y;
                e[16 * k + 4 * m + 2] = d.z; e[16 * k + 4 * m + 3] = d.w;
            }
        }
    } else {
        const float s = e4m3_decode(r.sc);
        uint32_t w[4];
        words_of(r.q[0], w);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float d[8];
            e2m1_decode8(w[m], d);
#pragma unroll
            for (int n = 0; n < 8; ++n) e[8 * m + n] = d[n] * s;
        }
    }
}

// The lane's A operands of entry block kb: B_{4kb+g}[8pl .. 8pl+7] as
// stored (8 bf16 or 8 fp32 values).
template <typename TIn>
struct B8 {
    uint4 q[sizeof(TIn) / 2];
};

template <typename TIn>
__device__ __forceinline__ void load_b8(const TIn *p, B8<TIn> &r) {
#pragma unroll
    for (int i = 0; i < (int)(sizeof(TIn) / 2); ++i) r.q[i] = reinterpret_cast<const uint4 *>(p)[i];
}

template <typename TIn>
__device__ __forceinline__ void widen_b8(const B8<TIn> &r, float (&v)[8]) {
    if constexpr (sizeof(TIn) == 2) {
        uint32_t w[4];
        words_of(r.q[0], w);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            v[2 * m] = __uint_as_float(w[m] << 16);
            v[2 * m + 1] = __uint_as_float(w[m] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint32_t w[4];
            words_of(r.q[i], w);
#pragma unroll
            for (int m = 0; m < 4; ++m) v[4 * i + m] = __uint_as_float(w[m]);
        }
    }
}

// e <- lam e + sum_{j<K} cf_j B_j on the lane's block; cf[kb] is the
// coefficient of entry j = 4kb + g for the lane's row (zero from K on), bo
// the lane's A operands (entries from K on are replaced by zeros here).  K
// is wave-uniform.
template <typename TIn, int KMAX>
__device__ __forceinline__ void mfma_update(float (&e)[32], float lam, const float (&cf)[KMAX / 4],
                                            const B8<TIn> (&bo)[KMAX / 4], int g, int K) {
    f4v acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f4v{lam * e[t], lam * e[8 + t], lam * e[16 + t], lam * e[24 + t]};
#pragma unroll
    for (int kb = 0; kb < KMAX / 4; ++kb) {
        if (4 * kb >= K) break;
        // widened at each use, not once for all calls (32 or 64 VGPRs)
        B8<TIn> braw = bo[kb];
#pragma unroll
        for (int i = 0; i < (int)(sizeof(TIn) / 2); ++i)
            asm volatile("" : "+v"(braw.q[i].x), "+v"(braw.q[i].y), "+v"(braw.q[i].z), "+v"(braw.q[i].w));
        float bv[8];
        widen_b8<TIn>(braw, bv);
        const bool live = 4 * kb + g < K;
#pragma unroll
        for (int t = 0; t < 8; ++t) bv[t] = live ? bv[t] : 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(bv[t], cf[kb], acc[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        e[t] = acc[t].x; e[8 + t] = acc[t].y; e[16 + t] = acc[t].z; e[24 + t] = acc[t].w;
    }
}

// bf16 stochastic rounding of two values by integer addition: adding
// 0xFFFF - r16 to the fp32 bits carries into bit 16 exactly when the dropped
// low half exceeds r16 (the rounding rule of bf16_sr), the carry moving into
// the exponent where it must.  Valid for |v| <= 0x7F7F0000 as bits (finite,
// no rounding past the largest bf16); draws: low half of w for v0, high
// half for v1.  Returns the two codes packed (v0 low).
__device__ __forceinline__ uint32_t bf16_sr_pair_plain(float v0, float v1, uint32_t w) {
    const uint32_t nw = ~w;
    const uint32_t x0 = __float_as_uint(v0) + (nw & 0xFFFFu);
    const uint32_t x1 = __float_as_uint(v1) + (nw >> 16);
    return __builtin_amdgcn_perm(x1, x0, 0x07060302u);   // high halves of x0, x1
}

// FP4 codes of 8 values (element n in nibble n) scaled by r, by gfx950's
// f32 -> E2M1 conversion at unit scale (round to nearest even, saturating at
// 6, sign kept: identical to the threshold encoding for every non-NaN fp32).
__device__ __forceinline__ uint32_t fp4_cvt8(const float *v, float r) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * r, v[1] * r, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * r, v[3] * r, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * r, v[5] * r, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * r, v[7] * r, 1.0f, 3);
    return w;
}

// FP4 codes of 8 values by the exact threshold comparisons.
__device__ __forceinline__ uint32_t fp4_exact8(const float *v, const Fp4Thresholds &t, bool z) {
    uint32_t w = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) w |= fp4_encode(v[n], t, z) << (4 * n);
    return w;
}

// Rounds and stores a lane's block of a new state (row row0 + r, columns
// 32g..32g+31): the update checkpoint by stochastic rounding with the draws
// of stream index `interval` (through `stage`, the wave's LDS tile of
// 16 x (128 x bytes + 16) bytes), the output copy by FP4 quantisation with
// the block's own scale.  Called by the whole wave with one row0.
//
// FP4 codes: RNE_E2M1(|v| / s) is decided exactly without comparing against
// the seven thresholds t s: with r = rcp(s), every product v r (1 -+ 2^-20)
// lies strictly below / above |v| / s in magnitude (rcp and the products
// are within a few ulps), so where the two products convert to the same
// code (monotone conversion) that code is the exact one.  Otherwise --
// |v| / s within about 2^-20 of a threshold, ties included -- the block is
// encoded again by the threshold comparisons.  Blocks holding a value
// beyond the largest bf16 (infinities, NaN) take the general quantisers.
template <int MODE>
__device__ __forceinline__ void quantize_store_block(const ReplayParams &a, const BlockAt &at, const float (&e)[32],
                                                     uint32_t interval, uint8_t *stage) {
    using MT = ModeTraits<MODE>;
    const int g = at.g;
    const uint32_t lrow = (uint32_t)(at.r * kN + 32 * g);   // the lane's element offset from row0
    if (a.dbg) {
        float *db = off_bytes(a.dbg + at.row0 * kN, lrow * 4);
#pragma unroll
        for (int k = 0; k < 8; ++k)
            stream_store4(db + 4 * k, make_float4(e[4 * k], e[4 * k + 1], e[4 * k + 2], e[4 * k + 3]));
    }
    // the largest magnitude bit pattern from two three-way reductions of the
    // raw bits: the unsigned maximum is the largest negative value's pattern
    // (sign set) when there is one, the signed maximum the largest
    // non-negative value's (negative when there is none)
    uint32_t umax = 0;
    int32_t imax = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
        umax = max(umax, max(__float_as_uint(e[i]), __float_as_uint(e[i + 1])));   // v_max3_u32
        imax = max(imax, max(__float_as_int(e[i]), __float_as_int(e[i + 1])));      // v_max3_i32
    }
    const uint32_t mmag = max(umax & 0x7FFFFFFFu, (uint32_t)imax);   // imax starts at 0: never negative
    const bool plain = mmag <= 0x7F7F0000u;
    if constexpr (MT::has_u) {
        // The rounded block goes through the wave's LDS tile (16 rows of the
        // update checkpoint) and leaves it in 1 KB contiguous stores: the
        // MFMA layout would store 16 or 8 bytes per lane 64 or 32 bytes
        // apart (four times the write requests of a contiguous store).
        constexpr int eb = MT::ubits / 8;               // bytes per element
        constexpr int rowb = kN * eb, pitch = stage_pitch<MT::ubits>();   // padded tile rows: no bank conflicts
        uint8_t *tile = stage + at.r * pitch + 32 * g * eb;
        // the draws of the lane's four counters (element index / 8 =
        // row * 16 + 4g + k); the key and the uniform counter words are
        // fenced per call so the uniform parts of the rounds are recomputed
        // (scalar ALU) rather than hoisted out of the caller's loops
        auto draws = [&](int k) {
            uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32), c1 = interval, c2 = (uint32_t)a.layer;
            asm volatile("" : "+s"(k0), "+s"(k1), "+s"(c1), "+s"(c2));
            return philox4x32_10((uint32_t)(at.row0 * (kN / 8)) + (lrow >> 3) + k, c1, c2, 0, k0, k1);
        };
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const Philox4 o = draws(k);
            const uint32_t w[4] = {o.x, o.y, o.z, o.w};
            const float *v = e + 8 * k;
            if constexpr (MT::ubits == 16) {
                uint32_t q[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) q[m] = bf16_sr_pair_plain(v[2 * m], v[2 * m + 1], w[m]);
                *reinterpret_cast<uint4 *>(tile + 16 * k) = make_uint4(q[0], q[1], q[2], q[3]);
            } else {
                uint32_t q[2];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    q[m] = e4m3_sr(v[4 * m], w[2 * m] & 0xFFFFu) | (e4m3_sr(v[4 * m + 1], w[2 * m] >> 16) << 8) |
                           (e4m3_sr(v[4 * m + 2], w[2 * m + 1] & 0xFFFFu) << 16) |
                           (e4m3_sr(v[4 * m + 3], w[2 * m + 1] >> 16) << 24);
                *reinterpret_cast<uint2 *>(tile + 8 * k) = make_uint2(q[0], q[1]);
            }
        }
        if constexpr (MT::ubits == 16) {
            if (!plain) {   // rare: a value beyond the largest bf16 (inf, NaN): the general rounding again
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const Philox4 o = draws(k);
                    const uint32_t w[4] = {o.x, o.y, o.z, o.w};
                    uint32_t q[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float v0 = e[8 * k + 2 * m], v1 = e[8 * k + 2 * m + 1];
                        q[m] = bf16_sr(v0, w[m] & 0xFFFFu) | (bf16_sr(v1, w[m] >> 16) << 16);
                    }
                    *reinterpret_cast<uint4 *>(tile + 16 * k) = make_uint4(q[0], q[1], q[2], q[3]);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        // 16 contiguous rows: lane l copies bytes 16 l + 1024 m of the tile
        uint8_t *ub = reinterpret_cast<uint8_t *>(a.u) + at.row0 * rowb;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int m = 0; m < 16 * rowb / 1024; ++m) {
            const uint32_t i = 1024 * m + 16 * lane;   // byte within the 16 rows
            const uint4 d = *reinterpret_cast<const uint4 *>(stage + (i / rowb) * pitch + i % rowb);
            stream_store16(off_bytes(reinterpret_cast<uint4 *>(ub), i), d);
        }
        __builtin_amdgcn_wave_barrier();
    }
    if constexpr (MT::has_o) {
        uint32_t c[4];
        uint32_t sc;
        bool exact = !plain;
        if (plain) {
            sc = fp4_scale_code(__uint_as_float(mmag));
            const float r = sc == 0u ? 0.f : __builtin_amdgcn_rcpf(e4m3_decode(sc));
            const float rlo = r * (1.0f - 0x1p-20f), rhi = r * (1.0f + 0x1p-20f);
            uint32_t diff = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                c[k] = fp4_cvt8(e + 8 * k, rlo);
                diff |= c[k] ^ fp4_cvt8(e + 8 * k, rhi);
            }
            exact = diff != 0u;
        }
        if (exact) {   // rare: a value within ~2^-20 of a threshold, or a non-plain block
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(e[i]));
            sc = fp4_scale_code(amax);
            const Fp4Thresholds t = fp4_thresholds(e4m3_decode(sc));
#pragma unroll
            for (int k = 0; k < 4; ++k) c[k] = fp4_exact8(e + 8 * k, t, sc == 0u);
        }
        // (the commit's stores are non-temporal: written back to memory as
        // they go, not left dirty in the fabric cache for the next launches
        // to evict)
        stream_store16(off_bytes(reinterpret_cast<uint4 *>(a.oq + at.row0 * (kN / 2)), lrow / 2),
                       make_uint4(c[0], c[1], c[2], c[3]));
        __builtin_nontemporal_store((uint8_t)sc, off_bytes(a.os + at.row0 * (kN / 32), lrow / 32));
    }
}

}  // namespace
}  // namespace rssm
