// quant.h -- low-precision state formats of the precision split on gfx950.
//
// Article ("NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"),
// section 4: a high-precision checkpoint for updates, a separate low-precision
// copy for outputs (4-bit float), and updates stored in 16- or 8-bit floats
// with stochastic rounding (a rounding to one of the two neighbouring
// representable values with probability set by the distance).
//
// Formats (little-endian, row-major like the fp32 checkpoint):
//   bf16   : the upper 16 bits of an fp32.
//   E4M3   : OCP FP8 E4M3 ("FN"): bias 7, no infinities, S.1111.111 = NaN,
//            max 448, subnormal step 2^-9.  Stored unscaled.
//   FP4    : OCP MX E2M1 {0, .5, 1, 1.5, 2, 3, 4, 6} x sign, two codes per
//            byte (even element in the low nibble), one E4M3 scale per 32
//            consecutive elements of a row; scale = RNE_E4M3(amax / 6),
//            code = RNE_E2M1(|v| / scale) saturating at 6 (zero when the
//            scale is zero).
// Stochastic rounding: with lo <= |v| < hi the neighbouring magnitudes and
// r16 a 16-bit draw, round up iff r16 / 2^16 < (|v| - lo) / (hi - lo);
// sign kept; saturating at the largest finite value; NaN -> canonical NaN.
// The draw for element e (flat index ((slot*H + h)*P + p)*N + n of the
// layer) when the state starting interval i is written:
//   Philox4x32-10 (Salmon et al., SC'11), key = (seed lo, seed hi),
//   counter = (e >> 3, i, layer, 0); r16 = 16-bit half (e & 7) of the
//   128-bit output, words in order, low half first.
//
// Everything here works on integer bit patterns and exact fp32 products
// (threshold products t * s have at most 7 significant bits), so results
// are exact and independent of division rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// ------------------------------------------------------------------ Philox --
struct Philox4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input xors (bitop3 truth table 0x96 = A ^ B ^ C), one
        // instruction each with the key word as the scalar operand
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// ------------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_decode(uint32_t code16) { return __uint_as_float(code16 << 16); }

// Written without branches (selects only): the quantisers run on every
// element of a commit.  An infinity needs no case of its own: its code
// 0x7F80 is above the saturation code and is clamped like an overflow.
__device__ __forceinline__ uint32_t bf16_sr(float v, uint32_t r16) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint32_t sign = (bits >> 16) & 0x8000u;
    uint32_t code = (mag >> 16) + (r16 < (mag & 0xFFFFu) ? 1u : 0u);   // a carry moves into the exponent
    code = code < 0x7F7Fu ? code : 0x7F7Fu;                             // saturate instead of inf
    return mag > 0x7F800000u ? 0x7FC0u : (sign | code);                 // NaN -> canonical NaN
}

// ------------------------------------------------------------------- E4M3 --
// Decoding uses gfx950's packed FP8 (OCP E4M3) -> f32 conversion with unit
// scale: exact for every finite code (subnormals m * 2^-9 included, sign
// kept).  The two NaN codes (S.1111.111) are mapped to the canonical quiet
// NaN 0x7FC00000, whatever payload the conversion gives them.
typedef float f2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e4m3_nan_fix(uint32_t code8, float v) {
    return ((code8 & 0x7Fu) == 0x7Fu) ? __uint_as_float(0x7FC00000u) : v;
}

__device__ __forceinline__ float e4m3_decode(uint32_t code8) {
    const f2v_t v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code8 & 0xFFu, 1.0f, false);
    return e4m3_nan_fix(code8 & 0xFFu, v.x);
}

// The four codes of a dword (byte n -> component n).
__device__ __forceinline__ float4 e4m3_decode4(uint32_t w) {
    const f2v_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
    const f2v_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
    return make_float4(e4m3_nan_fix(w & 0xFFu, lo.x), e4m3_nan_fix((w >> 8) & 0xFFu, lo.y),
                       e4m3_nan_fix((w >> 16) & 0xFFu, hi.x), e4m3_nan_fix(w >> 24, hi.y));
}

// Magnitude (fp32 bits, finite, < 448) -> (grid multiple k, quantum exponent
// qe) with k * 2^qe <= |v| and the dropped part D over s bits.
struct GridSplit {
    uint32_t lo;     // |v| truncated onto the E4M3 grid, in units of 2^qe
    uint32_t rem;    // dropped bits (value rem * 2^(qe - s))
    int s;           // number of dropped bits (>= 20)
    int qe;          // quantum exponent: -9 in the subnormal range, e - 3 above
};

__device__ __forceinline__ GridSplit e4m3_split(uint32_t mag) {
    const int E = (int)(mag >> 23);
    const uint32_t M = E ? ((mag & 0x7FFFFFu) | 0x800000u) : (mag & 0x7FFFFFu);
    const int u = E ? E - 150 : -149;                 // exponent of the fp32 ulp
    const int qe = (E - 127 >= -6) ? (E - 127 - 3) : -9;
    const int s = qe - u;
    GridSplit g;
    g.s = s;
    g.qe = qe;
    g.lo = s >= 32 ? 0u : (M >> s);
    g.rem = s >= 32 ? M : (M & ((1u << s) - 1u));
    return g;
}

// E4M3 code of magnitude k * 2^qe (k on the grid of that binade or below).
__device__ __forceinline__ uint32_t e4m3_encode_grid(uint32_t k, int qe) {
    if (qe == -9) return k;                                  // subnormals; k == 8 is 2^-6
    return ((uint32_t)(qe + 3 + 7) << 3) + (k - 8u);         // k in [8, 16]
}

constexpr uint32_t kE4M3MaxBits = 0x43E00000u;   // 448.0f

__device__ __forceinline__ uint32_t e4m3_sr_grid(float v, uint32_t r16) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint32_t sign = (bits >> 24) & 0x80u;
    const GridSplit g = e4m3_split(mag < kE4M3MaxBits ? mag : 0u);
    // up iff r16 * 2^s < rem * 2^16, i.e. r16 < ceil(rem / 2^d) with d = s - 16
    // (d >= 4); rem < 2^24, so clamping d at 31 keeps the ceiling exact
    const int d = g.s - 16 < 31 ? g.s - 16 : 31;
    const uint32_t ceilq = (g.rem >> d) + ((g.rem & ((1u << d) - 1u)) != 0u ? 1u : 0u);
    uint32_t code = e4m3_encode_grid(g.lo + (r16 < ceilq ? 1u : 0u), g.qe);
    code = code < 0x7Eu ? code : 0x7Eu;
    code = mag >= kE4M3MaxBits ? 0x7Eu : code;                  // saturate at 448 (inf too)
    return mag > 0x7F800000u ? 0x7Fu : (sign | code);          // NaN -> canonical NaN
}

// The same rounding in fewer operations (the form the kernels use; the
// conversion self-check compares the two over every fp32 pattern).  In the
// normal range [2^-6, 448) the grid drops the low 20 bits of the fp32
// pattern, and rem > 16 r16 is exactly the carry out of those bits when
// 0xFFFFF - 16 r16 is added, the carry moving into the 3-bit mantissa and
// the exponent where it must; the code is then the pattern's top bits less
// the exponent bias difference.  Below 2^-6 the grid is k 2^-9:
// y = |v| 2^9 = k + f exactly (scaling by a power of two, floor and the
// difference are exact), and the rounding goes up iff r16 < f 2^16.
__device__ __forceinline__ uint32_t e4m3_sr(float v, uint32_t r16) {
    const uint32_t bits = __float_as_uint(v);
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t cn = ((mag + (0xFFFFFu - (r16 << 4))) >> 20) - (120u << 3);
    const float y = __uint_as_float(mag) * 512.0f;
    const float k = floorf(y);
    const uint32_t cs = (uint32_t)k + (((float)r16 < (y - k) * 65536.0f) ? 1u : 0u);
    uint32_t code = mag >= 0x3C800000u ? cn : cs;    // 2^-6: the smallest normal
    code = mag >= kE4M3MaxBits ? 0x7Eu : code;        // saturate at 448 (inf too)
    return mag > 0x7F800000u ? 0x7Fu : (sign | code);  // NaN -> canonical NaN
}

// Round-to-nearest-even of a non-negative finite fp32 magnitude to E4M3,
// saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_mag(float m) {
    const uint32_t mag = __float_as_uint(m);
    const GridSplit g = e4m3_split(mag < kE4M3MaxBits ? mag : 0u);
    // compare rem with half a quantum (2^(s-1)); ties to even k.  rem < 2^24,
    // so from s - 1 >= 24 on the half quantum is larger and nothing rounds up
    const bool small = g.s - 1 < 24;
    const uint32_t half = 1u << (small ? g.s - 1 : 0);
    const bool up = small & ((g.rem > half) | ((g.rem == half) & ((g.lo & 1u) != 0u)));   // no short circuits
    uint32_t code = e4m3_encode_grid(g.lo + (up ? 1u : 0u), g.qe);
    code = code < 0x7Eu ? code : 0x7Eu;
    return mag >= kE4M3MaxBits ? 0x7Eu : code;
}

// ------------------------------------------------------------------- FP4 --
__device__ __forceinline__ float e2m1_decode(uint32_t code4) {
    // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
    const uint32_t e = (code4 >> 1) & 3u, m = code4 & 1u;
    const float mag = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
    return (code4 & 8u) ? -mag : mag;
}

// Scale code of a 32-element block from its max magnitude: RNE_E4M3(amax/6),
// decided exactly: start from the code of amax * (1/6) (within one code of
// the exact one: the product is within an ulp of the quotient, the codes are
// 2^-3 apart relatively) and fix it with exact comparisons against 6 x the
// midpoints between neighbouring codes.
// Both corrections are evaluated unconditionally (no branches; codes at the
// ends of the range compare against a midpoint that cannot be reached).
__device__ __forceinline__ uint32_t fp4_scale_code(float amax) {
    uint32_t c = e4m3_rne_mag(amax * (1.0f / 6.0f));
    // step up when amax is beyond the midpoint to the next code (none above 448)
    const float up6 = 3.0f * (e4m3_decode(c) + e4m3_decode(c + 1u));   // 6 * midpoint, exact
    const bool up = (c < 0x7Eu) & ((amax > up6) | ((amax == up6) & ((c & 1u) != 0u)));
    c += up ? 1u : 0u;
    // step down when amax is below the midpoint to the previous code (none below 0)
    const float dn6 = 3.0f * (e4m3_decode(c - 1u) + e4m3_decode(c));
    const bool dn = (c > 0u) & ((amax < dn6) | ((amax == dn6) & ((c & 1u) != 0u)));
    return c - (dn ? 1u : 0u);
}

// E2M1 code (sign in bit 3) of v against scale s > 0, by exact threshold
// comparisons of |v| with t * s, t in {.25, .75, 1.25, 1.75, 2.5, 3.5, 5};
// midpoints go to the even mantissa (0, 1, 2, 4).
struct Fp4Thresholds {
    float t025, t075, t125, t175, t250, t350, t500;
};

__device__ __forceinline__ Fp4Thresholds fp4_thresholds(float s) {
    return {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
}

// The code is the number of thresholds |v| passes (counted without branches).
__device__ __forceinline__ uint32_t fp4_encode(float v, const Fp4Thresholds &t, bool zero_scale) {
    const float a = fabsf(v);
    uint32_t k = (a > t.t025) + (a >= t.t075) + (a > t.t125) + (a >= t.t175) + (a > t.t250) +
                 (a >= t.t350) + (a > t.t500);
    if (zero_scale) k = 0;
    return k | ((__float_as_uint(v) >> 28) & 8u);
}

}  // namespace rssm
