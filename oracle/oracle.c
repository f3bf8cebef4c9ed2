/*
 * oracle.c -- plain fp64 CPU oracle for the ReplaySSM decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header, table or constant with
 * the HIP library; the two are written independently.
 *
 * Source: "NVIDIA ReplaySSM: hybrid model SSM decoding with a state buffer"
 * (devotd.net news article, English / Chinese / Korean editions).  The pages
 * state the method in words only; the per-token recurrence used here is the
 * conventional SSM decode update the article's section 1 ("Store recent inputs
 * instead of the full state") says every token performs:
 *
 *     a_t = exp(dt_t * A_h)
 *     S_t = a_t * S_{t-1} + dt_t * x_t (outer) B_t          (P x N per head)
 *     y_t = S_t . C_t + D_h * x_t                            (post-update state)
 *
 * with B and C shared by the heads of one group (g = h / (H/G), contiguous).
 *
 * Everything here is the plain definition, evaluated token by token in fp64:
 *  - oracle_recurrent:   the recurrence above (sections 1 and 2 of the pages:
 *                        ReplaySSM's outputs must match it within fp error).
 *  - oracle_spec_round:  speculative verification (section 3): the outputs of
 *                        T draft positions from a scratch copy of the state,
 *                        then only the first n_keep positions are applied to
 *                        the real state; rejected drafts never touch it.
 *  - codecs:             bf16, OCP FP8 E4M3 (E4M3FN) and OCP FP4 E2M1 with a
 *                        per-32-element E4M3 scale, decoded from their field
 *                        definitions and rounded in the value domain (no bit
 *                        tricks), for the precision split of section 4.
 *  - stochastic rounding (section 4: round to a neighbouring representable
 *                        value with probability set by the distance), driven
 *                        by Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 *                        "Parallel random numbers: as easy as 1, 2, 3",
 *                        SC'11), written from that paper's definition.
 *
 * Parallelism: OpenMP over independent (slot, head) pairs only; the arithmetic
 * of each pair is the sequential definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the following parallel regions (timing on 1 core vs all). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* Conventional per-token recurrence (the definition).                      */
/* ------------------------------------------------------------------------ */

/* One token for one (slot, head): S <- a*S + dt*x(outer)B ; y = S.C + D*x. */
static void token_update(int64_t P, int64_t N, double *s, double dt, double A,
                         double Dh, const double *x, const double *Bv,
                         const double *Cv, double *y)
{
    double a = exp(dt * A);
    for (int64_t p = 0; p < P; ++p) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            double v = a * s[p * N + n] + dt * x[p] * Bv[n];
            s[p * N + n] = v;
            acc += v * Cv[n];
        }
        y[p] = acc + Dh * x[p];
    }
}

/*
 * Run `steps` tokens of the recurrence for every slot and head.
 *   S  [batch, heads, P, N]        state, updated in place
 *   x  [steps, batch, heads, P]    B/C [steps, batch, groups, N]
 *   dt [steps, batch, heads]       A, D [heads]
 *   y  [steps, batch, heads, P]    outputs (may be NULL)
 */
void oracle_recurrent(int64_t batch, int64_t heads, int64_t P, int64_t N,
                      int64_t groups, int64_t steps, double *S,
                      const double *x, const double *Bm, const double *Cm,
                      const double *dt, const double *A, const double *D,
                      double *y)
{
    int64_t hpg = heads / groups;
    int64_t nbh = batch * heads;
#pragma omp parallel
    {
        double *ytmp = (double *)malloc(sizeof(double) * (size_t)P);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < nbh; ++bh) {
            int64_t b = bh / heads, h = bh % heads, g = h / hpg;
            double *s = S + bh * P * N;
            for (int64_t t = 0; t < steps; ++t) {
                int64_t tb = t * batch + b;
                double *yo = y ? y + (tb * heads + h) * P : ytmp;
                token_update(P, N, s, dt[tb * heads + h], A[h], D[h],
                             x + (tb * heads + h) * P, Bm + (tb * groups + g) * N,
                             Cm + (tb * groups + g) * N, yo);
            }
        }
        free(ytmp);
    }
}

/*
 * One speculative round: T draft positions per slot.
 *   outputs y[T, batch, heads, P] from a scratch copy of S stepped through all
 *   T positions; afterwards S holds the state after the first n_keep[b]
 *   positions (0 <= n_keep <= T; 0 leaves S unchanged).
 *   x [T, batch, heads, P], B/C [T, batch, groups, N], dt [T, batch, heads].
 */
void oracle_spec_round(int64_t batch, int64_t heads, int64_t P, int64_t N,
                       int64_t groups, int64_t T, double *S, const double *x,
                       const double *Bm, const double *Cm, const double *dt,
                       const double *A, const double *D, const int32_t *n_keep,
                       double *y)
{
    int64_t hpg = heads / groups;
    int64_t nbh = batch * heads;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(P * N));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < nbh; ++bh) {
            int64_t b = bh / heads, h = bh % heads, g = h / hpg;
            double *s = S + bh * P * N;
            memcpy(work, s, sizeof(double) * (size_t)(P * N));
            for (int64_t t = 0; t < T; ++t) {
                int64_t tb = t * batch + b;
                token_update(P, N, work, dt[tb * heads + h], A[h], D[h],
                             x + (tb * heads + h) * P, Bm + (tb * groups + g) * N,
                             Cm + (tb * groups + g) * N, y + (tb * heads + h) * P);
                if (t + 1 == (int64_t)n_keep[b])
                    memcpy(s, work, sizeof(double) * (size_t)(P * N));
            }
        }
        free(work);
    }
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11, section 4: Philox-4x32 with 10      */
/* rounds; multipliers and Weyl key increments as published there).        */
/* ------------------------------------------------------------------------ */

void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4])
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = M0 * (uint64_t)c0;   /* 32x32 -> 64 products */
        uint64_t p1 = M1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The 16-bit random draw for element `elem` of layer `layer` when the state
 * that starts interval `interval` is written:
 *   key = (seed low word, seed high word)
 *   counter = (elem / 8, interval, layer, 0)
 *   draw = 16-bit half (elem mod 8) of the 128-bit output, words in order,
 *          low half of each word first.
 */
uint32_t oracle_sr_draw(uint64_t seed, uint32_t layer, uint32_t interval,
                        uint64_t elem)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {(uint32_t)(elem / 8), interval, layer, 0};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    unsigned idx = (unsigned)(elem % 8);
    uint32_t word = out[idx / 2];
    return (idx % 2 == 0) ? (word & 0xFFFFu) : (word >> 16);
}

/* ------------------------------------------------------------------------ */
/* Small floating-point formats, value domain.                              */
/*                                                                          */
/* A binary format with `mant` stored mantissa bits, minimum normal          */
/* exponent `emin` and largest finite magnitude `maxv` represents, in each   */
/* binade [2^e, 2^(e+1)) with e >= emin, the multiples of 2^(e-mant); below  */
/* 2^emin it represents the multiples of 2^(emin-mant) (subnormals).         */
/*   bf16:  mant 7, emin -126, max (2 - 2^-7) * 2^127                       */
/*   E4M3:  mant 3, emin -6,   max 448  (OCP FP8, E4M3FN variant)           */
/*   E2M1:  mant 1, emin 0,    max 6    (OCP MX FP4)                        */
/* ------------------------------------------------------------------------ */

typedef struct { int mant; int emin; double maxv; } fmt_t;

static const fmt_t FMT_BF16 = {7, -126, 3.3895313892515355e38};
static const fmt_t FMT_E4M3 = {3, -6, 448.0};
static const fmt_t FMT_E2M1 = {1, 0, 6.0};

/* Grid spacing of the format around magnitude m > 0. */
static double quantum(const fmt_t *f, double m)
{
    int e;
    (void)frexp(m, &e);         /* m = fr * 2^e, fr in [0.5, 1) */
    int ex = e - 1;             /* floor(log2(m)) */
    if (ex < f->emin) ex = f->emin;
    return ldexp(1.0, ex - f->mant);
}

/* Representable neighbours lo <= m < hi of a magnitude m >= 0 (lo == m when
 * m is on the grid).  All quantities are exact in double for fp32 inputs. */
static void neighbours(const fmt_t *f, double m, double *lo, double *hi)
{
    if (m == 0.0) { *lo = 0.0; *hi = 0.0; return; }
    double q = quantum(f, m);
    double l = floor(m / q) * q;
    *lo = l;
    *hi = l + q;
}

/* Round-to-nearest, ties to even mantissa, saturating at maxv. */
static double round_rne(const fmt_t *f, double m)
{
    double lo, hi;
    neighbours(f, m, &lo, &hi);
    double r;
    if (m == lo) r = lo;
    else {
        double dlo = m - lo, dhi = hi - m;
        if (dlo < dhi) r = lo;
        else if (dhi < dlo) r = hi;
        else {
            double q = hi - lo;
            double k = lo / q;      /* integer multiple; even mantissa <=> even k */
            r = (fmod(k, 2.0) == 0.0) ? lo : hi;
        }
    }
    return r > f->maxv ? f->maxv : r;
}

/* Stochastic rounding of magnitude m with a 16-bit draw r: round up to the
 * upper neighbour iff r / 2^16 < (m - lo) / (hi - lo); saturating at maxv. */
static double round_sr(const fmt_t *f, double m, uint32_t r16)
{
    double lo, hi;
    neighbours(f, m, &lo, &hi);
    double r = lo;
    if (m != lo) {
        double frac = (m - lo) / (hi - lo);         /* exact: hi - lo is 2^k */
        if ((double)r16 < frac * 65536.0) r = hi;
    }
    return r > f->maxv ? f->maxv : r;
}

/* ---- bf16 ---------------------------------------------------------------- */
/* bf16 value = (-1)^s * 2^(E-127) * (1 + M/128) for E in 1..254,
 *              (-1)^s * 2^-126 * M/128 for E == 0; E == 255: inf/NaN. */
double oracle_bf16_decode(uint16_t code)
{
    int s = (code >> 15) & 1, E = (code >> 7) & 0xFF, M = code & 0x7F;
    double v;
    if (E == 0xFF) v = (M == 0) ? INFINITY : NAN;
    else if (E == 0) v = ldexp((double)M / 128.0, -126);
    else v = ldexp(1.0 + (double)M / 128.0, E - 127);
    return s ? -v : v;
}

static uint16_t bf16_encode_exact(double m, int neg)
{
    /* m is a representable non-negative bf16 magnitude */
    uint16_t code;
    if (m == 0.0) code = 0;
    else {
        int e; double fr = frexp(m, &e);    /* m = fr*2^e */
        int ex = e - 1;
        if (ex < -126) {                     /* subnormal */
            code = (uint16_t)(m / ldexp(1.0, -133));
        } else {
            double mant = fr * 2.0 - 1.0;    /* in [0,1) */
            code = (uint16_t)(((ex + 127) << 7) | (int)(mant * 128.0));
        }
    }
    return (uint16_t)(code | (neg ? 0x8000 : 0));
}

uint16_t oracle_bf16_sr(float v, uint32_t r16)
{
    if (isnan(v)) return 0x7FC0;
    double d = (double)v;
    int neg = signbit(d) != 0;
    double m = fabs(d);
    if (isinf(m)) m = FMT_BF16.maxv;
    return bf16_encode_exact(round_sr(&FMT_BF16, m, r16), neg);
}

/* ---- E4M3 (OCP FP8, "FN": no infinities, S.1111.111 is NaN) --------------- */
double oracle_e4m3_decode(uint8_t code)
{
    int s = (code >> 7) & 1, E = (code >> 3) & 0xF, M = code & 7;
    double v;
    if (E == 0xF && M == 7) v = NAN;
    else if (E == 0) v = ldexp((double)M / 8.0, -6);
    else v = ldexp(1.0 + (double)M / 8.0, E - 7);
    return s ? -v : v;
}

static uint8_t e4m3_encode_exact(double m, int neg)
{
    uint8_t code;
    if (m == 0.0) code = 0;
    else {
        int e; double fr = frexp(m, &e);
        int ex = e - 1;
        if (ex < -6) code = (uint8_t)(m / ldexp(1.0, -9));
        else code = (uint8_t)(((ex + 7) << 3) | (int)((fr * 2.0 - 1.0) * 8.0));
    }
    return (uint8_t)(code | (neg ? 0x80 : 0));
}

uint8_t oracle_e4m3_rne(double v)
{
    if (isnan(v)) return 0x7F;
    int neg = signbit(v) != 0;
    double m = fabs(v);
    if (isinf(m)) m = FMT_E4M3.maxv;
    return e4m3_encode_exact(round_rne(&FMT_E4M3, m), neg);
}

uint8_t oracle_e4m3_sr(float v, uint32_t r16)
{
    if (isnan(v)) return 0x7F;
    double d = (double)v;
    int neg = signbit(d) != 0;
    double m = fabs(d);
    if (isinf(m)) m = FMT_E4M3.maxv;
    return e4m3_encode_exact(round_sr(&FMT_E4M3, m, r16), neg);
}

/* ---- E2M1 (OCP MX FP4) ---------------------------------------------------- */
double oracle_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, E = (code >> 1) & 3, M = code & 1;
    double v = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
    return s ? -v : v;
}

static uint8_t e2m1_encode_exact(double m, int neg)
{
    /* magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 -> codes 0..7 */
    uint8_t code;
    if (m < 1.0) code = (uint8_t)(m * 2.0);          /* 0 or 0.5 */
    else {
        int e; double fr = frexp(m, &e);
        int ex = e - 1;                               /* 0, 1, 2 */
        code = (uint8_t)(((ex + 1) << 1) | (int)((fr * 2.0 - 1.0) * 2.0));
    }
    return (uint8_t)(code | (neg ? 8 : 0));
}

/*
 * Quantize n values (n a multiple of 32) to FP4 E2M1 with one E4M3 scale per
 * block of 32 consecutive values:
 *   scale s = RNE_E4M3(amax / 6)   (saturating at 448)
 *   code_i  = sign(v_i) | RNE_E2M1(|v_i| / s)   (saturating at 6; 0 if s == 0)
 * codes: n/2 bytes, element 2i in the low nibble of byte i, 2i+1 in the high.
 */
void oracle_fp4_quantize(const float *v, int64_t n, uint8_t *codes,
                         uint8_t *scales)
{
    for (int64_t blk = 0; blk < n / 32; ++blk) {
        const float *vb = v + blk * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) {
            double m = fabs((double)vb[i]);
            if (m > amax) amax = m;
        }
        uint8_t sc = oracle_e4m3_rne(amax / 6.0);
        scales[blk] = sc;
        double s = oracle_e4m3_decode(sc);
        for (int i = 0; i < 32; ++i) {
            double d = (double)vb[i];
            int neg = signbit(d) != 0;
            uint8_t c;
            if (s == 0.0) c = (uint8_t)(neg ? 8 : 0);
            else c = e2m1_encode_exact(round_rne(&FMT_E2M1, fabs(d) / s), neg);
            int64_t e = blk * 32 + i;
            if (e % 2 == 0) codes[e / 2] = c;
            else codes[e / 2] = (uint8_t)(codes[e / 2] | (c << 4));
        }
    }
}

void oracle_fp4_dequantize(const uint8_t *codes, const uint8_t *scales,
                           int64_t n, double *out)
{
    for (int64_t e = 0; e < n; ++e) {
        uint8_t byte = codes[e / 2];
        uint8_t c = (e % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        out[e] = oracle_e2m1_decode(c) * oracle_e4m3_decode(scales[e / 32]);
    }
}

/*
 * Update-checkpoint quantizer with stochastic rounding.  v holds n fp32
 * values whose global element indices are elem0 .. elem0+n-1 (element index
 * = ((slot*H + h)*P + p)*N + n within the layer).  fmt: 0 = bf16 (2 bytes per
 * value, little-endian), 1 = E4M3 (1 byte).
 */
void oracle_sr_quantize(const float *v, int64_t n, int fmt, uint64_t seed,
                        uint32_t layer, uint32_t interval, uint64_t elem0,
                        uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t r = oracle_sr_draw(seed, layer, interval, elem0 + (uint64_t)i);
        if (fmt == 0) {
            uint16_t c = oracle_bf16_sr(v[i], r);
            out[2 * i] = (uint8_t)(c & 0xFF);
            out[2 * i + 1] = (uint8_t)(c >> 8);
        } else {
            out[i] = oracle_e4m3_sr(v[i], r);
        }
    }
}
