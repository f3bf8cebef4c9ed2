/* The fp64 oracle under AddressSanitizer / UndefinedBehaviorSanitizer: every
 * exported function on small odd shapes and on the special values of each
 * codec (signed zeros, subnormals, the largest finite values, infinities,
 * NaN), so any out-of-bounds access or undefined operation stops the run.
 * Built with gcc from oracle/oracle.c by tests/test_sanitizers.py. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_recurrent(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double *, const double *,
                      const double *, const double *, const double *, const double *, const double *, double *);
void oracle_spec_round(int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double *, const double *,
                       const double *, const double *, const double *, const double *, const double *,
                       const int32_t *, double *);
void oracle_philox4x32_10(const uint32_t[4], const uint32_t[2], uint32_t[4]);
uint32_t oracle_sr_draw(uint64_t, uint32_t, uint32_t, uint64_t);
double oracle_bf16_decode(uint16_t);
uint16_t oracle_bf16_sr(float, uint32_t);
double oracle_e4m3_decode(uint8_t);
uint8_t oracle_e4m3_rne(double);
uint8_t oracle_e4m3_sr(float, uint32_t);
double oracle_e2m1_decode(uint8_t);
void oracle_fp4_quantize(const float *, int64_t, uint8_t *, uint8_t *);
void oracle_fp4_dequantize(const uint8_t *, const uint8_t *, int64_t, double *);
void oracle_sr_quantize(const float *, int64_t, int, uint64_t, uint32_t, uint32_t, uint64_t, uint8_t *);
int oracle_num_threads(void);
void oracle_set_num_threads(int);

static double urand(uint64_t *s) {
    *s = *s * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(*s >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *fill(size_t n, uint64_t *s, double scale) {
    double *a = malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) a[i] = scale * urand(s);
    return a;
}

int main(void) {
    uint64_t seed = 12345;
    const int64_t B = 2, H = 4, G = 2, P = 3, N = 5, T = 7;
    double *S = fill(B * H * P * N, &seed, 0.1);
    double *x = fill(T * B * H * P, &seed, 1.0), *Bm = fill(T * B * G * N, &seed, 1.0);
    double *Cm = fill(T * B * G * N, &seed, 1.0), *dt = fill(T * B * H, &seed, 0.5);
    double *A = fill(H, &seed, 4.0), *D = fill(H, &seed, 1.0);
    for (int64_t i = 0; i < T * B * H; ++i) dt[i] = fabs(dt[i]);
    for (int64_t h = 0; h < H; ++h) A[h] = -fabs(A[h]) - 1.0;
    double *y = malloc(T * B * H * P * sizeof(double));
    for (int threads = 1; threads <= 3; threads += 2) {
        oracle_set_num_threads(threads);
        oracle_recurrent(B, H, P, N, G, T, S, x, Bm, Cm, dt, A, D, y);
        oracle_recurrent(B, H, P, N, G, T, S, x, Bm, Cm, dt, A, D, NULL);
        int32_t keep[2] = {0, 5};
        oracle_spec_round(B, H, P, N, G, 5, S, x, Bm, Cm, dt, A, D, keep, y);
        keep[0] = 5; keep[1] = 1;
        oracle_spec_round(B, H, P, N, G, 5, S, x, Bm, Cm, dt, A, D, keep, y);
    }
    double acc = 0.0;
    for (int64_t i = 0; i < T * B * H * P; ++i) acc += y[i];

    uint32_t ctr[4] = {0xFFFFFFFFu, 1, 2, 3}, key[2] = {0xFFFFFFFFu, 0xFFFFFFFFu}, out[4];
    oracle_philox4x32_10(ctr, key, out);
    uint32_t draws = 0;
    for (uint64_t e = 0; e < 64; ++e) draws ^= oracle_sr_draw(~0ull, 7, 0xFFFFFFFFu, 0xFFFFFFF8ull + e);

    const float specials[] = {0.0f, -0.0f, 1e-45f, -1e-45f, 1.1754942e-38f, 1.0f, -1.5f, 3.3895314e38f,
                              3.4028235e38f, -3.4028235e38f, INFINITY, -INFINITY, NAN, -NAN, 448.0f, 449.0f,
                              464.0f, -480.0f, 1e-3f, 0.0009765625f, 0.001953125f, 6.0f, 5.0f, 2.5f};
    const int ns = (int)(sizeof(specials) / sizeof(specials[0]));
    uint32_t codes = 0;
    for (int i = 0; i < ns; ++i)
        for (uint32_t r = 0; r < 65536; r += 4099) {
            codes += oracle_bf16_sr(specials[i], r);
            codes += oracle_e4m3_sr(specials[i], r);
        }
    for (int c = 0; c < 65536; ++c) acc += isnan(oracle_bf16_decode((uint16_t)c)) ? 0.0 : 1e-300;
    for (int c = 0; c < 256; ++c) {
        const double v = oracle_e4m3_decode((uint8_t)c);
        if (!isnan(v)) codes += oracle_e4m3_rne(fabs(v) * 1.0001);
    }
    for (int c = 0; c < 16; ++c) acc += oracle_e2m1_decode((uint8_t)c);
    codes += oracle_e4m3_rne(1e300) + oracle_e4m3_rne(0.0) + oracle_e4m3_rne(1e-300);

    enum { NV = 96 };
    float v[NV];
    for (int i = 0; i < NV; ++i) v[i] = i < ns ? specials[i] : (float)(urand(&seed) * 10.0);
    for (int i = 0; i < NV; ++i) if (isnan(v[i]) || isinf(v[i])) v[i] = 1.0f;   /* FP4 takes finite states */
    uint8_t q[NV / 2], sc[NV / 32], u[2 * NV];
    double deq[NV];
    oracle_fp4_quantize(v, NV, q, sc);
    oracle_fp4_dequantize(q, sc, NV, deq);
    oracle_sr_quantize(v, NV, 0, 99, 3, 5, 1000, u);
    oracle_sr_quantize(v, NV, 1, 99, 3, 5, 1000, u);
    printf("oracle sanitizer run: %d threads max, checksum %.6g %u %u %u\n", oracle_num_threads(), acc,
           (unsigned)out[0], (unsigned)draws, (unsigned)codes);
    free(S); free(x); free(Bm); free(Cm); free(dt); free(A); free(D); free(y);
    return 0;
}
