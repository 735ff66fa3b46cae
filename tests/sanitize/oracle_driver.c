/*
 * Runs the CPU oracle's exported functions on small inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: every element type, a
 * channel subset, a continued state, and the impulse response (an impulse in
 * u = k v through the recurrence gives back the closed-form filter).
 * Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_abi(void);
int oracle_threads(void);
int oracle_filter(int64_t H, int64_t d, const double *poles, const double *residues, const double *skip,
                  int64_t L, double *h);
int oracle_modal_scan(int64_t B, int64_t D, int64_t H, int64_t d, const double *poles, const double *residues,
                      const double *skip, int64_t T, int dtype, const void *q, const void *k, const void *v,
                      int64_t stride_b, int64_t stride_t, int64_t n_sel, const int64_t *sel, double *y,
                      double *state);

static unsigned long long rng = 88172645463325252ULL;
static double uniform(void) {  /* xorshift64 in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

int main(void) {
    enum { B = 2, D = 12, H = 3, d = 5, T = 40 };
    double poles[H * d * 2], res[H * d * 2], skip[H];
    for (int i = 0; i < H * d; ++i) {
        const double r = 0.5 + 0.45 * fabs(uniform()), th = 3.0 * fabs(uniform());
        poles[2 * i] = r * cos(th);
        poles[2 * i + 1] = r * sin(th);
        res[2 * i] = uniform();
        res[2 * i + 1] = uniform();
    }
    for (int g = 0; g < H; ++g) skip[g] = uniform();
    if (oracle_abi() != 1 || oracle_threads() < 1) return 1;

    double h[H * T];
    if (oracle_filter(H, d, poles, res, skip, T, h)) return 2;

    /* impulse: q = 1, k = v = 1 at t = 0 and 0 after, float64 inputs */
    double *q = calloc(B * T * D, sizeof(double)), *k = calloc(B * T * D, sizeof(double));
    double *y = malloc(sizeof(double) * B * T * D), *st = calloc(B * D * d * 2, sizeof(double));
    for (int i = 0; i < B * T * D; ++i) q[i] = 1.0;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < D; ++c) k[(b * T) * D + c] = 1.0;
    if (oracle_modal_scan(B, D, H, d, poles, res, skip, T, 2, q, k, k, T * D, D, D, NULL, y, st)) return 3;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int c = 0; c < D; ++c)
                if (fabs(y[(b * T + t) * D + c] - h[(c / (D / H)) * T + t]) > 1e-12) {
                    printf("impulse mismatch b=%d t=%d c=%d\n", b, t, c);
                    return 4;
                }

    /* float32 and bfloat16 inputs, a channel subset, then one more step from the state */
    float *qf = malloc(sizeof(float) * B * T * D), *kf = malloc(sizeof(float) * B * T * D);
    uint16_t *qb = malloc(2 * B * T * D), *kb = malloc(2 * B * T * D);
    for (int i = 0; i < B * T * D; ++i) {
        qf[i] = (float)uniform();
        kf[i] = (float)uniform();
        uint32_t w;
        memcpy(&w, &qf[i], 4);
        qb[i] = (uint16_t)(w >> 16);
        memcpy(&w, &kf[i], 4);
        kb[i] = (uint16_t)(w >> 16);
    }
    const int64_t sel[3] = {0, 5, D - 1};
    double ys[B * T * 3], ss[B * 3 * d * 2];
    memset(ss, 0, sizeof ss);
    if (oracle_modal_scan(B, D, H, d, poles, res, skip, T, 0, qf, kf, kf, T * D, D, 3, sel, ys, ss)) return 5;
    memset(ss, 0, sizeof ss);
    if (oracle_modal_scan(B, D, H, d, poles, res, skip, T, 1, qb, kb, kb, T * D, D, 3, sel, ys, ss)) return 6;
    if (oracle_modal_scan(B, D, H, d, poles, res, skip, 1, 1, qb, kb, kb, T * D, D, 3, sel, ys, ss)) return 7;
    /* rejected arguments */
    if (!oracle_modal_scan(B, D, 5, d, poles, res, skip, T, 0, qf, kf, kf, T * D, D, D, NULL, y, st)) return 8;
    if (!oracle_modal_scan(B, D, H, d, poles, res, skip, T, 9, qf, kf, kf, T * D, D, D, NULL, y, st)) return 9;
    if (!oracle_filter(H, d, poles, res, skip, 0, h)) return 10;
    free(q); free(k); free(y); free(st); free(qf); free(kf); free(qb); free(kb);
    printf("oracle ok\n");
    return 0;
}
