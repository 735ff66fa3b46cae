/*
 * modal_oracle.c -- plain float64 CPU oracle of the modal-SSM Hyena operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg do.  It shares no code with the GPU
 * library.
 *
 * What it computes (order-2 Hyena operator with a distilled modal filter):
 *
 *   Hyena is a recursion of long convolutions and element-wise gates, and its
 *   order-2 form is y = q * (h conv (k * v)) with a causal long filter h
 *   (StripedHyena article, sections "Hyena塊" and "Hyena層次結構", which also
 *   give the matrix form y = diag(q) T_h diag(k) v with T_h causal Toeplitz).
 *
 *   Laughing Hyena replaces each per-head, weight-tied long filter by a
 *   low-dimensional linear state-space model (Laughing Hyena Distillery review,
 *   ABSTRACT and "提出的方法"), which generates in O(d) memory and O(dK) time
 *   for K tokens ("主要发现").  Taken in diagonal (modal) form with d complex
 *   poles lambda_n, residues R_n and a skip D_h, the SSM
 *       x_n <- lambda_n x_n + u,   output Re(sum_n R_n x_n) + D_h u
 *   read before the update has impulse response
 *       h[0] = D_h,   h[t] = Re(sum_n R_n lambda_n^(t-1))   (t >= 1).
 *
 * Functions:
 *   oracle_filter      h[g][t] for t < L, from the closed form (powers by
 *                      repeated float64 complex multiplication).
 *   oracle_modal_scan  the recurrence over T steps for every (batch, channel):
 *                        u = k v;  z = D_h u + Re(sum_n R_n x_n);  y = q z;
 *                        then x_n <- lambda_n x_n + u.
 *                      With a zero initial state and T = L this is prefill;
 *                      its final state is x_n = sum_t lambda_n^(L-1-t) u_t.
 *                      Called with the prefill state and T = 1 per generated
 *                      token it is one decode step.
 *
 * Channel c belongs to head c / (D / H) (contiguous blocks).  Everything is
 * IEEE float64 with round-to-nearest; build without -ffast-math and without
 * floating-point contraction.  Inputs are float32, bfloat16 bit patterns or
 * float64; all widen exactly to float64.
 *
 * Parity pins: brute-force direct convolution with the closed-form filter, the
 * d = 1 geometric series, Horner evaluation of the final state, FFT
 * convolution, impulse response, composition, linearity, shift invariance and
 * the stability bound (the oracle tests).
 */

#include <complex.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2
#define ORACLE_MAX_MODES 256

typedef double complex cplx;

static double act_load(const void *base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[idx];
    if (dtype == ORACLE_F64)
        return ((const double *)base)[idx];
    /* bfloat16 is the high half of an IEEE binary32 pattern */
    uint32_t w = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static cplx table_at(const double *tab, int64_t i)
{
    return CMPLX(tab[2 * i], tab[2 * i + 1]);
}

int oracle_abi(void) { return 1; }

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* h[g*L + t], t < L.  poles/residues: [H][d][2] (re, im); skip: [H]. */
int oracle_filter(int64_t H, int64_t d, const double *poles, const double *residues,
                  const double *skip, int64_t L, double *h)
{
    if (H <= 0 || d <= 0 || L <= 0)
        return 1;
    for (int64_t g = 0; g < H; ++g) {
        double *hg = h + g * L;
        hg[0] = skip[g];
        for (int64_t t = 1; t < L; ++t)
            hg[t] = 0.0;
        for (int64_t n = 0; n < d; ++n) {
            cplx lam = table_at(poles, g * d + n);
            cplx R = table_at(residues, g * d + n);
            cplx p = 1.0; /* lambda^(t-1) at t = 1 */
            for (int64_t t = 1; t < L; ++t) {
                hg[t] += creal(R * p);
                p *= lam;
            }
        }
    }
    return 0;
}

/*
 * Recurrence over T steps.
 *   Activation element (b, t, c) sits at index b*stride_b + t*stride_t + c.
 *   sel: n_sel channel indices (NULL: n_sel must equal D, channels 0..D-1).
 *   y:     [B][T][n_sel] float64 out.
 *   state: [B][n_sel][d][2] float64, in (initial state) and out (final state).
 */
int oracle_modal_scan(int64_t B, int64_t D, int64_t H, int64_t d,
                      const double *poles, const double *residues, const double *skip,
                      int64_t T, int dtype, const void *q, const void *k, const void *v,
                      int64_t stride_b, int64_t stride_t, int64_t n_sel, const int64_t *sel,
                      double *y, double *state)
{
    if (B <= 0 || D <= 0 || H <= 0 || d <= 0 || T < 0 || D % H != 0)
        return 1;
    if (d > ORACLE_MAX_MODES || (sel == NULL && n_sel != D))
        return 1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64)
        return 1;
    const int64_t P = D / H;

#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t i = 0; i < n_sel; ++i) {
            const int64_t c = sel ? sel[i] : i;
            const int64_t g = c / P;
            const double Dg = skip[g];
            cplx x[ORACLE_MAX_MODES];
            cplx lam[ORACLE_MAX_MODES];
            cplx R[ORACLE_MAX_MODES];
            double *st = state + (b * n_sel + i) * d * 2;
            for (int64_t n = 0; n < d; ++n) {
                x[n] = CMPLX(st[2 * n], st[2 * n + 1]);
                lam[n] = table_at(poles, g * d + n);
                R[n] = table_at(residues, g * d + n);
            }
            for (int64_t t = 0; t < T; ++t) {
                const int64_t a = b * stride_b + t * stride_t + c;
                const double u = act_load(k, dtype, a) * act_load(v, dtype, a);
                double z = Dg * u;
                for (int64_t n = 0; n < d; ++n)
                    z += creal(R[n] * x[n]);
                y[(b * T + t) * n_sel + i] = act_load(q, dtype, a) * z;
                for (int64_t n = 0; n < d; ++n)
                    x[n] = lam[n] * x[n] + u;
            }
            for (int64_t n = 0; n < d; ++n) {
                st[2 * n] = creal(x[n]);
                st[2 * n + 1] = cimag(x[n]);
            }
        }
    }
    return 0;
}
