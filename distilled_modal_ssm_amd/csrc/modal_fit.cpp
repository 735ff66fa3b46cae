// modal_fit.cpp -- host-side initial fit of modal filters (distillation set-up).
//
// The distillation review (Laughing Hyena Distillery, 提出的方法) picks the state
// dimension from the spectrum of each filter's Hankel operator and reduces the
// filter by modal truncation with a Prony-like parametrisation.  This file
// gives the two host steps that need no GPU:
//
//   * Hankel singular values of a filter: the n x n Hankel matrix
//     Hk[i][j] = h[1 + i + j] is symmetric, so its singular values are the
//     absolute eigenvalues, found by cyclic Jacobi rotations.  The number
//     above a relative threshold is the (real) order of the filter's minimal
//     realisation; d complex modes give at most 2d.
//   * An initial modal fit by the matrix pencil method (Hua and Sarkar, "Matrix
//     pencil method for estimating parameters of exponentially damped/undamped
//     sinusoids in noise", IEEE Trans. ASSP 1990), a Prony-type method.  The
//     taps x_k = h[1 + k] of a sum of M exponentials span, in every window of
//     n consecutive taps, the M vectors (z^0 .. z^(n-1)).  With Y the Hankel
//     data matrix of such windows, the top-M right singular vectors V span the
//     same space; V without its last row (V1) and without its first row (V2)
//     satisfy V2 = V1 Psi with Psi similar to diag(z), so the poles are the
//     eigenvalues of Psi = V1^+ V2.  Real taps give conjugate pairs; each pair
//     is one mode lambda of h[t] = Re sum R lambda^(t-1) (the upper half-plane
//     member).  The residues then solve the linear least-squares problem of
//     the filter-discrepancy objective over all taps for those poles, and the
//     skip is h[0].
//
// All arithmetic is float64 on the host; inputs and outputs are float32.
#include "hyena_modal.h"

#include <algorithm>
#include <cmath>
#include <complex>
#include <thread>
#include <vector>

namespace {

using cd = std::complex<double>;

// Eigenvalues (and optionally eigenvectors, columns of V) of a symmetric n x n
// matrix A (row-major, destroyed) by cyclic Jacobi rotations.
void sym_eig(int n, std::vector<double> &A, std::vector<double> &w, std::vector<double> *V) {
    if (V) {
        V->assign((size_t)n * n, 0.0);
        for (int i = 0; i < n; ++i) (*V)[(size_t)i * n + i] = 1.0;
    }
    for (int sweep = 0; sweep < 60; ++sweep) {
        double off = 0.0, diag = 0.0;
        for (int i = 0; i < n; ++i) {
            diag += A[(size_t)i * n + i] * A[(size_t)i * n + i];
            for (int j = i + 1; j < n; ++j) off += A[(size_t)i * n + j] * A[(size_t)i * n + j];
        }
        if (off <= 1e-32 * diag || off == 0.0) break;
        for (int p = 0; p < n - 1; ++p)
            for (int q = p + 1; q < n; ++q) {
                const double apq = A[(size_t)p * n + q];
                if (apq == 0.0) continue;
                const double app = A[(size_t)p * n + p], aqq = A[(size_t)q * n + q];
                // rotation angle that zeroes A[p][q]: tan(2 phi) = 2 apq / (aqq - app)
                const double tau = (aqq - app) / (2.0 * apq);
                const double t = (tau >= 0 ? 1.0 : -1.0) / (std::fabs(tau) + std::sqrt(1.0 + tau * tau));
                const double c = 1.0 / std::sqrt(1.0 + t * t), s = t * c;
                for (int k = 0; k < n; ++k) {  // columns p, q
                    const double akp = A[(size_t)k * n + p], akq = A[(size_t)k * n + q];
                    A[(size_t)k * n + p] = c * akp - s * akq;
                    A[(size_t)k * n + q] = s * akp + c * akq;
                }
                for (int k = 0; k < n; ++k) {  // rows p, q
                    const double apk = A[(size_t)p * n + k], aqk = A[(size_t)q * n + k];
                    A[(size_t)p * n + k] = c * apk - s * aqk;
                    A[(size_t)q * n + k] = s * apk + c * aqk;
                }
                if (V)
                    for (int k = 0; k < n; ++k) {
                        const double vkp = (*V)[(size_t)k * n + p], vkq = (*V)[(size_t)k * n + q];
                        (*V)[(size_t)k * n + p] = c * vkp - s * vkq;
                        (*V)[(size_t)k * n + q] = s * vkp + c * vkq;
                    }
            }
    }
    w.resize(n);
    for (int i = 0; i < n; ++i) w[i] = A[(size_t)i * n + i];
}

// Eigenvalues of a general real n x n matrix (row-major): Householder reduction
// to upper Hessenberg form, then shifted QR iterations on the complex
// Hessenberg matrix (Wilkinson shift from the trailing 2 x 2 block, Givens
// rotations, deflation on negligible subdiagonal entries).
std::vector<cd> general_eigenvalues(int n, const std::vector<double> &A0) {
    std::vector<cd> H((size_t)n * n);
    for (size_t i = 0; i < H.size(); ++i) H[i] = A0[i];
    auto at = [&](int i, int j) -> cd & { return H[(size_t)i * n + j]; };
    // Hessenberg: zero column k below row k + 1 with a reflector
    for (int k = 0; k + 2 < n; ++k) {
        double alpha = 0.0;
        for (int i = k + 1; i < n; ++i) alpha += std::norm(at(i, k));
        alpha = std::sqrt(alpha);
        if (alpha == 0.0) continue;
        const cd x0 = at(k + 1, k);
        const cd ph = std::abs(x0) > 0 ? x0 / std::abs(x0) : cd(1.0, 0.0);
        std::vector<cd> v(n, 0.0);
        v[k + 1] = x0 + ph * alpha;
        for (int i = k + 2; i < n; ++i) v[i] = at(i, k);
        double vn = 0.0;
        for (int i = k + 1; i < n; ++i) vn += std::norm(v[i]);
        if (vn == 0.0) continue;
        // H <- (I - 2 v v^H / |v|^2) H (I - 2 v v^H / |v|^2)
        for (int j = 0; j < n; ++j) {
            cd s = 0.0;
            for (int i = k + 1; i < n; ++i) s += std::conj(v[i]) * at(i, j);
            s *= 2.0 / vn;
            for (int i = k + 1; i < n; ++i) at(i, j) -= v[i] * s;
        }
        for (int i = 0; i < n; ++i) {
            cd s = 0.0;
            for (int j = k + 1; j < n; ++j) s += at(i, j) * v[j];
            s *= 2.0 / vn;
            for (int j = k + 1; j < n; ++j) at(i, j) -= s * std::conj(v[j]);
        }
    }
    std::vector<cd> eig(n);
    int hi = n - 1, iter = 0;
    while (hi >= 0) {
        if (hi == 0) {
            eig[0] = at(0, 0);
            break;
        }
        int lo = hi;
        while (lo > 0) {
            const double scale = std::abs(at(lo - 1, lo - 1)) + std::abs(at(lo, lo));
            if (std::abs(at(lo, lo - 1)) <= 1e-15 * (scale > 0 ? scale : 1.0)) {
                at(lo, lo - 1) = 0.0;
                break;
            }
            --lo;
        }
        if (lo == hi) {
            eig[hi] = at(hi, hi);
            --hi;
            iter = 0;
            continue;
        }
        // Wilkinson shift: the eigenvalue of the trailing 2 x 2 block closer to H[hi][hi]
        const cd a = at(hi - 1, hi - 1), b = at(hi - 1, hi), c = at(hi, hi - 1), d = at(hi, hi);
        const cd tr = a + d, det = a * d - b * c;
        const cd disc = std::sqrt(tr * tr - 4.0 * det);
        const cd e1 = 0.5 * (tr + disc), e2 = 0.5 * (tr - disc);
        cd mu = std::abs(e1 - d) < std::abs(e2 - d) ? e1 : e2;
        if (++iter % 12 == 0) mu = d + std::abs(c) * cd(0.75, 0.5);  // exceptional shift
        if (iter > 3000) {  // no convergence: report the diagonal as it stands
            for (int i = lo; i <= hi; ++i) eig[i] = at(i, i);
            hi = lo - 1;
            iter = 0;
            continue;
        }
        // one QR step on rows/columns lo..hi: H - mu I = Q R, H <- R Q + mu I
        std::vector<cd> gc(hi - lo), gs(hi - lo);
        for (int i = lo; i <= hi; ++i) at(i, i) -= mu;
        for (int k = lo; k < hi; ++k) {
            const cd x = at(k, k), y = at(k + 1, k);
            const double r = std::sqrt(std::norm(x) + std::norm(y));
            const cd cc = r > 0 ? x / r : cd(1.0, 0.0), ss = r > 0 ? y / r : cd(0.0, 0.0);
            gc[k - lo] = cc;
            gs[k - lo] = ss;
            for (int j = k; j <= hi; ++j) {  // rows k, k+1: G^H applied from the left
                const cd t1 = at(k, j), t2 = at(k + 1, j);
                at(k, j) = std::conj(cc) * t1 + std::conj(ss) * t2;
                at(k + 1, j) = -ss * t1 + cc * t2;
            }
        }
        for (int k = lo; k < hi; ++k) {  // columns k, k+1: G applied from the right
            const cd cc = gc[k - lo], ss = gs[k - lo];
            for (int i = lo; i <= std::min(k + 2, hi); ++i) {
                const cd t1 = at(i, k), t2 = at(i, k + 1);
                at(i, k) = t1 * cc + t2 * ss;
                at(i, k + 1) = -t1 * std::conj(ss) + t2 * std::conj(cc);
            }
        }
        for (int i = lo; i <= hi; ++i) at(i, i) += mu;
    }
    return eig;
}

// Solve the symmetric positive definite system G x = r (n x n, row-major) by
// Cholesky, with a relative ridge added to the diagonal if needed.
bool spd_solve(int n, std::vector<double> G, std::vector<double> &x) {
    double dmax = 0.0;
    for (int i = 0; i < n; ++i) dmax = std::max(dmax, G[(size_t)i * n + i]);
    if (dmax <= 0.0) return false;
    for (int i = 0; i < n; ++i) G[(size_t)i * n + i] += 1e-13 * dmax;
    for (int j = 0; j < n; ++j) {
        double s = G[(size_t)j * n + j];
        for (int k = 0; k < j; ++k) s -= G[(size_t)j * n + k] * G[(size_t)j * n + k];
        if (s <= 0.0) return false;
        const double ljj = std::sqrt(s);
        G[(size_t)j * n + j] = ljj;
        for (int i = j + 1; i < n; ++i) {
            double t = G[(size_t)i * n + j];
            for (int k = 0; k < j; ++k) t -= G[(size_t)i * n + k] * G[(size_t)j * n + k];
            G[(size_t)i * n + j] = t / ljj;
        }
    }
    for (int i = 0; i < n; ++i) {  // L y = r
        double t = x[i];
        for (int k = 0; k < i; ++k) t -= G[(size_t)i * n + k] * x[k];
        x[i] = t / G[(size_t)i * n + i];
    }
    for (int i = n - 1; i >= 0; --i) {  // L^T x = y
        double t = x[i];
        for (int k = i + 1; k < n; ++k) t -= G[(size_t)k * n + i] * x[k];
        x[i] = t / G[(size_t)i * n + i];
    }
    return true;
}

// Pencil window length for M exponentials and N taps: two windows' worth of
// rows at least, capped so the work stays O(M^3).
void pencil_shape(int64_t N, int M, int &rows, int &cols) {
    cols = std::min<int64_t>(2 * M + 8, N / 2);      // window length n
    rows = (int)std::min<int64_t>(N - cols + 1, 2 * cols);
}

struct HeadFit {
    std::vector<cd> lam;  // fitted poles (d)
    std::vector<cd> res;  // residues (d)
};

// Residues of h[t] ~ Re sum_n R_n lambda_n^(t-1), t = 1..L-1, by least squares
// over (Re R_n, Im R_n): columns Re(lambda^(t-1)) and -Im(lambda^(t-1)).
void fit_residues(const float *h, int64_t L, HeadFit &f) {
    const int d = (int)f.lam.size(), m = 2 * d;
    std::vector<double> G((size_t)m * m, 0.0), r(m, 0.0), col(m);
    std::vector<cd> p(d, cd(1.0, 0.0));
    for (int64_t t = 1; t < L; ++t) {
        for (int n = 0; n < d; ++n) {
            col[2 * n] = p[n].real();
            col[2 * n + 1] = -p[n].imag();
            p[n] *= f.lam[n];
        }
        const double ht = h[t];
        for (int i = 0; i < m; ++i) {
            r[i] += col[i] * ht;
            for (int j = 0; j <= i; ++j) G[(size_t)i * m + j] += col[i] * col[j];
        }
    }
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < i; ++j) G[(size_t)j * m + i] = G[(size_t)i * m + j];
    // a real pole has no imaginary column: pin its Im R to zero
    for (int n = 0; n < d; ++n)
        if (G[(size_t)(2 * n + 1) * m + 2 * n + 1] <= 1e-300) {
            for (int j = 0; j < m; ++j) G[(size_t)(2 * n + 1) * m + j] = G[(size_t)j * m + 2 * n + 1] = 0.0;
            G[(size_t)(2 * n + 1) * m + 2 * n + 1] = 1.0;
            r[2 * n + 1] = 0.0;
        }
    std::vector<double> x = r;
    f.res.assign(d, cd(0.0, 0.0));
    if (!spd_solve(m, G, x)) return;
    for (int n = 0; n < d; ++n) f.res[n] = cd(x[2 * n], x[2 * n + 1]);
}

// Poles of one filter by the matrix pencil with M = 2d exponentials, then the
// d modes: one member of each conjugate pair (Im > 0), real poles as they are;
// if more than d remain, the d with the largest energy |R|^2 / (1 - |lambda|^2).
void fit_head(const float *h, int64_t L, int d, double r_max, HeadFit &out) {
    const int64_t N = L - 1;  // taps from t = 1
    const int M = 2 * d;
    int rows, n;
    pencil_shape(N, M, rows, n);
    // Gram matrix Y^T Y of the Hankel data matrix Y[i][j] = x[i + j]
    std::vector<double> Gm((size_t)n * n, 0.0);
    for (int i = 0; i < rows; ++i)
        for (int a = 0; a < n; ++a) {
            const double ya = h[1 + i + a];
            for (int b = 0; b <= a; ++b) Gm[(size_t)a * n + b] += ya * h[1 + i + b];
        }
    for (int a = 0; a < n; ++a)
        for (int b = 0; b < a; ++b) Gm[(size_t)b * n + a] = Gm[(size_t)a * n + b];
    std::vector<double> w, V;
    sym_eig(n, Gm, w, &V);
    std::vector<int> idx(n);
    for (int i = 0; i < n; ++i) idx[i] = i;
    std::sort(idx.begin(), idx.end(), [&](int a, int b) { return w[a] > w[b]; });
    const int Mk = std::min(M, n - 1);
    // V1 = rows 0..n-2, V2 = rows 1..n-1 of the top-Mk eigenvectors; Psi solves V1 Psi = V2
    std::vector<double> A((size_t)Mk * Mk, 0.0), Bm((size_t)Mk * Mk, 0.0);
    for (int i = 0; i < Mk; ++i)
        for (int j = 0; j < Mk; ++j) {
            double s1 = 0.0, s2 = 0.0;
            for (int k = 0; k + 1 < n; ++k) {
                const double v1i = V[(size_t)k * n + idx[i]];
                s1 += v1i * V[(size_t)k * n + idx[j]];
                s2 += v1i * V[(size_t)(k + 1) * n + idx[j]];
            }
            A[(size_t)i * Mk + j] = s1;
            Bm[(size_t)i * Mk + j] = s2;
        }
    std::vector<double> Psi((size_t)Mk * Mk);
    for (int j = 0; j < Mk; ++j) {
        std::vector<double> x(Mk);
        for (int i = 0; i < Mk; ++i) x[i] = Bm[(size_t)i * Mk + j];
        spd_solve(Mk, A, x);
        for (int i = 0; i < Mk; ++i) Psi[(size_t)i * Mk + j] = x[i];
    }
    const std::vector<cd> z = general_eigenvalues(Mk, Psi);
    std::vector<cd> cand;
    for (const cd &p : z) {
        const double tol = 1e-9 * std::max(1.0, std::abs(p));
        if (p.imag() > tol) cand.push_back(p);
        else if (std::fabs(p.imag()) <= tol) cand.push_back(cd(p.real(), 0.0));
    }
    for (cd &p : cand)  // keep the recurrence stable
        if (std::abs(p) > r_max) p *= r_max / std::abs(p);
    HeadFit f;
    f.lam = cand;
    fit_residues(h, L, f);
    if ((int)f.lam.size() > d) {
        std::vector<int> o(f.lam.size());
        for (size_t i = 0; i < o.size(); ++i) o[i] = (int)i;
        auto energy = [&](int i) {
            const double r2 = std::norm(f.res[i]), a = std::norm(f.lam[i]);
            return r2 / std::max(1e-12, 1.0 - a);
        };
        std::sort(o.begin(), o.end(), [&](int a, int b) { return energy(a) > energy(b); });
        HeadFit g;
        for (int i = 0; i < d; ++i) g.lam.push_back(f.lam[o[i]]);
        fit_residues(h, L, g);
        f = g;
    }
    // fewer than d modes found (a lower-order filter): pad with zero-residue poles
    while ((int)f.lam.size() < d) {
        f.lam.push_back(cd(0.0, 0.0));
        f.res.push_back(cd(0.0, 0.0));
    }
    out = f;
}

template <typename F> void for_heads(int64_t H, F &&fn) {
    const int nt = (int)std::max<int64_t>(1, std::min<int64_t>(H, std::max(1u, std::thread::hardware_concurrency())));
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t)
        pool.emplace_back([&, t]() {
            for (int64_t g = t; g < H; g += nt) fn(g);
        });
    for (auto &th : pool) th.join();
}

}  // namespace

extern "C" {

hm_status hyena_hankel_singular_values(const float *h, int64_t L, int64_t n, double *sv) {
    if (!h || !sv || n < 1 || L < 2 * n) return HM_ERR_INVALID_ARG;
    if (n > 4096) return HM_ERR_UNSUPPORTED;
    std::vector<double> Hk((size_t)n * n);
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j) Hk[(size_t)i * n + j] = h[1 + i + j];
    std::vector<double> w;
    sym_eig((int)n, Hk, w, nullptr);
    for (auto &x : w) x = std::fabs(x);
    std::sort(w.begin(), w.end(), [](double a, double b) { return a > b; });
    for (int64_t i = 0; i < n; ++i) sv[i] = w[i];
    return HM_OK;
}

hm_status hyena_modal_order(const float *h, int64_t H, int64_t L, int64_t n, double rel_tol, int64_t *order) {
    if (!h || !order || H < 1 || n < 1 || L < 2 * n || !(rel_tol > 0.0 && rel_tol < 1.0)) return HM_ERR_INVALID_ARG;
    if (n > 4096) return HM_ERR_UNSUPPORTED;
    std::vector<hm_status> st(H, HM_OK);
    for_heads(H, [&](int64_t g) {
        std::vector<double> sv(n);
        st[g] = hyena_hankel_singular_values(h + g * L, L, n, sv.data());
        int64_t r = 0;
        while (r < n && sv[r] > rel_tol * sv[0]) ++r;
        order[g] = sv[0] > 0 ? r : 0;
    });
    for (auto s : st)
        if (s != HM_OK) return s;
    return HM_OK;
}

hm_status hyena_modal_fit_init(const float *h, int64_t H, int64_t L, int64_t d, float r_max, float *poles,
                               float *residues, float *skip) {
    if (!h || !poles || !residues || !skip || H < 1 || d < 1 || !(r_max > 0.f && r_max < 1.f))
        return HM_ERR_INVALID_ARG;
    if (d > HM_MAX_MODES) return HM_ERR_UNSUPPORTED;
    int rows, n;
    pencil_shape(L - 1, (int)(2 * d), rows, n);
    if (L < 2 || n < 2 * d + 1 || rows < 1) return HM_ERR_INVALID_ARG;  // too few taps for 2d exponentials
    for_heads(H, [&](int64_t g) {
        HeadFit f;
        fit_head(h + g * L, L, (int)d, (double)r_max, f);
        for (int64_t m = 0; m < d; ++m) {
            poles[(g * d + m) * 2] = (float)f.lam[m].real();
            poles[(g * d + m) * 2 + 1] = (float)f.lam[m].imag();
            residues[(g * d + m) * 2] = (float)f.res[m].real();
            residues[(g * d + m) * 2 + 1] = (float)f.res[m].imag();
        }
        skip[g] = h[g * L];
    });
    return HM_OK;
}

}  // extern "C"
