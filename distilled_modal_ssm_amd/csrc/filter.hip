// filter.hip -- materialise the first L taps of every head's modal filter.
//
//     h[g][0] = D_g,    h[g][t] = Re(sum_n R_gn lambda_gn^(t-1)),  1 <= t < L,
//
// the impulse response of a d-mode diagonal SSM (the distilled form of a long
// convolution filter, Laughing Hyena Distillery review, ABSTRACT; the
// distillation objective is stated on filters, same review, "提出的方法").
//
// Accuracy: a pole radius can be 0.9999 and t reaches 64k, so powers are never
// formed by a long float32 product.  Each thread owns a run of kRun consecutive
// taps of one head; per mode it evaluates lambda^(t0-1) once from the polar form
// in float64 (|lambda|^e = exp(e log|lambda|), angle e*arg(lambda)), then walks
// the run by float64 complex multiplication and accumulates in float64.  Every
// tap is rounded once to float32.
//
// Work is O(H L d) float64 FMAs (about 6 per tap and mode) and the output is
// H*L*4 bytes; the kernel is small next to prefill.
#include "hm_internal.hpp"

namespace hm {
namespace {

constexpr int kRun = 32;

__global__ __launch_bounds__(256) void filter_kernel(FilterArgs a) {
    const int64_t L = a.L, d = a.s.d;
    const int64_t runs = (L + kRun - 1) / kRun;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= a.s.H * runs) return;
    const int64_t g = tid / runs;
    const int64_t t0 = (tid - g * runs) * kRun;

    double acc[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) acc[j] = 0.0;

    // Tap t uses lambda^(t-1); the run starts at exponent e0 = t0 - 1 (t0 >= 1)
    // or covers t = 0 (the skip) and then exponents 0, 1, ... .
    const int64_t first = (t0 == 0) ? 1 : 0;  // index in the run of the first tap >= 1
    const double e0 = (t0 == 0) ? 0.0 : (double)(t0 - 1);
    for (int64_t n = 0; n < d; ++n) {
        const float2 lf = a.s.poles[g * d + n], rf = a.s.residues[g * d + n];
        const double lr = lf.x, li = lf.y, rr = rf.x, ri = rf.y;
        const double mag = (e0 == 0.0) ? 1.0 : exp(e0 * log(hypot(lr, li)));
        double s, c;
        sincos(e0 * atan2(li, lr), &s, &c);
        double pr = mag * c, pi = mag * s;
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            if (j >= first) {
                acc[j] = fma(rr, pr, fma(-ri, pi, acc[j]));
                const double nr = fma(lr, pr, -li * pi);
                const double ni = fma(lr, pi, li * pr);
                pr = nr;
                pi = ni;
            }
        }
    }
    float *out = a.h + g * L + t0;
    const int64_t cnt = (L - t0 < kRun) ? (L - t0) : kRun;
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
        if (j < cnt) out[j] = (t0 + j == 0) ? a.s.skip[g] : (float)acc[j];
    }
}

}  // namespace

hipError_t launch_filter(const FilterArgs &a, hipStream_t stream) {
    if (a.L == 0) return hipSuccess;
    const int64_t threads = a.s.H * ((a.L + kRun - 1) / kRun);
    filter_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace hm
