// filter.hip -- materialise the first L taps of every head's modal filter.
//
//     h[g][0] = D_g,    h[g][t] = Re(sum_n R_gn lambda_gn^(t-1)),  1 <= t < L,
//
// the impulse response of a d-mode diagonal SSM (the distilled form of a long
// convolution filter, Laughing Hyena Distillery review, ABSTRACT; the
// distillation objective is stated on filters, same review, "提出的方法").
//
// Accuracy: a pole radius can be 0.9999 and t reaches 64k, so powers are never
// formed by a long float32 product.  One thread owns one mode of one run of
// kRun consecutive taps of a head: it forms lambda^(t0-1) for the run's first
// tap by binary powering in float64 (at most 2 log2(L) complex products,
// relative error ~1e-15), walks the run by float64 complex multiplication, and
// leaves Re(R lambda^(t-1)) per tap in LDS; the workgroup then sums the modes
// of each tap in float64 and rounds it once to float32.
//
// Mapping: a workgroup is one head and 256/DPAD runs, DPAD = d rounded up to a
// power of two (lanes n >= d idle), so H * L * DPAD / kRun threads carry the
// O(H L d) float64 work (about 6 FMAs per tap and mode plus the powering).
#include "hm_internal.hpp"

namespace hm {
namespace {

constexpr int kRun = 32;

template <int DPAD>
__global__ __launch_bounds__(256) void filter_kernel(FilterArgs a) {
    constexpr int RPB = 256 / DPAD;  // runs per workgroup
    constexpr int TPB = RPB * kRun;  // taps per workgroup
    constexpr int LP = kRun + 1;     // LDS row (one run and mode), padded
    __shared__ double part[RPB * DPAD * LP];
    const int64_t L = a.L, d = a.s.d;
    const int64_t tiles = (L + TPB - 1) / TPB;
    const int64_t g = blockIdx.x / tiles, tile = blockIdx.x - g * tiles;
    const int n = threadIdx.x % DPAD, rl = threadIdx.x / DPAD;
    const int64_t t0 = tile * TPB + (int64_t)rl * kRun;  // first tap of this thread's run

    double acc[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) acc[j] = 0.0;
    if (n < d && t0 < L) {
        const float2 lf = a.s.poles[g * d + n], rf = a.s.residues[g * d + n];
        const double lr = lf.x, li = lf.y, rr = rf.x, ri = rf.y;
        // tap t uses lambda^(t-1): the run starts at exponent t0 - 1, or at
        // tap 0 (the skip term, added below) followed by exponents 0, 1, ...
        double pr, pi;
        complex_pow(lr, li, (t0 == 0) ? 0 : t0 - 1, pr, pi);
        const int first = (t0 == 0) ? 1 : 0;
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            if (j >= first) {
                acc[j] = fma(rr, pr, -ri * pi);
                const double nr = fma(lr, pr, -li * pi);
                const double ni = fma(lr, pi, li * pr);
                pr = nr;
                pi = ni;
            }
        }
    }
    double *row = part + (rl * DPAD + n) * LP;
#pragma unroll
    for (int j = 0; j < kRun; ++j) row[j] = acc[j];
    __syncthreads();

    for (int tau = threadIdx.x; tau < TPB; tau += 256) {
        const int64_t t = tile * TPB + tau;
        if (t >= L) break;
        const int run = tau / kRun, j = tau % kRun;
        double sum = 0.0;
        for (int m = 0; m < d; ++m) sum += part[(run * DPAD + m) * LP + j];
        a.h[g * L + t] = (t == 0) ? a.s.skip[g] : (float)sum;
    }
}

template <int DPAD>
hipError_t launch_dpad(const FilterArgs &a, hipStream_t stream) {
    constexpr int TPB = (256 / DPAD) * kRun;
    const int64_t blocks = a.s.H * ((a.L + TPB - 1) / TPB);
    filter_kernel<DPAD><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_filter(const FilterArgs &a, hipStream_t stream) {
    if (a.L == 0) return hipSuccess;
    const int64_t d = a.s.d;
    if (d <= 1) return launch_dpad<1>(a, stream);
    if (d <= 2) return launch_dpad<2>(a, stream);
    if (d <= 4) return launch_dpad<4>(a, stream);
    if (d <= 8) return launch_dpad<8>(a, stream);
    if (d <= 16) return launch_dpad<16>(a, stream);
    if (d <= 32) return launch_dpad<32>(a, stream);
    return launch_dpad<64>(a, stream);
}

}  // namespace hm
