// fft.hip -- prefill through the FFT: Hyena's own way of evaluating its long
// convolution (StripedHyena article, Hyena層次結構: the convolution with a
// filter as long as the input, evaluated by FFT in O(L log L)), here as the
// comparison point for the modal prefill.
//
// Per batch row b and channel c in head g, with u = k v:
//     y[t] = q[t] * sum_{s<=t} h_g[t-s] u[s],   t < L,
// computed as the first L samples of IFFT( FFT(u, N) * FFT(h_g, N) ) with
// N = the power of two >= 2L (zero padding makes the circular convolution the
// causal one).  Two channels of one head share one complex transform (u_c in
// the real part, u_{c+1} in the imaginary part): the filter is real and the
// same for both, so the real and imaginary parts of the result are the two
// convolutions, with no untangling.
//
// Kernels: filter taps (the materialise kernel) into the workspace; twiddles
// exp(-2 pi i k / N) in float64 rounded to float32; one forward transform per
// head (the filter spectra); then one workgroup per (batch row, group of NP
// channel pairs): u into LDS at bit-reversed positions, radix-2
// decimation-in-time passes (natural-order spectrum), multiply by the head's
// spectrum, decimation-in-frequency passes with conjugate twiddles (result at
// bit-reversed positions), gate with q and store.  The transforms run in LDS
// (N complex float32 per pair); HBM traffic equals the modal prefill's
// (q, k, v read once, y written once), the work is O(L log L) per channel.
// No end-of-prompt modal state comes out of this path.
#include "hm_internal.hpp"

namespace hm {
namespace {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 cmul_conj(float2 a, float2 w) {  // a * conj(w)
    return make_float2(a.x * w.x + a.y * w.y, a.y * w.x - a.x * w.y);
}
__device__ __forceinline__ unsigned bitrev(unsigned i, int logn) { return __brev(i) >> (32 - logn); }

// In-place radix-2 DIT over NP transforms of length N = 2^logn held back to
// back in x (input bit-reversed, output natural).  tw[k] = exp(-2 pi i k / N).
__device__ void fft_dit(float2 *x, const float2 *tw, int logn, int np) {
    const int N = 1 << logn;
    for (int s = 1; s <= logn; ++s) {
        const int half = 1 << (s - 1), stride = N >> s;
        for (int i = threadIdx.x; i < np * (N / 2); i += blockDim.x) {
            const int p = i / (N / 2), k = i % (N / 2);
            const int j = k & (half - 1), a = ((k >> (s - 1)) << s) + j;
            float2 *xp = x + p * N;
            const float2 t = cmul(tw[j * stride], xp[a + half]);
            const float2 u = xp[a];
            xp[a] = make_float2(u.x + t.x, u.y + t.y);
            xp[a + half] = make_float2(u.x - t.x, u.y - t.y);
        }
        __syncthreads();
    }
}

// In-place radix-2 DIF with conjugate twiddles (the inverse transform without
// its 1/N): input natural, output bit-reversed.
__device__ void ifft_dif(float2 *x, const float2 *tw, int logn, int np) {
    const int N = 1 << logn;
    for (int s = logn; s >= 1; --s) {
        const int half = 1 << (s - 1), stride = N >> s;
        for (int i = threadIdx.x; i < np * (N / 2); i += blockDim.x) {
            const int p = i / (N / 2), k = i % (N / 2);
            const int j = k & (half - 1), a = ((k >> (s - 1)) << s) + j;
            float2 *xp = x + p * N;
            const float2 u = xp[a], v = xp[a + half];
            xp[a] = make_float2(u.x + v.x, u.y + v.y);
            xp[a + half] = cmul_conj(make_float2(u.x - v.x, u.y - v.y), tw[j * stride]);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void fft_twiddle_kernel(float2 *tw, int logn) {
    const int N = 1 << logn;
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= N / 2) return;
    double s, c;
    sincospi(-2.0 * (double)k / (double)N, &s, &c);
    tw[k] = make_float2((float)c, (float)s);
}

// One workgroup per head: spectrum of the zero-padded taps.
__global__ __launch_bounds__(256) void fft_filter_spectrum_kernel(FftArgs a) {
    extern __shared__ float2 lds[];
    const int N = 1 << a.logn;
    float2 *tw = lds, *x = lds + N / 2;
    const int64_t g = blockIdx.x;
    for (int i = threadIdx.x; i < N / 2; i += blockDim.x) tw[i] = a.tw[i];
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const float v = i < a.L ? a.h[g * a.L + i] : 0.f;
        x[bitrev((unsigned)i, a.logn)] = make_float2(v, 0.f);
    }
    __syncthreads();
    fft_dit(x, tw, a.logn, 1);
    for (int i = threadIdx.x; i < N; i += blockDim.x) a.spec[g * N + i] = x[i];
}

template <int ACT>
__global__ __launch_bounds__(256) void fft_conv_kernel(FftArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    extern __shared__ float2 lds[];
    const int N = 1 << a.logn, np = a.np;
    float2 *tw = lds, *x = lds + N / 2;
    const int64_t b = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * 2 * np;  // first channel of the group (one head)
    const int64_t g = c0 / a.s.P;
    for (int i = threadIdx.x; i < N / 2; i += blockDim.x) tw[i] = a.tw[i];
    // u = k v of the 2 np channels: pair p -> real part channel c0+2p, imaginary c0+2p+1
    const T *kb = static_cast<const T *>(a.k) + b * a.L * a.ld_in + c0;
    const T *vb = static_cast<const T *>(a.v) + b * a.L * a.ld_in + c0;
    for (int i = threadIdx.x; i < np * N; i += blockDim.x) {
        const int p = i / N, t = i % N;
        float2 z = make_float2(0.f, 0.f);
        if (t < a.L) {
            const int64_t o = (int64_t)t * a.ld_in + 2 * p;
            z = make_float2(A::ld(kb + o) * A::ld(vb + o), A::ld(kb + o + 1) * A::ld(vb + o + 1));
        }
        x[p * N + bitrev((unsigned)t, a.logn)] = z;
    }
    __syncthreads();
    fft_dit(x, tw, a.logn, np);
    const float2 *hs = a.spec + g * N;
    for (int i = threadIdx.x; i < np * N; i += blockDim.x) x[i] = cmul(x[i], hs[i % N]);
    __syncthreads();
    ifft_dif(x, tw, a.logn, np);
    const float inv_n = 1.0f / (float)N;
    const T *qb = static_cast<const T *>(a.q) + b * a.L * a.ld_in + c0;
    T *yb = static_cast<T *>(a.y) + b * a.L * a.ld_y + c0;
    for (int i = threadIdx.x; i < np * a.L; i += blockDim.x) {
        const int p = i / a.L, t = i % a.L;
        const float2 r = x[p * N + bitrev((unsigned)t, a.logn)];
        const int64_t oi = (int64_t)t * a.ld_in + 2 * p, oy = (int64_t)t * a.ld_y + 2 * p;
        A::st(yb + oy, A::ld(qb + oi) * r.x * inv_n);
        A::st(yb + oy + 1, A::ld(qb + oi + 1) * r.y * inv_n);
    }
}

}  // namespace

int fft_log_n(int64_t L) {
    int logn = 1;
    while ((int64_t(1) << logn) < 2 * L) ++logn;
    return logn;
}

// One channel pair per workgroup: N/2 twiddles + N points of LDS (48 KB at
// N = 4096, 96 KB at N = 8192).
int fft_pairs_per_group(int64_t, int) { return 1; }

size_t fft_lds_bytes(int logn, int np) { return ((size_t)(1 << logn) / 2 + (size_t)np * (1 << logn)) * sizeof(float2); }

hipError_t launch_fft_prefill(const FftArgs &a, hipStream_t stream) {
    const int N = 1 << a.logn;
    fft_twiddle_kernel<<<dim3((unsigned)((N / 2 + 255) / 256)), dim3(256), 0, stream>>>(a.tw, a.logn);
    hipError_t e0 = hipFuncSetAttribute(reinterpret_cast<const void *>(&fft_filter_spectrum_kernel),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)fft_lds_bytes(a.logn, 1));
    if (e0 != hipSuccess) return e0;
    fft_filter_spectrum_kernel<<<dim3((unsigned)a.s.H), dim3(256), fft_lds_bytes(a.logn, 1), stream>>>(a);
    const dim3 grid((unsigned)(a.s.D / (2 * a.np)), (unsigned)a.s.B);
    const size_t lds = fft_lds_bytes(a.logn, a.np);
    hipError_t err;
    if (a.s.act == kBF16) {
        if ((err = hipFuncSetAttribute(reinterpret_cast<const void *>(&fft_conv_kernel<kBF16>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return err;
        fft_conv_kernel<kBF16><<<grid, dim3(256), lds, stream>>>(a);
    } else {
        if ((err = hipFuncSetAttribute(reinterpret_cast<const void *>(&fft_conv_kernel<kF32>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
            return err;
        fft_conv_kernel<kF32><<<grid, dim3(256), lds, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace hm
