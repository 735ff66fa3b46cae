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
// channel pairs): u into LDS, Stockham passes (radix 16 in registers, then the
// remaining radix; natural order in and out), multiply by the head's spectrum,
// the inverse as conj(FFT(conj(.))), gate with q and store.  The transforms run
// in LDS (N complex float32 per pair); HBM traffic equals the modal prefill's
// (q, k, v read once, y written once), the work is O(L log L) per channel.
// No end-of-prompt modal state comes out of this path.
#include "hm_internal.hpp"

namespace hm {
namespace {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 conj2(float2 a) { return make_float2(a.x, -a.y); }

// LDS index with one pad entry per 16: the first Stockham pass writes with a
// stride of R = 16 entries, which the pad spreads over all banks.
__device__ __forceinline__ int pad(int i) { return i + (i >> 4); }
constexpr int padded(int n) { return n + (n >> 4); }

// cos / sin of 2 pi m / 16, m < 8
__device__ constexpr float kC16[8] = {1.0f, 0.92387953251128674f, 0.70710678118654752f, 0.38268343236508977f,
                                      0.0f, -0.38268343236508977f, -0.70710678118654752f, -0.92387953251128674f};
__device__ constexpr float kS16[8] = {0.0f, 0.38268343236508977f, 0.70710678118654752f, 0.92387953251128674f,
                                      1.0f, 0.92387953251128674f, 0.70710678118654752f, 0.38268343236508977f};

constexpr int rev_bits(int i, int bits) {
    int r = 0;
    for (int b = 0; b < bits; ++b) r |= ((i >> b) & 1) << (bits - 1 - b);
    return r;
}

// In-register DFT of R points (R in {2, 4, 8, 16}): X[k] = sum_r v[r] exp(-2 pi i r k / R),
// radix-2 decimation in time on the bit-reversed register order (all indices
// compile-time constants).
template <int R>
__device__ __forceinline__ void dft_regs(float2 (&v)[R]) {
    constexpr int LR = R == 2 ? 1 : R == 4 ? 2 : R == 8 ? 3 : 4;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int j = rev_bits(i, LR);
        if (i < j) {
            const float2 t = v[i];
            v[i] = v[j];
            v[j] = t;
        }
    }
#pragma unroll
    for (int len = 2; len <= R; len <<= 1)
#pragma unroll
        for (int i = 0; i < R; i += len)
#pragma unroll
            for (int k = 0; k < len / 2; ++k) {
                const int m = k * (16 / len);  // exp(-2 pi i k / len) = exp(-2 pi i m / 16)
                const float2 w = make_float2(kC16[m], -kS16[m]);
                const float2 t = cmul(w, v[i + k + len / 2]);
                const float2 a = v[i + k];
                v[i + k] = make_float2(a.x + t.x, a.y + t.y);
                v[i + k + len / 2] = make_float2(a.x - t.x, a.y - t.y);
            }
}

// exp(-2 pi i k / N) for k < N from the half table tw[0 .. N/2)
__device__ __forceinline__ float2 twiddle(const float2 *tw, int k, int half) {
    const float2 w = tw[k < half ? k : k - half];
    return k < half ? w : make_float2(-w.x, -w.y);
}

// One Stockham radix-R pass over N points (Ns = product of the radices
// already applied): butterfly j reads x[j + r N/R], twiddles by
// exp(-2 pi i (j mod Ns) r / (Ns R)), and writes x[(j / Ns) Ns R + j mod Ns +
// r Ns] -- natural order in and out, in place through registers (read all,
// barrier, write all).  256 threads.
template <int R, int N>
__device__ __forceinline__ void stockham_pass(float2 *x, const float2 *tw, int Ns) {
    constexpr int nb = N / R;
    constexpr int MI = nb > 256 ? (nb + 255) / 256 : 1;  // butterflies per thread
    const int tid = threadIdx.x;
    float2 v[MI][R];
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int j = tid + 256 * it;
        if (j < nb) {
            const int k = j & (Ns - 1), step = N / (Ns * R);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float2 a = x[pad(j + r * nb)];
                v[it][r] = r == 0 ? a : cmul(twiddle(tw, k * r * step, N / 2), a);
            }
            dft_regs<R>(v[it]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int j = tid + 256 * it;
        if (j < nb) {
            const int base = (j / Ns) * Ns * R + (j & (Ns - 1));
#pragma unroll
            for (int r = 0; r < R; ++r) x[pad(base + r * Ns)] = v[it][r];
        }
    }
    __syncthreads();
}

// Forward transform of N = 2^LOGN points in place (natural order).  Radix 16
// from N = 4096 up (256 butterflies per pass or more), radix 4 below, so every
// thread holds a butterfly; then one pass of the remaining radix.
template <int LOGN>
__device__ void fft_forward(float2 *x, const float2 *tw) {
    constexpr int N = 1 << LOGN;
    constexpr int LR = LOGN >= 12 ? 4 : 2;  // log2 of the main radix
    constexpr int MAIN = LOGN / LR, REST = LOGN % LR;
    int Ns = 1;
#pragma unroll
    for (int p = 0; p < MAIN; ++p, Ns <<= LR) stockham_pass<(1 << LR), N>(x, tw, Ns);
    if constexpr (REST == 3) stockham_pass<8, N>(x, tw, Ns);
    if constexpr (REST == 2) stockham_pass<4, N>(x, tw, Ns);
    if constexpr (REST == 1) stockham_pass<2, N>(x, tw, Ns);
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
template <int LOGN>
__global__ __launch_bounds__(256) void fft_filter_spectrum_kernel(FftArgs a) {
    extern __shared__ float2 lds[];
    constexpr int N = 1 << LOGN;
    float2 *tw = lds, *x = lds + N / 2;
    const int64_t g = blockIdx.x;
    for (int i = threadIdx.x; i < N / 2; i += blockDim.x) tw[i] = a.tw[i];
    for (int i = threadIdx.x; i < N; i += blockDim.x)
        x[pad(i)] = make_float2(i < a.L ? a.h[g * a.L + i] : 0.f, 0.f);
    __syncthreads();
    fft_forward<LOGN>(x, tw);
    for (int i = threadIdx.x; i < N; i += blockDim.x) a.spec[g * N + i] = x[pad(i)];
}

// Workgroup = (batch row, NP channel pairs of one head).
template <int ACT, int NP, int LOGN>
__global__ __launch_bounds__(256) void fft_conv_kernel(FftArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    extern __shared__ float2 lds[];
    constexpr int N = 1 << LOGN, NPD = padded(1 << LOGN);
    float2 *tw = lds, *xs = lds + N / 2;
    // Neighbouring channel groups share the cache lines of every row: give
    // each XCD (workgroups are dealt to the 8 XCDs round robin) a contiguous
    // range of groups so those lines are fetched into one L2.
    const int64_t nwg = (int64_t)gridDim.x * gridDim.y;
    int64_t id = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    if (nwg % 8 == 0) id = (id % 8) * (nwg / 8) + id / 8;
    const int64_t b = id / gridDim.x;
    const int64_t c0 = (id % gridDim.x) * 2 * NP;
    const int64_t g = c0 / a.s.P;
    for (int i = threadIdx.x; i < N / 2; i += blockDim.x) tw[i] = a.tw[i];
    // u = k v: pair p holds channel c0+2p (real part) and c0+2p+1 (imaginary part)
    const T *kb = static_cast<const T *>(a.k) + b * a.L * a.ld_in + c0;
    const T *vb = static_cast<const T *>(a.v) + b * a.L * a.ld_in + c0;
    for (int t = threadIdx.x; t < N; t += blockDim.x) {
        float uk[2 * NP];
        if (t < a.L) {
            const int64_t o = (int64_t)t * a.ld_in;
#pragma unroll
            for (int e = 0; e < 2 * NP; ++e) uk[e] = A::ld(kb + o + e) * A::ld(vb + o + e);
        } else {
#pragma unroll
            for (int e = 0; e < 2 * NP; ++e) uk[e] = 0.f;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) xs[p * NPD + pad(t)] = make_float2(uk[2 * p], uk[2 * p + 1]);
    }
    __syncthreads();
    const float2 *hs = a.spec + g * N;
    for (int p = 0; p < NP; ++p) {
        float2 *x = xs + p * NPD;
        fft_forward<LOGN>(x, tw);
        // inverse through the forward transform: conj(FFT(conj(X H)))
        for (int i = threadIdx.x; i < N; i += blockDim.x) x[pad(i)] = conj2(cmul(x[pad(i)], hs[i]));
        __syncthreads();
        fft_forward<LOGN>(x, tw);
    }
    const float inv_n = 1.0f / (float)N;
    const T *qb = static_cast<const T *>(a.q) + b * a.L * a.ld_in + c0;
    T *yb = static_cast<T *>(a.y) + b * a.L * a.ld_y + c0;
    for (int t = threadIdx.x; t < a.L; t += blockDim.x) {
        const int64_t oi = (int64_t)t * a.ld_in, oy = (int64_t)t * a.ld_y;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float2 r = xs[p * NPD + pad(t)];  // conj of the result: imaginary part negated
            A::st(yb + oy + 2 * p, A::ld(qb + oi + 2 * p) * r.x * inv_n);
            A::st(yb + oy + 2 * p + 1, -A::ld(qb + oi + 2 * p + 1) * r.y * inv_n);
        }
    }
}

// ------------------------------------------------------------ multi-pass transforms
//
// Past N = 8192 a transform no longer fits one workgroup's LDS, so it runs in
// three passes over HBM (the four-step factorisation).  With N = NA NB,
// t = ta + NA tb and k = kb + NB ka,
//     X[kb + NB ka] = sum_ta W_NA^(ta ka) W_N^(ta kb) sum_tb x[ta + NA tb] W_NB^(tb kb)
// (W_n = exp(-2 pi i / n)).  The work buffer z holds one complex value per
// (batch row, frequency or time index, channel pair) in rows of D/2 pairs, and
// a workgroup always takes kLongCB adjacent pairs of every row it touches, so
// HBM sees whole 128-byte row pieces while the transforms run down the
// columns of an LDS tile ([rows][kLongCB], all columns at once):
//   pass 1, per ta: u = k v (or the filter taps) at t = ta + NA tb < L, zero
//           beyond; length-NB transform over tb; times W_N^(ta kb); to z[kb][ta];
//   pass 2, per kb: length-NA transform over ta (X[kb + NB ka] by ka); for the
//           filter, stored as its spectrum [H][kb][ka]; for the convolution,
//           times the head's spectrum, conjugated, transformed again, times
//           W_N^(ta kb) -- the conjugate of the inverse's first half -- back to
//           z[kb][ta];
//   pass 3, per ta: length-NB transform over kb; y[ta + NA tb] is its
//           conjugate over N, gated by q, for t < L.
constexpr int kLongCB = 16;  // channel pairs (complex columns) per workgroup

// One Stockham radix-R pass over the NS rows of an LDS tile x[NS][kLongCB]
// (the same butterflies as stockham_pass, for every column).  256 threads.
template <int R, int NS>
__device__ __forceinline__ void tile_pass(float2 *x, const float2 *tw, int Ns) {
    constexpr int CB = kLongCB, nb = NS / R, items = nb * CB, MI = (items + 255) / 256;
    const int tid = threadIdx.x;
    float2 v[MI][R];
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int i = tid + 256 * it;
        if (i < items) {
            const int ch = i % CB, j = i / CB;
            const int k = j & (Ns - 1), step = NS / (Ns * R);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float2 a = x[(j + r * nb) * CB + ch];
                v[it][r] = r == 0 ? a : cmul(twiddle(tw, k * r * step, NS / 2), a);
            }
            dft_regs<R>(v[it]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int i = tid + 256 * it;
        if (i < items) {
            const int ch = i % CB, j = i / CB;
            const int base = (j / Ns) * Ns * R + (j & (Ns - 1));
#pragma unroll
            for (int r = 0; r < R; ++r) x[(base + r * Ns) * CB + ch] = v[it][r];
        }
    }
    __syncthreads();
}

// Forward transform of every column of the tile (2^LOGNS rows, natural order).
template <int LOGNS>
__device__ void tile_fft(float2 *x, const float2 *tw) {
    constexpr int NS = 1 << LOGNS, MAIN = LOGNS / 4, REST = LOGNS % 4;
    int Ns = 1;
#pragma unroll
    for (int p = 0; p < MAIN; ++p, Ns <<= 4) tile_pass<16, NS>(x, tw, Ns);
    if constexpr (REST == 3) tile_pass<8, NS>(x, tw, Ns);
    if constexpr (REST == 2) tile_pass<4, NS>(x, tw, Ns);
    if constexpr (REST == 1) tile_pass<2, NS>(x, tw, Ns);
}

// exp(-2 pi i m / NS) for m < NS/2, from the N-point table (stride N / NS)
template <int NS>
__device__ __forceinline__ void load_subtable(float2 *tws, const float2 *tw, int64_t stride) {
    for (int i = threadIdx.x; i < NS / 2; i += blockDim.x) tws[i] = tw[(int64_t)i * stride];
}

// Global <-> tile moves.  Every item of a workgroup's load is issued before
// the first LDS store, so a thread has all its loads in flight at once (a loop
// that stores each value as it arrives waits out one memory round trip per
// item).  Column pairs move as 16-byte pieces when the row length is even.

// Load columns p0 .. p0 + kLongCB - 1 of NR rows (row r at base + r rstride,
// in complex elements) into the tile; columns >= npairs read as 0.
template <int NR>
// Tiles of the long transforms stream through HBM once per pass (the arrays are
// far larger than the caches), so whole 16-byte column pairs are loaded and
// stored non-temporally (measured on MI355X, B = 4, D = 4096, N = 131072:
// 17.6 -> 15.7 ms for the prefill).
__device__ __forceinline__ void tile_load(float2 *xs, const float2 *base, int64_t rstride, int64_t p0,
                                          int64_t npairs) {
    constexpr int CB = kLongCB, IT = NR * CB / 512;
    static_assert(NR * CB % 512 == 0, "whole column pairs per thread");
    const int tid = threadIdx.x;
    float4 t[IT];
    if ((npairs & 1) == 0) {  // p0 is even: a pair of columns is 16 aligned bytes, both in range or out
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = tid + 256 * i, r = e / (CB / 2), c = 2 * (e % (CB / 2));
            typedef float f32v4 __attribute__((ext_vector_type(4)));
            f32v4 v = {0.f, 0.f, 0.f, 0.f};
            if (p0 + c < npairs) v = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(base + r * rstride + p0 + c));
            t[i] = make_float4(v.x, v.y, v.z, v.w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = tid + 256 * i, r = e / (CB / 2), c = 2 * (e % (CB / 2));
            const float2 lo = p0 + c < npairs ? base[r * rstride + p0 + c] : make_float2(0.f, 0.f);
            const float2 hi = p0 + c + 1 < npairs ? base[r * rstride + p0 + c + 1] : make_float2(0.f, 0.f);
            t[i] = make_float4(lo.x, lo.y, hi.x, hi.y);
        }
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = tid + 256 * i, r = e / (CB / 2), c = 2 * (e % (CB / 2));
        *reinterpret_cast<float4 *>(&xs[r * CB + c]) = t[i];
    }
}

// Store tile row r times W_N^(m r) (m = ta or kb, the fixed index of the
// workgroup) to row r of the global block (row r at base + r rstride).
template <int NR>
__device__ __forceinline__ void tile_store_twiddled(const float2 *xs, float2 *base, int64_t rstride, int64_t p0,
                                                    int64_t npairs, const float2 *tw, int m, int half) {
    constexpr int CB = kLongCB, IT = NR * CB / 512;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = tid + 256 * i, r = e / (CB / 2), c = 2 * (e % (CB / 2));
        const float2 w = twiddle(tw, m * r, half);
        const float2 lo = cmul(w, xs[r * CB + c]), hi = cmul(w, xs[r * CB + c + 1]);
        if ((npairs & 1) == 0) {
            typedef float f32v4 __attribute__((ext_vector_type(4)));
            if (p0 + c < npairs)
                __builtin_nontemporal_store(f32v4{lo.x, lo.y, hi.x, hi.y}, reinterpret_cast<f32v4 *>(base + r * rstride + p0 + c));
        } else {
            if (p0 + c < npairs) base[r * rstride + p0 + c] = lo;
            if (p0 + c + 1 < npairs) base[r * rstride + p0 + c + 1] = hi;
        }
    }
}

// Pass 1.  Workgroup = (block of kLongCB pairs, ta, batch row).  FILTER: the
// columns are heads, x = their taps (imaginary part 0); else pair p is
// channels 2p (real part) and 2p + 1 (imaginary part) of u = k v.
template <int ACT, bool FILTER, int LOGNA, int LOGNB>
__global__ __launch_bounds__(256) void fftl_pass1_kernel(FftArgs a, int64_t npairs) {
    using A = Act<ACT>;
    using T = typename A::T;
    constexpr int NA = 1 << LOGNA, NB = 1 << LOGNB, CB = kLongCB;
    constexpr int64_t N = (int64_t)NA * NB;
    __shared__ __attribute__((aligned(16))) float2 xs[NB * CB];
    __shared__ float2 tws[NB / 2];
    const int ta = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * CB, b = blockIdx.z;
    load_subtable<NB>(tws, a.tw, NA);
    if constexpr (FILTER) {
        constexpr int IT = NB * CB / 256;
        float hv[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = threadIdx.x + 256 * i, tb = e / CB, c = e % CB;
            const int64_t t = ta + (int64_t)NA * tb, g = p0 + c;
            hv[i] = (t < a.L && g < npairs) ? a.h[g * a.L + t] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = threadIdx.x + 256 * i;
            xs[(e / CB) * CB + e % CB] = make_float2(hv[i], 0.f);
        }
    } else {
        constexpr int IT = NB * 2 * CB / 256;  // one channel of one row per item
        const T *kb = static_cast<const T *>(a.k) + b * a.L * a.ld_in;
        const T *vb = static_cast<const T *>(a.v) + b * a.L * a.ld_in;
        float kv[IT], vv[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = threadIdx.x + 256 * i, tb = e / (2 * CB), c = e % (2 * CB);
            const int64_t t = ta + (int64_t)NA * tb, ch = 2 * p0 + c;
            const bool in = t < a.L && ch < a.s.D;
            const int64_t o = in ? t * a.ld_in + ch : 0;
            kv[i] = in ? A::ld(kb + o) : 0.f;
            vv[i] = in ? A::ld(vb + o) : 0.f;
        }
        float *xf = reinterpret_cast<float *>(xs);  // pair c / 2, real (c even) or imaginary part
#pragma unroll
        for (int i = 0; i < IT; ++i) xf[threadIdx.x + 256 * i] = kv[i] * vv[i];
    }
    __syncthreads();
    tile_fft<LOGNB>(xs, tws);
    // times W_N^(ta kb), to rows kb NA + ta of z
    tile_store_twiddled<NB>(xs, a.z + b * N * npairs + (int64_t)ta * npairs, (int64_t)NA * npairs, p0, npairs,
                            a.tw, ta, (int)(N / 2));
}

// Pass 2.  Workgroup = (block of kLongCB pairs, kb, batch row).  FILTER: store
// the spectra; else the spectrum product and the first half of the inverse,
// in place.
template <bool FILTER, int LOGNA, int LOGNB>
__global__ __launch_bounds__(256) void fftl_pass2_kernel(FftArgs a, int64_t npairs) {
    constexpr int NA = 1 << LOGNA, NB = 1 << LOGNB, CB = kLongCB;
    constexpr int64_t N = (int64_t)NA * NB;
    __shared__ __attribute__((aligned(16))) float2 xs[NA * CB];
    __shared__ float2 tws[NA / 2];
    const int kb = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * CB, b = blockIdx.z;
    load_subtable<NA>(tws, a.tw, NB);
    float2 *zr = a.z + (b * N + (int64_t)kb * NA) * npairs;  // row ta at zr + ta npairs
    tile_load<NA>(xs, zr, npairs, p0, npairs);
    __syncthreads();
    tile_fft<LOGNA>(xs, tws);
    if constexpr (FILTER) {
        for (int e = threadIdx.x; e < NA * CB; e += 256) {
            const int ka = e / CB, c = e % CB;
            const int64_t g = p0 + c;
            if (g < npairs) a.spec[(g * NB + kb) * NA + ka] = xs[ka * CB + c];
        }
        return;
    } else {
        constexpr int IT = NA * CB / 256;
        float2 hs[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = threadIdx.x + 256 * i, ka = e / CB, c = e % CB;
            const int64_t p = p0 + c;
            const int64_t g = (p < npairs ? 2 * p : 0) / a.s.P;  // both channels of a pair are in one head
            hs[i] = a.spec[(g * NB + kb) * NA + ka];
        }
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int e = threadIdx.x + 256 * i;
            xs[e] = conj2(cmul(xs[e], hs[i]));
        }
        __syncthreads();
        tile_fft<LOGNA>(xs, tws);
        tile_store_twiddled<NA>(xs, zr, npairs, p0, npairs, a.tw, kb, (int)(N / 2));
    }
}

// Pass 3.  Workgroup = (block of kLongCB pairs, ta, batch row): the second
// half of the inverse, gate and store the steps t = ta + NA tb < L.
template <int ACT, int LOGNA, int LOGNB>
__global__ __launch_bounds__(256) void fftl_pass3_kernel(FftArgs a, int64_t npairs) {
    using A = Act<ACT>;
    using T = typename A::T;
    constexpr int NA = 1 << LOGNA, NB = 1 << LOGNB, CB = kLongCB;
    constexpr int64_t N = (int64_t)NA * NB;
    __shared__ __attribute__((aligned(16))) float2 xs[NB * CB];
    __shared__ float2 tws[NB / 2];
    const int ta = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * CB, b = blockIdx.z;
    load_subtable<NB>(tws, a.tw, NA);
    tile_load<NB>(xs, a.z + b * N * npairs + (int64_t)ta * npairs, (int64_t)NA * npairs, p0, npairs);
    __syncthreads();
    tile_fft<LOGNB>(xs, tws);
    const float inv_n = 1.0f / (float)N;
    const T *qb = static_cast<const T *>(a.q) + b * a.L * a.ld_in;
    T *yb = static_cast<T *>(a.y) + b * a.L * a.ld_y;
    constexpr int IT = NB * 2 * CB / 256;  // one channel of one row per item
    float qv[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = threadIdx.x + 256 * i, tb = e / (2 * CB), c = e % (2 * CB);
        const int64_t t = ta + (int64_t)NA * tb, ch = 2 * p0 + c;
        qv[i] = (t < a.L && ch < a.s.D) ? A::ld(qb + t * a.ld_in + ch) : 0.f;
    }
    const float *xf = reinterpret_cast<const float *>(xs);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int e = threadIdx.x + 256 * i, tb = e / (2 * CB), c = e % (2 * CB);
        const int64_t t = ta + (int64_t)NA * tb, ch = 2 * p0 + c;
        if (t >= a.L || ch >= a.s.D) continue;
        const float r = xf[e];  // pair c / 2: real part (c even) or imaginary part, conjugated
        A::st(yb + t * a.ld_y + ch, qv[i] * ((c & 1) ? -r : r) * inv_n);
    }
}

template <int LOGNA, int LOGNB>
hipError_t launch_long(const FftArgs &a, hipStream_t stream) {
    constexpr int NA = 1 << LOGNA, NB = 1 << LOGNB, CB = kLongCB;
    const dim3 block(256);
    // filter spectra: one "batch row" whose columns are the heads
    const int64_t H = a.s.H, np = a.s.D / 2;
    // x = pair block (fastest): workgroups that run together read neighbouring pieces of the same rows
    const dim3 gf1((unsigned)((H + CB - 1) / CB), NA, 1), gf2((unsigned)((H + CB - 1) / CB), NB, 1);
    fftl_pass1_kernel<kF32, true, LOGNA, LOGNB><<<gf1, block, 0, stream>>>(a, H);
    fftl_pass2_kernel<true, LOGNA, LOGNB><<<gf2, block, 0, stream>>>(a, H);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 g1((unsigned)((np + CB - 1) / CB), NA, (unsigned)a.s.B), g2(g1.x, NB, g1.z);
    if (a.s.act == kBF16) {
        fftl_pass1_kernel<kBF16, false, LOGNA, LOGNB><<<g1, block, 0, stream>>>(a, np);
        fftl_pass2_kernel<false, LOGNA, LOGNB><<<g2, block, 0, stream>>>(a, np);
        fftl_pass3_kernel<kBF16, LOGNA, LOGNB><<<g1, block, 0, stream>>>(a, np);
    } else {
        fftl_pass1_kernel<kF32, false, LOGNA, LOGNB><<<g1, block, 0, stream>>>(a, np);
        fftl_pass2_kernel<false, LOGNA, LOGNB><<<g2, block, 0, stream>>>(a, np);
        fftl_pass3_kernel<kF32, LOGNA, LOGNB><<<g1, block, 0, stream>>>(a, np);
    }
    return hipGetLastError();
}

}  // namespace

int fft_log_n(int64_t L) {
    int logn = 1;
    while ((int64_t(1) << logn) < 2 * L) ++logn;
    return logn;
}

// Channel pairs per workgroup: measured on MI355X (bf16, D = 2048), four pairs
// win at N = 1024 (2.5 vs 3.0 ms for B = 256, L = 512) and one pair at
// N = 4096 (0.95 vs 1.43 ms for B = 16, L = 2048), where four fill the LDS.
int fft_pairs_per_group(int64_t P, int logn) {
    int np = (logn <= 10) ? 4 : 1;
    while (np > 1 && P % (2 * np) != 0) np >>= 1;
    return np;
}

size_t fft_lds_bytes(int logn, int np) {
    const size_t N = size_t(1) << logn;
    return (N / 2 + (size_t)np * (N + (N >> 4))) * sizeof(float2);
}

template <int ACT, int NP, int LOGN>
static hipError_t launch_conv(const FftArgs &a, hipStream_t stream) {
    const size_t lds = fft_lds_bytes(LOGN, NP);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&fft_conv_kernel<ACT, NP, LOGN>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const dim3 grid((unsigned)(a.s.D / (2 * NP)), (unsigned)a.s.B);
    fft_conv_kernel<ACT, NP, LOGN><<<grid, dim3(256), lds, stream>>>(a);
    return hipGetLastError();
}

template <int LOGN>
static hipError_t launch_logn(const FftArgs &a, hipStream_t stream) {
    const size_t lds1 = fft_lds_bytes(LOGN, 1);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&fft_filter_spectrum_kernel<LOGN>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
    if (err != hipSuccess) return err;
    fft_filter_spectrum_kernel<LOGN><<<dim3((unsigned)a.s.H), dim3(256), lds1, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const bool bf = a.s.act == kBF16;
    switch (a.np) {
        case 4: return bf ? launch_conv<kBF16, 4, LOGN>(a, stream) : launch_conv<kF32, 4, LOGN>(a, stream);
        case 2: return bf ? launch_conv<kBF16, 2, LOGN>(a, stream) : launch_conv<kF32, 2, LOGN>(a, stream);
        default: return bf ? launch_conv<kBF16, 1, LOGN>(a, stream) : launch_conv<kF32, 1, LOGN>(a, stream);
    }
}

hipError_t launch_fft_prefill(const FftArgs &a, hipStream_t stream) {
    const int N = 1 << a.logn;
    fft_twiddle_kernel<<<dim3((unsigned)((N / 2 + 255) / 256)), dim3(256), 0, stream>>>(a.tw, a.logn);
    switch (a.logn) {
        case 1: return launch_logn<1>(a, stream);
        case 2: return launch_logn<2>(a, stream);
        case 3: return launch_logn<3>(a, stream);
        case 4: return launch_logn<4>(a, stream);
        case 5: return launch_logn<5>(a, stream);
        case 6: return launch_logn<6>(a, stream);
        case 7: return launch_logn<7>(a, stream);
        case 8: return launch_logn<8>(a, stream);
        case 9: return launch_logn<9>(a, stream);
        case 10: return launch_logn<10>(a, stream);
        case 11: return launch_logn<11>(a, stream);
        case 12: return launch_logn<12>(a, stream);
        case 13: return launch_logn<13>(a, stream);
        case 14: return launch_long<7, 7>(a, stream);
        case 15: return launch_long<8, 7>(a, stream);
        case 16: return launch_long<8, 8>(a, stream);
        case 17: return launch_long<9, 8>(a, stream);
        case 18: return launch_long<9, 9>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace hm
