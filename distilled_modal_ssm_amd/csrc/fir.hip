// fir.hip -- the non-distilled Hyena decode baseline: one generated token
// through the explicit long filter instead of the modal recurrence.
//
// Per (batch row b, channel c in head g) at step t, with u = k v kept in a
// cache in the activation dtype:
//     y_t = q_t * sum_{j=0}^{min(t, W-1)} h[g][j] u_{t-j},
// the causal long convolution of the Hyena operator (StripedHyena article,
// Hyena層次結構) evaluated directly: O(t) work and O(t) memory per token, the
// cost the distilled recurrence removes (Laughing Hyena Distillery review,
// 研究动机与目标 and 主要发现).  W = 0 uses every past step; W > 0 truncates the
// filter to its first W taps.
//
// Bound: HBM.  A step reads the cached rows [t-W+1, t) of every batch row
// (B * rows * D * s_act bytes) and writes one row; the filter taps are tiny.
// Pass 1 splits the rows into R ranges: workgroup (512-channel block, range,
// batch row), each lane 8 adjacent channels (16- or 32-byte loads), the 4
// waves striding over the range's rows, fp32 partial sums per range.  Pass 2
// sums the ranges, adds the current token's h[0] u_t, gates with q, writes y
// and appends u_t to the cache.
#include "hm_internal.hpp"

namespace hm {
namespace {

constexpr int kFirBlk = 512;  // channels per pass-1 workgroup (64 lanes x 8)

// 8 adjacent channels of one cache row.  NT: non-temporal loads, for windows
// larger than the 256 MB Infinity Cache (bf16 rows; measured on MI355X, B = 256,
// D = 2048: 140.7 -> 132.3 us per step; a window that fits the cache, B = 16,
// D = 2048, is re-read from it step after step and takes 27.1 -> 55.5 us with them).
template <int ACT, bool NT> struct Row8;
template <bool NT> struct Row8<kBF16, NT> {
    uint4 w;
    __device__ void load(const void *p) {
        if constexpr (NT) {
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            w = make_uint4(t.x, t.y, t.z, t.w);
        } else {
            w = *reinterpret_cast<const uint4 *>(p);
        }
    }
    __device__ void get(float *o) const {
        const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o[2 * e] = bf16_lo(v[e]);
            o[2 * e + 1] = bf16_hi(v[e]);
        }
    }
};
// float32: two 16-byte halves, adjacent (SPLIT = 4 floats) or half a block apart
// (SPLIT = 256, so that each load instruction of a wave covers whole lines and
// non-temporal loads stay efficient)
template <bool NT> struct Row8<kF32, NT> {
    float4 a, b;
    template <int SPLIT = 4> __device__ void load(const void *p) {
        const float *f = static_cast<const float *>(p);
        if constexpr (NT) {
            typedef float f32v4 __attribute__((ext_vector_type(4)));
            const f32v4 x = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(f));
            const f32v4 y = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(f + SPLIT));
            a = make_float4(x.x, x.y, x.z, x.w);
            b = make_float4(y.x, y.y, y.z, y.w);
        } else {
            a = *reinterpret_cast<const float4 *>(f);
            b = *reinterpret_cast<const float4 *>(f + SPLIT);
        }
    }
    __device__ void get(float *o) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// SPLIT: the lane's channels are c0 .. c0 + 3 and c0 + SPLIT .. + 3 (SPLIT = 4:
// eight adjacent channels; SPLIT = 256, float32 with D a multiple of the block:
// two halves half a block apart, possibly in different heads).
template <int ACT, bool NT, int SPLIT = 4>
__global__ __launch_bounds__(256) void fir_partial_kernel(FirArgs a) {
    using T = typename Act<ACT>::T;
    static_assert(SPLIT == 4 || (ACT == kF32 && SPLIT == kFirBlk / 2), "lane channel layout");
    __shared__ float red[4][kWave][8];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t c0 = (int64_t)blockIdx.x * kFirBlk + (SPLIT == 4 ? 8 : 4) * lane;
    const int r = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int64_t n = a.t - a.lo;                       // cached rows in the window
    const int64_t chunk = (n + a.R - 1) / a.R;
    const int64_t s_begin = a.lo + (int64_t)r * chunk;
    const int64_t s_end = (s_begin + chunk < a.t) ? s_begin + chunk : a.t;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (c0 < a.s.D) {
        const int64_t g = c0 / a.s.P, g2 = (c0 + SPLIT) / a.s.P;
        const float *hg = a.h + g * a.h_len + a.t;      // tap of row s: hg[-s] (channels e < 4)
        const float *hg2 = a.h + g2 * a.h_len + a.t;    // channels e >= 4
        const T *base = static_cast<const T *>(a.cache) + (b * a.cache_len) * a.s.D + c0;
        int64_t s = s_begin + w;
        // four rows per wave in flight
        for (; s + 12 < s_end; s += 16) {
            Row8<ACT, NT> x[4];
            float hv[4], hv2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (ACT == kF32)
                    x[i].template load<SPLIT>(base + (s + 4 * i) * a.s.D);
                else
                    x[i].load(base + (s + 4 * i) * a.s.D);
                hv[i] = hg[-(s + 4 * i)];
                hv2[i] = hg2[-(s + 4 * i)];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float u[8];
                x[i].get(u);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(e < 4 ? hv[i] : hv2[i], u[e], acc[e]);
            }
        }
        for (; s < s_end; s += 4) {
            Row8<ACT, NT> x;
            if constexpr (ACT == kF32)
                x.template load<SPLIT>(base + s * a.s.D);
            else
                x.load(base + s * a.s.D);
            const float hv = hg[-s], hv2 = hg2[-s];
            float u[8];
            x.get(u);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(e < 4 ? hv : hv2, u[e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w][lane][e] = acc[e];
    __syncthreads();
    if (w == 0 && c0 < a.s.D) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = red[0][lane][e] + red[1][lane][e] + red[2][lane][e] + red[3][lane][e];
        float *dst = a.part + ((int64_t)r * a.s.B + b) * a.s.D + c0;
        *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4 *>(dst + SPLIT) = make_float4(o[4], o[5], o[6], o[7]);
    }
}

template <int ACT>
__global__ __launch_bounds__(256) void fir_finish_kernel(FirArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.s.B * a.s.D) return;
    const int64_t b = i / a.s.D, c = i - b * a.s.D;
    const int64_t g = c / a.s.P;
    const float u = A::ld(static_cast<const T *>(a.k) + b * a.ld_in + c) *
                    A::ld(static_cast<const T *>(a.v) + b * a.ld_in + c);
    T *slot = static_cast<T *>(a.cache) + (b * a.cache_len + a.t) * a.s.D + c;
    A::st(slot, u);
    const float uq = A::ld(slot);  // u as the cache holds it (rounded to the activation dtype)
    float tot = a.h[g * a.h_len] * uq;
    for (int r = 0; r < a.R; ++r) tot += a.part[((int64_t)r * a.s.B + b) * a.s.D + c];
    A::st(static_cast<T *>(a.y) + b * a.ld_y + c, A::ld(static_cast<const T *>(a.q) + b * a.ld_in + c) * tot);
}

template <int ACT>
__global__ __launch_bounds__(256) void fir_fill_kernel(FirArgs a, int64_t L, int64_t total) {
    using A = Act<ACT>;
    using T = typename A::T;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t c = i % a.s.D, bt = i / a.s.D, t = bt % L, b = bt / L;
        const int64_t in = (b * L + t) * a.ld_in + c;
        const float u = A::ld(static_cast<const T *>(a.k) + in) * A::ld(static_cast<const T *>(a.v) + in);
        A::st(static_cast<T *>(a.cache) + (b * a.cache_len + t) * a.s.D + c, u);
    }
}

}  // namespace

int fir_ranges(int64_t B, int64_t D) {
    const int64_t blocks = B * ((D + kFirBlk - 1) / kFirBlk);
    // about one pass-1 workgroup per CU: fewer, longer row ranges stream faster
    // and leave fewer partial sums (measured on MI355X, full window: B = 16,
    // D = 2048 34.1 -> 27.1 us per step; B = 4, D = 4096, 64k steps 750 -> 699 us;
    // targets of 128 and 512 workgroups were slower)
    int64_t R = (256 + blocks - 1) / (blocks > 0 ? blocks : 1);
    if (R < 1) R = 1;
    if (R > 64) R = 64;
    return (int)R;
}

hipError_t launch_fir_decode(const FirArgs &a, hipStream_t stream) {
    const dim3 g1((unsigned)((a.s.D + kFirBlk - 1) / kFirBlk), (unsigned)a.R, (unsigned)a.s.B);
    const dim3 g2((unsigned)((a.s.B * a.s.D + 255) / 256));
    // non-temporal cache loads for windows larger than the 256 MB Infinity Cache,
    // unless the caller chose (a.loads)
    const int64_t window_bytes = a.s.B * (a.t - a.lo) * a.s.D * (a.s.act == kBF16 ? 2 : 4);
    const bool nt = a.loads == 0 ? window_bytes > (int64_t(256) << 20) : a.loads == 2;
    if (a.s.act == kBF16) {
        if (nt)
            fir_partial_kernel<kBF16, true><<<g1, dim3(256), 0, stream>>>(a);
        else
            fir_partial_kernel<kBF16, false><<<g1, dim3(256), 0, stream>>>(a);
        fir_finish_kernel<kBF16><<<g2, dim3(256), 0, stream>>>(a);
    } else {
        if (a.s.D % kFirBlk != 0) {
            if (nt) return hipErrorInvalidValue;  // the host rejects this case first
            fir_partial_kernel<kF32, false><<<g1, dim3(256), 0, stream>>>(a);
        } else if (nt) {
            fir_partial_kernel<kF32, true, kFirBlk / 2><<<g1, dim3(256), 0, stream>>>(a);
        } else {
            fir_partial_kernel<kF32, false, kFirBlk / 2><<<g1, dim3(256), 0, stream>>>(a);
        }
        fir_finish_kernel<kF32><<<g2, dim3(256), 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_fir_fill(const FirArgs &a, int64_t L, hipStream_t stream) {
    const int64_t total = a.s.B * L * a.s.D;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (a.s.act == kBF16)
        fir_fill_kernel<kBF16><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a, L, total);
    else
        fir_fill_kernel<kF32><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a, L, total);
    return hipGetLastError();
}

}  // namespace hm
