// decode.hip -- one generation step of the modal Hyena operator on gfx950.
//
// Per (batch row b, channel c in head g), with u = k v:
//     y = q (D_g u + Re(sum_n R_gn x_n)),    then  x_n <- lambda_gn x_n + u,
// the O(d)-per-token recurrence that replaces the long convolution at
// generation time (Laughing Hyena Distillery review, "主要发现").  The output
// reads the state before the update: with that order the recurrence continues
// the causal convolution with h[0] = D_g, h[t] = Re(sum_n R_gn lambda_gn^(t-1)).
//
// The step is a pure stream over the state (16 d bytes per channel read and
// written) plus four activations, so it is bound by HBM bandwidth.  Layout and
// mapping:
//   - a thread owns CPT adjacent channels (2 when aligned) of one batch row and
//     all their modes in registers;
//   - the state is [B][H][d][P] complex float32, so for a fixed mode the
//     threads of a wave touch consecutive 16-byte pairs: every state access of a
//     wave is one contiguous 1 KiB segment;
//   - when a wave stays inside one head (P a multiple of 64*CPT) the head
//     index is made wave-uniform, and the pole/residue tables are fetched with
//     scalar loads into SGPRs, once per wave.
#include "hm_internal.hpp"

namespace hm {
namespace {

template <int DP, int ACT, int CPT, bool UNIFORM>
__global__ __launch_bounds__(256) void decode_step_fixed(DecodeArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    const int64_t D = a.s.D, P = a.s.P, H = a.s.H;
    const int64_t per_row = D / CPT;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= a.s.B * per_row) return;
    const int64_t b = tid / per_row;
    const int64_t c = (tid - b * per_row) * CPT;
    int g = (int)(c / P);
    if (UNIFORM) g = __builtin_amdgcn_readfirstlane(g);
    const int64_t p = c - (int64_t)g * P;

    const T *qp = static_cast<const T *>(a.q) + b * a.ld_in + c;
    const T *kp = static_cast<const T *>(a.k) + b * a.ld_in + c;
    const T *vp = static_cast<const T *>(a.v) + b * a.ld_in + c;
    T *yp = static_cast<T *>(a.y) + b * a.ld_y + c;
    const float2 *lam = a.s.poles + (int64_t)g * DP;
    const float2 *res = a.s.residues + (int64_t)g * DP;
    float2 *st = a.state + ((b * H + g) * DP) * P + p;

    float u[CPT], qv[CPT], acc[CPT];
    if constexpr (CPT == 2) {
        const float2 k2 = A::ld2(kp), v2 = A::ld2(vp), q2 = A::ld2(qp);
        u[0] = k2.x * v2.x;
        u[1] = k2.y * v2.y;
        qv[0] = q2.x;
        qv[1] = q2.y;
    } else {
        u[0] = A::ld(kp) * A::ld(vp);
        qv[0] = A::ld(qp);
    }

    // All state loads first: DP independent 8*CPT-byte loads in flight per thread.
    float2 x[DP][CPT];
#pragma unroll
    for (int n = 0; n < DP; ++n) {
        if constexpr (CPT == 2) {
            const float4 t = *reinterpret_cast<const float4 *>(st + n * P);
            x[n][0] = make_float2(t.x, t.y);
            x[n][1] = make_float2(t.z, t.w);
        } else {
            x[n][0] = st[n * P];
        }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
#pragma unroll
    for (int n = 0; n < DP; ++n) {
        const float2 l = lam[n], r = res[n];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const float2 xo = x[n][j];
            acc[j] = fmaf(r.x, xo.x, acc[j]);
            acc[j] = fmaf(-r.y, xo.y, acc[j]);
            x[n][j] = make_float2(fmaf(l.x, xo.x, fmaf(-l.y, xo.y, u[j])),
                                  fmaf(l.x, xo.y, l.y * xo.x));
        }
    }
#pragma unroll
    for (int n = 0; n < DP; ++n) {
        if constexpr (CPT == 2) {
            *reinterpret_cast<float4 *>(st + n * P) =
                make_float4(x[n][0].x, x[n][0].y, x[n][1].x, x[n][1].y);
        } else {
            st[n * P] = x[n][0];
        }
    }
    const float Dg = a.s.skip[g];
    if constexpr (CPT == 2) {
        A::st2(yp, qv[0] * fmaf(Dg, u[0], acc[0]), qv[1] * fmaf(Dg, u[1], acc[1]));
    } else {
        A::st(yp, qv[0] * fmaf(Dg, u[0], acc[0]));
    }
}

// Any d <= 64, one channel per thread, modes streamed one at a time.
template <int ACT>
__global__ __launch_bounds__(256) void decode_step_generic(DecodeArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    const int64_t D = a.s.D, P = a.s.P, H = a.s.H, d = a.s.d;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= a.s.B * D) return;
    const int64_t b = tid / D;
    const int64_t c = tid - b * D;
    const int64_t g = c / P, p = c - g * P;
    const float u = A::ld(static_cast<const T *>(a.k) + b * a.ld_in + c) *
                    A::ld(static_cast<const T *>(a.v) + b * a.ld_in + c);
    const float qv = A::ld(static_cast<const T *>(a.q) + b * a.ld_in + c);
    float2 *st = a.state + ((b * H + g) * d) * P + p;
    float acc = 0.f;
    for (int64_t n = 0; n < d; ++n) {
        const float2 l = a.s.poles[g * d + n], r = a.s.residues[g * d + n];
        const float2 xo = st[n * P];
        acc = fmaf(r.x, xo.x, acc);
        acc = fmaf(-r.y, xo.y, acc);
        st[n * P] = make_float2(fmaf(l.x, xo.x, fmaf(-l.y, xo.y, u)), fmaf(l.x, xo.y, l.y * xo.x));
    }
    A::st(static_cast<T *>(a.y) + b * a.ld_y + c, qv * fmaf(a.s.skip[g], u, acc));
}

template <int DP, int ACT>
hipError_t launch_fixed(const DecodeArgs &a, bool pair, bool uniform, hipStream_t stream) {
    const int64_t threads = a.s.B * a.s.D / (pair ? 2 : 1);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (pair) {
        if (uniform)
            decode_step_fixed<DP, ACT, 2, true><<<grid, block, 0, stream>>>(a);
        else
            decode_step_fixed<DP, ACT, 2, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (uniform)
            decode_step_fixed<DP, ACT, 1, true><<<grid, block, 0, stream>>>(a);
        else
            decode_step_fixed<DP, ACT, 1, false><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_act(const DecodeArgs &a, hipStream_t stream) {
    const int64_t P = a.s.P, d = a.s.d;
    const int esz = Act<ACT>::kBytes;
    auto aligned = [](const void *p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) % m) == 0; };
    const bool pair = (P % 2 == 0) && (a.ld_in % 2 == 0) && (a.ld_y % 2 == 0) &&
                      aligned(a.q, 2 * esz) && aligned(a.k, 2 * esz) && aligned(a.v, 2 * esz) &&
                      aligned(a.y, 2 * esz) && aligned(a.state, 16);
    const bool uniform = (P % (kWave * (pair ? 2 : 1)) == 0);
    switch (d) {
        case 8: return launch_fixed<8, ACT>(a, pair, uniform, stream);
        case 16: return launch_fixed<16, ACT>(a, pair, uniform, stream);
        case 32: return launch_fixed<32, ACT>(a, pair, uniform, stream);
        default: break;
    }
    const int64_t threads = a.s.B * a.s.D;
    decode_step_generic<ACT><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream) {
    if (a.s.B == 0) return hipSuccess;
    return a.s.act == kBF16 ? launch_act<kBF16>(a, stream) : launch_act<kF32>(a, stream);
}

}  // namespace hm
