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
// written) plus four activations, so it is bound by HBM bandwidth -- or, for
// small batches, by the fixed cost of a dispatch (about 1.6 us per launch on
// MI355X, graph-replayed) plus one memory round trip.  Layout and mapping:
//   - the state is [B][H][d][P] complex float32, so for a fixed mode the lanes
//     of a wave touch consecutive channels: each state access of a wave is one
//     contiguous segment (1 KiB with two channels per lane);
//   - large batches: a lane owns two adjacent channels and all their modes
//     (16-byte state accesses); when a wave stays inside one head the head index
//     is made wave-uniform and the pole/residue tables come through the scalar
//     cache into SGPRs;
//   - d = 32: one lane per channel and all 32 modes when the batch holds fewer
//     than 64 K channels (fewer, longer lanes finish sooner than split ones:
//     measured on MI355X, B = 4, D = 4096), else SPLIT = 2 adjacent lanes share
//     a channel with 16 modes each; d = 64: four lanes of 16 modes.  Partial
//     readouts of a channel are summed with DPP.
#include "hm_internal.hpp"

namespace hm {
namespace {

// State and output stores are nontemporal: neither is read again in this
// launch, and streaming them out keeps them from sitting dirty in L2 until the
// end-of-kernel write-back (measured on the state: 4 % faster at B = 256,
// D = 2048).
typedef float vf4 __attribute__((ext_vector_type(4)));
typedef float vf2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store_state(float2 *p, float2 a, float2 b) {
    const vf4 v = {a.x, a.y, b.x, b.y};
    __builtin_nontemporal_store(v, reinterpret_cast<vf4 *>(p));
}
__device__ __forceinline__ void store_state(float2 *p, float2 a) {
    const vf2 v = {a.x, a.y};
    __builtin_nontemporal_store(v, reinterpret_cast<vf2 *>(p));
}
// The outputs too (batch 64, D = 2048: 5.55 -> 5.33 us per step; no change at 16 or 256).
template <int ACT>
__device__ __forceinline__ void store_y(typename Act<ACT>::T *p, float a, float b) {
    if constexpr (ACT == kBF16) {
        __builtin_nontemporal_store(pack_bf16x2(a, b), reinterpret_cast<uint32_t *>(p));
    } else {
        const vf2 v = {a, b};
        __builtin_nontemporal_store(v, reinterpret_cast<vf2 *>(p));
    }
}
template <int ACT>
__device__ __forceinline__ void store_y(typename Act<ACT>::T *p, float a) {
    if constexpr (ACT == kBF16)
        __builtin_nontemporal_store((uint16_t)f32_to_bf16(a), p);
    else
        __builtin_nontemporal_store(a, p);
}

// Sum over the SPLIT adjacent lanes of a channel (DPP quad permutations).
template <int SPLIT>
__device__ __forceinline__ float lane_group_sum(float v) {
    if constexpr (SPLIT >= 2)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (SPLIT >= 4)
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    return v;
}

// The operands come as separate parameters, ordered so that the ones the
// first loads need (q, k, v, state, row stride, P, H: 14 SGPRs) are preloaded
// at wave launch (the library builds this file with kernarg preloading;
// measured on MI355X: 2.75 -> 2.60 us per step at B = 16, D = 2048, d = 16).
// Grid: x = lane blocks over the channels of one batch row, y = batch row.
// The block size BS is a compile-time constant and, when the lane blocks tile
// the row exactly (FULL), there is no early exit: every argument load is then
// issued at once at entry, instead of a block-size load, a branch and a second
// round of loads (measured on MI355X: 3.00 -> 2.75 us per step at B = 16,
// D = 2048, d = 16; the launch is latency-bound there).
// A lane owns CPT adjacent channels (CPT = 2 only with SPLIT = 1) and DL of
// their modes; SPLIT lanes share a channel when the batch is too small to fill
// the GPU otherwise, and their partial outputs are summed with DPP.
template <int DL, int SPLIT, int CPT, int ACT, bool UNIFORM, int BS, bool FULL>
__global__ __launch_bounds__(BS) void decode_step_fixed(const void *q_, const void *k_, const void *v_,
                                                        float2 *state, int64_t ld_in, int32_t P32, int32_t H32,
                                                        void *y_, int64_t ld_y, const float2 *poles,
                                                        const float2 *residues, const float *skip, int32_t D32) {
    using A = Act<ACT>;
    using T = typename A::T;
    constexpr int DP = DL * SPLIT;
    const int64_t P = P32, H = H32;
    const int lane_id = (int)(blockIdx.x * BS + threadIdx.x);  // within the batch row
    const int part = lane_id % SPLIT;
    const int c = (lane_id / SPLIT) * CPT;
    if constexpr (!FULL) {
        if (c >= D32) return;
    }
    const int64_t b = blockIdx.y;
    int g = c / (int)P;
    if (UNIFORM) g = __builtin_amdgcn_readfirstlane(g);
    const int64_t p = c - (int64_t)g * P;
    const int n0 = part * DL;

    const T *qp = static_cast<const T *>(q_) + b * ld_in + c;
    const T *kp = static_cast<const T *>(k_) + b * ld_in + c;
    const T *vp = static_cast<const T *>(v_) + b * ld_in + c;
    T *yp = static_cast<T *>(y_) + b * ld_y + c;
    const float2 *lam = poles + (int64_t)g * DP + n0;
    const float2 *res = residues + (int64_t)g * DP + n0;
    float2 *st = state + ((b * H + g) * DP + n0) * P + p;

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

    // All state loads first: DL independent 8*CPT-byte loads in flight per lane.
    float2 x[DL][CPT];
#pragma unroll
    for (int n = 0; n < DL; ++n) {
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
    for (int n = 0; n < DL; ++n) {
        const float2 l = lam[n], r = res[n];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const float2 xo = x[n][j];
            acc[j] = fmaf(r.x, xo.x, acc[j]);
            acc[j] = fmaf(-r.y, xo.y, acc[j]);
            x[n][j] = make_float2(fmaf(l.x, xo.x, fmaf(-l.y, xo.y, u[j])), fmaf(l.x, xo.y, l.y * xo.x));
        }
    }
#pragma unroll
    for (int n = 0; n < DL; ++n) {
        if constexpr (CPT == 2) {
            store_state(st + n * P, x[n][0], x[n][1]);
        } else {
            store_state(st + n * P, x[n][0]);
        }
    }
    const float Dg = skip[g];
    if constexpr (CPT == 2) {
        store_y<ACT>(yp, qv[0] * fmaf(Dg, u[0], acc[0]), qv[1] * fmaf(Dg, u[1], acc[1]));
    } else {
        // every lane of the group holds the same sum and stores it
        store_y<ACT>(yp, qv[0] * fmaf(Dg, u[0], lane_group_sum<SPLIT>(acc[0])));
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

#define FIXED_ARGS a.q, a.k, a.v, a.state, a.ld_in, (int32_t)a.s.P, (int32_t)a.s.H, a.y, a.ld_y, a.s.poles, \
                   a.s.residues, a.s.skip, (int32_t)a.s.D
template <int DL, int SPLIT, int CPT, int ACT>
hipError_t launch_fixed(const DecodeArgs &a, hipStream_t stream) {
    const int64_t lanes = a.s.D / CPT * SPLIT;  // per batch row
    // small launches: one-wave workgroups spread the work over more CUs
    const int bs = (lanes * a.s.B >= 256 * 1024) ? 256 : 64;
    const dim3 grid((unsigned)((lanes + bs - 1) / bs), (unsigned)a.s.B), block(bs);
    const bool uniform = SPLIT == 1 && (a.s.P % (kWave * CPT) == 0);
    const bool full = lanes % bs == 0;
    if (bs == 256) {
        if (uniform && full) decode_step_fixed<DL, SPLIT, CPT, ACT, (SPLIT == 1), 256, true><<<grid, block, 0, stream>>>(FIXED_ARGS);
        else if (full) decode_step_fixed<DL, SPLIT, CPT, ACT, false, 256, true><<<grid, block, 0, stream>>>(FIXED_ARGS);
        else decode_step_fixed<DL, SPLIT, CPT, ACT, false, 256, false><<<grid, block, 0, stream>>>(FIXED_ARGS);
    } else {
        if (uniform && full) decode_step_fixed<DL, SPLIT, CPT, ACT, (SPLIT == 1), 64, true><<<grid, block, 0, stream>>>(FIXED_ARGS);
        else if (full) decode_step_fixed<DL, SPLIT, CPT, ACT, false, 64, true><<<grid, block, 0, stream>>>(FIXED_ARGS);
        else decode_step_fixed<DL, SPLIT, CPT, ACT, false, 64, false><<<grid, block, 0, stream>>>(FIXED_ARGS);
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
    const bool small = a.s.B * a.s.D < 65536;
    switch (d) {
        case 8:
            return pair ? launch_fixed<8, 1, 2, ACT>(a, stream) : launch_fixed<8, 1, 1, ACT>(a, stream);
        case 16:
            return pair ? launch_fixed<16, 1, 2, ACT>(a, stream) : launch_fixed<16, 1, 1, ACT>(a, stream);
        case 32:
            return small ? launch_fixed<32, 1, 1, ACT>(a, stream) : launch_fixed<16, 2, 1, ACT>(a, stream);
        case 64:
            return launch_fixed<16, 4, 1, ACT>(a, stream);
        default:
            break;
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
