// prefill.hip -- prompt processing of the modal Hyena operator on gfx950.
//
// For every batch row b and channel c of head g, with u_t = k_t v_t:
//     y_t = q_t (D_g u_t + Re(sum_n R_gn x_n(t))),   x_n(t+1) = lambda_gn x_n(t) + u_t,
// i.e. the causal long convolution y = q (h conv u) with the modal filter,
// evaluated without materialising the Toeplitz matrix (StripedHyena article,
// "Hyena層次結構"), plus the end-of-prompt state
//     x_n(L) = lambda^L x_n(0) + sum_t lambda_n^(L-1-t) u_t.
//
// The prompt is cut into NC chunks of T steps (the last may be shorter) so that
// batch x channels x chunks gives the GPU enough independent lanes even for few
// channels and a 64k-token prompt.  Three kernels:
//
//   1. chunk_state   (matrix cores)  for every chunk c < NC-1 the chunk-local
//      Vandermonde contraction S_c[n][b,p] = sum_j lambda_n^(T-1-j) u[b, cT+j, p].
//      Per head this is a real GEMM [2d x T] x [T x P]: the Vandermonde matrix is
//      shared by all channels of the head (weight tying, Laughing Hyena
//      Distillery review, "提出的方法").  It runs on bf16 MFMA with each operand
//      split into a high and a low bfloat16 part (hi*hi + hi*lo + lo*hi,
//      float32 accumulation), about 16 significant bits per product.
//   2. carry_scan    X_0 = x(0); X_{c+1} = lambda^T X_c + S_c: the state entering
//      every chunk, one thread per (b, g, n, p).
//   3. chunk_scan    (VALU) every lane runs the recurrence over its chunk from
//      X_c, streaming q, k, v in and y out; the lanes of the last chunk write
//      the end-of-prompt state.  12 d + 5 float32 flops per element.
//
// That is the lane-scan plan (any d, any head dimension).  A matrix-core plan
// (prefill_mfma.hip) replaces steps 1 and 3 by its 64-step sub-block kernel:
// the same contraction, chained through lambda^64, in a state-only pass, and
// the full pass from the carries; step 2 is shared.
//
// Workspace (from make_prefill_plan): for the lane-scan plan, bf16 fragments of
// the Vandermonde matrices in MFMA A-operand order; for a chunked prompt,
// lambda^T and NC chunk-state slots; for the matrix-core plan, its per-head
// sub-block tables.
#include "hm_internal.hpp"

namespace hm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKB = 64;        // time steps staged in LDS per iteration of chunk_state
constexpr int kChanBlk = 128;  // channels per chunk_state workgroup
constexpr int kLdsRow = kKB + 8;  // LDS row (one channel) in bf16 elements, padded

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// lambda^e in float64 from the polar form.
__device__ inline void pole_power(double lnr, double th, double e, double &re, double &im) {
    const double mag = (e == 0.0) ? 1.0 : exp(e * lnr);
    double s, c;
    sincos(e * th, &s, &c);
    re = mag * c;
    im = mag * s;
}

// ------------------------------------------------------------- tables

// One thread per (head g, m-tile, 32-step k-block, lane): the eight bf16 A-operand
// values lane `lane` feeds to v_mfma_f32_16x16x32_bf16 for that tile.  A row r of
// the [2d x T] Vandermonde matrix is Re (r even) or Im (r odd) of
// lambda_{r/2}^(T-1-j) at column j; rows >= 2d are zero.  A-operand layout: lane
// l holds row l%16, columns 8*(l/16) .. 8*(l/16)+7 of the 16x32 tile.
__global__ __launch_bounds__(256) void vand_tables_kernel(OpShape s, int64_t T, int64_t mtiles,
                                                          uint4 *vhi, uint4 *vlo, float2 *lamT) {
    const int64_t ks_n = T / 32;
    const int64_t total = s.H * mtiles * ks_n * kWave;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int lane = (int)(idx % kWave);
    int64_t rest = idx / kWave;
    const int64_t ks = rest % ks_n;
    rest /= ks_n;
    const int64_t mt = rest % mtiles;
    const int64_t g = rest / mtiles;
    const int64_t row = 16 * mt + (lane % 16);
    const int64_t n = row / 2;
    const bool imag = (row % 2) != 0;
    uint32_t hi[8], lo[8];
    double lnr = 0.0, th = 0.0;
    if (n < s.d) {
        const float2 l = s.poles[g * s.d + n];
        lnr = log(hypot((double)l.x, (double)l.y));
        th = atan2((double)l.y, (double)l.x);
    }
    for (int i = 0; i < 8; ++i) {
        const int64_t j = 32 * ks + 8 * (lane / 16) + i;
        float val = 0.f;
        if (n < s.d) {
            double re, im;
            pole_power(lnr, th, (double)(T - 1 - j), re, im);
            val = (float)(imag ? im : re);
        }
        hi[i] = f32_to_bf16(val);
        lo[i] = f32_to_bf16(val - __uint_as_float(hi[i] << 16));
    }
    const int64_t o = ((g * mtiles + mt) * ks_n + ks) * kWave + lane;
    vhi[o] = make_uint4(hi[0] | hi[1] << 16, hi[2] | hi[3] << 16, hi[4] | hi[5] << 16, hi[6] | hi[7] << 16);
    vlo[o] = make_uint4(lo[0] | lo[1] << 16, lo[2] | lo[3] << 16, lo[4] | lo[5] << 16, lo[6] | lo[7] << 16);
    if (mt == 0 && ks == 0 && lane < s.d) {
        const float2 l = s.poles[g * s.d + lane];
        double re, im;
        pole_power(log(hypot((double)l.x, (double)l.y)), atan2((double)l.y, (double)l.x), (double)T, re,
                   im);
        lamT[g * s.d + lane] = make_float2((float)re, (float)im);
    }
}

// ------------------------------------------------------------- phase 1

// Workgroup (channel block cb of head g, chunk c < NC-1, batch row b), 4 waves.
// Each 64-step slab of u = k v for up to 128 channels is split into bf16 hi/lo,
// transposed into LDS as [channel][time], and contracted with the head's
// Vandermonde fragments: wave w owns channel tiles 2w and 2w+1 (16 channels
// each) and all MT row tiles.  Output rows (Re, Im of mode n) land in the
// chunk-state slot c+1.
template <int MT, int ACT, bool VEC>
__global__ __launch_bounds__(256) void chunk_state_kernel(PrefillArgs a) {
    using A = Act<ACT>;
    using T = typename A::T;
    __shared__ __attribute__((aligned(16))) uint16_t u_hi[kChanBlk * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t u_lo[kChanBlk * kLdsRow];

    const OpShape &s = a.s;
    const int64_t P = s.P, d = s.d, Tc = a.plan.T;
    const int64_t ncb = (P + kChanBlk - 1) / kChanBlk;
    const int64_t g = blockIdx.x / ncb, cb = blockIdx.x % ncb;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    const int64_t p0 = cb * kChanBlk;
    const int64_t nvalid = (P - p0 < kChanBlk) ? (P - p0) : kChanBlk;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;

    // staging role: 8 channels x 4 time steps
    const int tw = tid % 16, tt = tid / 16;
    const int64_t chl = 8 * tw;  // local channel of the first of the 8
    const int64_t cglob = g * P + p0 + chl;
    const T *kbase = static_cast<const T *>(a.k) + (b * a.plan.L + c * Tc) * a.ld_in + cglob;
    const T *vbase = static_cast<const T *>(a.v) + (b * a.plan.L + c * Tc) * a.ld_in + cglob;

    const int64_t ks_n = Tc / 32;
    const uint4 *vhi = reinterpret_cast<const uint4 *>(a.ws + a.plan.off_vand_hi) + (g * MT) * ks_n * kWave;
    const uint4 *vlo = reinterpret_cast<const uint4 *>(a.ws + a.plan.off_vand_lo) + (g * MT) * ks_n * kWave;

    f32x4 acc[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb = 0; kb < Tc; kb += kKB) {
        // ---- stage u = k v for 4 steps x 8 channels, split, transpose into LDS
        float u[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t off = (kb + 4 * tt + r) * a.ld_in;
            if constexpr (VEC) {
                if (chl < nvalid) {
                    if constexpr (ACT == kBF16) {
                        const uint4 kv = *reinterpret_cast<const uint4 *>(kbase + off);
                        const uint4 vv = *reinterpret_cast<const uint4 *>(vbase + off);
                        const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            u[r][2 * e] = bf16_lo(kw[e]) * bf16_lo(vw[e]);
                            u[r][2 * e + 1] = bf16_hi(kw[e]) * bf16_hi(vw[e]);
                        }
                    } else {
                        const float4 k0 = *reinterpret_cast<const float4 *>(kbase + off);
                        const float4 k1 = *reinterpret_cast<const float4 *>(kbase + off + 4);
                        const float4 v0 = *reinterpret_cast<const float4 *>(vbase + off);
                        const float4 v1 = *reinterpret_cast<const float4 *>(vbase + off + 4);
                        u[r][0] = k0.x * v0.x; u[r][1] = k0.y * v0.y;
                        u[r][2] = k0.z * v0.z; u[r][3] = k0.w * v0.w;
                        u[r][4] = k1.x * v1.x; u[r][5] = k1.y * v1.y;
                        u[r][6] = k1.z * v1.z; u[r][7] = k1.w * v1.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) u[r][e] = 0.f;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    u[r][e] = (chl + e < nvalid) ? A::ld(kbase + off + e) * A::ld(vbase + off + e) : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t h[4], l[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                h[r] = f32_to_bf16(u[r][e]);
                l[r] = f32_to_bf16(u[r][e] - __uint_as_float(h[r] << 16));
            }
            const int o = (int)(chl + e) * kLdsRow + 4 * tt;
            *reinterpret_cast<uint2 *>(&u_hi[o]) = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
            *reinterpret_cast<uint2 *>(&u_lo[o]) = make_uint2(l[0] | l[1] << 16, l[2] | l[3] << 16);
        }
        __syncthreads();

        // ---- contract: two 32-step MFMA k-blocks per slab
#pragma unroll
        for (int kk = 0; kk < kKB / 32; ++kk) {
            const int64_t ks = kb / 32 + kk;
            bf16x8 ahi[MT], alo[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const uint4 h4 = vhi[(m * ks_n + ks) * kWave + lane];
                const uint4 l4 = vlo[(m * ks_n + ks) * kWave + lane];
                ahi[m] = __builtin_bit_cast(bf16x8, h4);
                alo[m] = __builtin_bit_cast(bf16x8, l4);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ch = 16 * (2 * w + j) + (lane % 16);
                const int o = ch * kLdsRow + 32 * kk + 8 * (lane / 16);
                const bf16x8 bhi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&u_hi[o]));
                const bf16x8 blo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(&u_lo[o]));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[m], bhi, acc[m][j], 0, 0, 0);
                    acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[m], blo, acc[m][j], 0, 0, 0);
                    acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[m], bhi, acc[m][j], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // ---- write S_c: C-tile lane l holds column l%16, rows 4*(l/16) .. +3,
    // i.e. (Re, Im) of modes 8m + 2*(l/16) and 8m + 2*(l/16) + 1.
    const int64_t slot = s.B * s.H * d * P;
    float2 *out = reinterpret_cast<float2 *>(a.ws + a.plan.off_carry) + (c + 1) * slot +
                  ((b * s.H + g) * d) * P;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t pl = 16 * (2 * w + j) + (lane % 16);
        if (pl >= nvalid) continue;
        const int64_t p = p0 + pl;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int64_t n0 = 8 * m + 2 * (lane / 16);
            if (n0 < d) out[n0 * P + p] = make_float2(acc[m][j][0], acc[m][j][1]);
            if (n0 + 1 < d) out[(n0 + 1) * P + p] = make_float2(acc[m][j][2], acc[m][j][3]);
        }
    }
}

// ------------------------------------------------------------- phase 2

// One thread per state element (b, g, n, p): X_0 = x(0) (copied to slot 0 when
// given), then X_{c+1} = lambda^T X_c + S_c in place over slots 1 .. NC-1.
__global__ __launch_bounds__(256) void carry_scan_kernel(PrefillArgs a) {
    const OpShape &s = a.s;
    const int64_t slot = s.B * s.H * s.d * s.P;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= slot) return;
    const int64_t n = (e / s.P) % s.d;
    const int64_t g = (e / (s.P * s.d)) % s.H;
    const float2 lt = reinterpret_cast<const float2 *>(a.ws + a.plan.off_lamT)[g * s.d + n];
    float2 *carry = reinterpret_cast<float2 *>(a.ws + a.plan.off_carry) + e;
    float2 X = make_float2(0.f, 0.f);
    if (a.state_in) {
        X = a.state_in[e];
        carry[0] = X;
    }
    const int64_t NC = a.plan.NC;
    int64_t c = 1;
    for (; c + 4 <= NC; c += 4) {
        float2 S[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) S[i] = carry[(c + i) * slot];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            X = make_float2(fmaf(lt.x, X.x, fmaf(-lt.y, X.y, S[i].x)), fmaf(lt.x, X.y, fmaf(lt.y, X.x, S[i].y)));
            carry[(c + i) * slot] = X;
        }
    }
    for (; c < NC; ++c) {
        const float2 S = carry[c * slot];
        X = make_float2(fmaf(lt.x, X.x, fmaf(-lt.y, X.y, S.x)), fmaf(lt.x, X.y, fmaf(lt.y, X.x, S.y)));
        carry[c * slot] = X;
    }
}

// ------------------------------------------------------------- phase 3

// Sum of v over the SPLIT adjacent lanes of one channel (SPLIT = 1, 2 or 4),
// with DPP quad permutations: one VALU op per halving.
template <int SPLIT>
__device__ __forceinline__ float lane_group_sum(float v) {
    if constexpr (SPLIT >= 2)  // swap lanes 0<->1, 2<->3
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (SPLIT >= 4)  // swap pairs 01<->23
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    return v;
}

// In-chunk modal scan.  A channel's d = DL*SPLIT modes are held by SPLIT
// adjacent lanes (DL each), so one lane never holds more than 16 modes: the
// complex state (2 DL floats) and, with SPLIT = 1 and a wave inside one head,
// the pole/residue tables fit in registers (scalar registers when wave-uniform,
// vector registers otherwise).  Each lane group runs the recurrence over its
// chunk U steps at a time with q, k, v of the next U steps already in flight;
// the output sums the lane group with DPP.  Activations go through raw-buffer
// accesses whose per-step offset is a scalar (no vector address arithmetic).
// Workgroup: 256 lanes = 256 / SPLIT channels of one batch row and chunk.
template <int DL, int SPLIT, int ACT, bool UNIFORM, int U>
__global__ __launch_bounds__(256) void chunk_scan_kernel(PrefillArgs a, const float2 *carry0) {
    using T = typename Act<ACT>::T;
    using BA = BufAct<ACT>;
    constexpr uint32_t esz = Act<ACT>::kBytes;
    constexpr int DP = DL * SPLIT;  // modes per channel
    constexpr int CPB = 256 / SPLIT;  // channels per workgroup
    const OpShape &s = a.s;
    const int64_t P = s.P, H = s.H, L = a.plan.L, Tc = a.plan.T;
    const int part = (int)(threadIdx.x % SPLIT);
    const int ch = (int)(blockIdx.x * CPB + threadIdx.x / SPLIT);
    const int64_t c = blockIdx.y, b = blockIdx.z;
    if (ch >= s.D) return;
    int g = ch / (int)P;
    if (UNIFORM) g = __builtin_amdgcn_readfirstlane(g);
    const int64_t p = ch - (int64_t)g * P;
    const int n0 = part * DL;  // first mode of this lane

    float lr[DL], li[DL], rr[DL], ri[DL];
#pragma unroll
    for (int n = 0; n < DL; ++n) {
        const float2 l = s.poles[(int64_t)g * DP + n0 + n], r = s.residues[(int64_t)g * DP + n0 + n];
        lr[n] = l.x;
        li[n] = l.y;
        rr[n] = r.x;
        ri[n] = r.y;
    }
    const float Dg = (part == 0) ? s.skip[g] : 0.f;  // the skip term is added once per channel

    const int64_t sidx = ((b * H + g) * DP + n0) * P + p;  // mode n0 of this channel in a state slot
    const float2 *src = (c == 0) ? (carry0 ? carry0 + sidx : nullptr)
                                 : reinterpret_cast<const float2 *>(a.ws + a.plan.off_carry) +
                                       c * (s.B * H * DP * P) + sidx;
    float xr[DL], xi[DL];
#pragma unroll
    for (int n = 0; n < DL; ++n) {
        const float2 v = src ? src[n * P] : make_float2(0.f, 0.f);
        xr[n] = v.x;
        xi[n] = v.y;
    }

    // Regions of this (batch row, chunk): nsteps rows of ld elements each; the
    // host guarantees they fit 31-bit byte offsets.
    const int64_t t0 = c * Tc;
    const int nsteps = (int)(((L - t0) < Tc) ? (L - t0) : Tc);
    const uint32_t ldi = (uint32_t)(a.ld_in * esz), ldo = (uint32_t)(a.ld_y * esz);
    const uint32_t in_bytes = (uint32_t)(nsteps - 1) * ldi + (uint32_t)s.D * esz;
    const uint32_t out_bytes = (uint32_t)(nsteps - 1) * ldo + (uint32_t)s.D * esz;
    const auto rq = make_region(static_cast<const T *>(a.q) + (b * L + t0) * a.ld_in, in_bytes);
    const auto rk = make_region(static_cast<const T *>(a.k) + (b * L + t0) * a.ld_in, in_bytes);
    const auto rv = make_region(static_cast<const T *>(a.v) + (b * L + t0) * a.ld_in, in_bytes);
    const auto ry = make_region(static_cast<T *>(a.y) + (b * L + t0) * a.ld_y, out_bytes);
    const uint32_t lane_off = (uint32_t)ch * esz;

    auto step = [&](float qv, float kv, float vv) -> float {
        const float u = kv * vv;
        float z0 = Dg * u, z1 = 0.f;
#pragma unroll
        for (int n = 0; n < DL; ++n) {
            z0 = fmaf(rr[n], xr[n], z0);
            z1 = fmaf(-ri[n], xi[n], z1);
            const float cross = li[n] * xr[n];
            xr[n] = fmaf(lr[n], xr[n], fmaf(-li[n], xi[n], u));
            xi[n] = fmaf(lr[n], xi[n], cross);
        }
        return qv * lane_group_sum<SPLIT>(z0 + z1);
    };
    // every lane of a group holds the same y and stores it: one instruction, no branch
    auto store = [&](int t, float yv) { BA::st(ry, lane_off, (uint32_t)t * ldo, yv); };

    float cq[U], ck[U], cv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const uint32_t o = (uint32_t)(i < nsteps ? i : nsteps - 1) * ldi;
        cq[i] = BA::ld(rq, lane_off, o);
        ck[i] = BA::ld(rk, lane_off, o);
        cv[i] = BA::ld(rv, lane_off, o);
    }
    const int nfull = nsteps - nsteps % U;
    for (int t = 0; t < nfull; t += U) {
        float nq[U], nk[U], nv[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {  // next U steps, clamped into the chunk
            const int tt = (t + U + i < nsteps) ? t + U + i : nsteps - 1;
            const uint32_t o = (uint32_t)tt * ldi;
            nq[i] = BA::ld(rq, lane_off, o);
            nk[i] = BA::ld(rk, lane_off, o);
            nv[i] = BA::ld(rv, lane_off, o);
        }
#pragma unroll
        for (int i = 0; i < U; ++i) store(t + i, step(cq[i], ck[i], cv[i]));
#pragma unroll
        for (int i = 0; i < U; ++i) {
            cq[i] = nq[i];
            ck[i] = nk[i];
            cv[i] = nv[i];
        }
    }
#pragma unroll
    for (int i = 0; i < U; ++i)  // ragged tail: fewer than U steps, already loaded
        if (nfull + i < nsteps) store(nfull + i, step(cq[i], ck[i], cv[i]));

    if (c == a.plan.NC - 1) {
        float2 *dst = a.state_out + sidx;
#pragma unroll
        for (int n = 0; n < DL; ++n) dst[n * P] = make_float2(xr[n], xi[n]);
    }
}

// Modes streamed from memory: any d <= 64, one lane per (b, chunk, channel).
// The state of the lane lives in a chunk slot (or state_out) and is updated in
// place every step; used only for mode counts without a register variant.
template <int ACT>
__global__ __launch_bounds__(256) void chunk_scan_generic_kernel(PrefillArgs a, const float2 *carry0) {
    using A = Act<ACT>;
    using T = typename A::T;
    const OpShape &s = a.s;
    const int64_t D = s.D, P = s.P, H = s.H, d = s.d, L = a.plan.L, Tc = a.plan.T;
    const int64_t ch = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    if (ch >= D) return;
    const int64_t g = ch / P, p = ch - g * P;
    const int64_t sidx = ((b * H + g) * d) * P + p;
    float2 x[kMaxModes];
    const float2 *src = (c == 0) ? (carry0 ? carry0 + sidx : nullptr)
                                 : reinterpret_cast<const float2 *>(a.ws + a.plan.off_carry) +
                                       c * (s.B * H * d * P) + sidx;
    for (int64_t n = 0; n < d; ++n) x[n] = src ? src[n * P] : make_float2(0.f, 0.f);
    const int64_t t0 = c * Tc;
    const int64_t nsteps = ((L - t0) < Tc) ? (L - t0) : Tc;
    for (int64_t t = 0; t < nsteps; ++t) {
        const int64_t ri = (b * L + t0 + t) * a.ld_in + ch;
        const float u = A::ld(static_cast<const T *>(a.k) + ri) * A::ld(static_cast<const T *>(a.v) + ri);
        float z = s.skip[g] * u;
        for (int64_t n = 0; n < d; ++n) {
            const float2 l = s.poles[g * d + n], r = s.residues[g * d + n], xo = x[n];
            z = fmaf(r.x, xo.x, z);
            z = fmaf(-r.y, xo.y, z);
            x[n] = make_float2(fmaf(l.x, xo.x, fmaf(-l.y, xo.y, u)), fmaf(l.x, xo.y, l.y * xo.x));
        }
        A::st(static_cast<T *>(a.y) + (b * L + t0 + t) * a.ld_y + ch,
              A::ld(static_cast<const T *>(a.q) + ri) * z);
    }
    if (c == a.plan.NC - 1)
        for (int64_t n = 0; n < d; ++n) a.state_out[sidx + n * P] = x[n];
}

// Empty prompt: state_out = state_in (or zero).
__global__ __launch_bounds__(256) void state_copy_kernel(const float2 *in, float2 *out, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e < n) out[e] = in ? in[e] : make_float2(0.f, 0.f);
}

template <int MT, int ACT>
hipError_t launch_chunk_state_mt(const PrefillArgs &a, bool vec, hipStream_t stream) {
    const int64_t ncb = (a.s.P + kChanBlk - 1) / kChanBlk;
    const dim3 grid((unsigned)(a.s.H * ncb), (unsigned)(a.plan.NC - 1), (unsigned)a.s.B);
    if (vec)
        chunk_state_kernel<MT, ACT, true><<<grid, dim3(256), 0, stream>>>(a);
    else
        chunk_state_kernel<MT, ACT, false><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_chunk_state(const PrefillArgs &a, bool vec, hipStream_t stream) {
    switch (a.plan.mtiles) {
        case 1: return launch_chunk_state_mt<1, ACT>(a, vec, stream);
        case 2: return launch_chunk_state_mt<2, ACT>(a, vec, stream);
        case 4: return launch_chunk_state_mt<4, ACT>(a, vec, stream);
        default: return launch_chunk_state_mt<8, ACT>(a, vec, stream);
    }
}

template <int DL, int SPLIT, int ACT, int U>
hipError_t launch_scan_dp(const PrefillArgs &a, const float2 *carry0, hipStream_t stream) {
    constexpr int cpb = 256 / SPLIT;
    const dim3 grid((unsigned)((a.s.D + cpb - 1) / cpb), (unsigned)a.plan.NC, (unsigned)a.s.B);
    if constexpr (SPLIT == 1) {
        if (a.s.P % kWave == 0) {
            chunk_scan_kernel<DL, SPLIT, ACT, true, U><<<grid, dim3(256), 0, stream>>>(a, carry0);
            return hipGetLastError();
        }
    }
    chunk_scan_kernel<DL, SPLIT, ACT, false, U><<<grid, dim3(256), 0, stream>>>(a, carry0);
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_scan(const PrefillArgs &a, const float2 *carry0, hipStream_t stream) {
    const int64_t esz = Act<ACT>::kBytes;
    const int64_t ld = a.ld_in > a.ld_y ? a.ld_in : a.ld_y;
    const bool fits = a.plan.T * ld * esz < (int64_t(1) << 31);
    switch (fits ? a.s.d : 0) {
        case 8: return launch_scan_dp<8, 1, ACT, 8>(a, carry0, stream);
        case 16: return launch_scan_dp<16, 1, ACT, 8>(a, carry0, stream);
        case 32: return launch_scan_dp<16, 2, ACT, 8>(a, carry0, stream);
        case 64: return launch_scan_dp<16, 4, ACT, 8>(a, carry0, stream);
        default: break;
    }
    const dim3 grid((unsigned)((a.s.D + 255) / 256), (unsigned)a.plan.NC, (unsigned)a.s.B);
    chunk_scan_generic_kernel<ACT><<<grid, dim3(256), 0, stream>>>(a, carry0);
    return hipGetLastError();
}

}  // namespace

PrefillPlan make_prefill_plan(const OpShape &s, int64_t L, int64_t chunk, int algo) {
    PrefillPlan p{};
    p.L = L;
    const int pt = mfma_channel_tile(s);
    p.algo = (algo == kAlgoScan || pt == 0) ? kAlgoScan : kAlgoMfma;
    if (L <= 0) {
        p.T = 0;
        p.NC = 0;
        return p;
    }
    int64_t T;
    if (chunk > 0) {
        T = chunk;
    } else {
        int64_t nc;
        if (p.algo == kAlgoMfma) {
            // one workgroup (batch row, head, channel tile) per CU: chunk the
            // prompt only when there are fewer such tiles than CUs
            const int64_t tiles = s.B * s.H * (s.P / pt);
            nc = (256 + tiles - 1) / (tiles > 0 ? tiles : 1);
        } else {
            // enough independent (b, chunk, channel) lanes for ~32 waves per CU
            const int64_t waves_per_chunk = (s.B * s.D + kWave - 1) / kWave;
            nc = (8192 + waves_per_chunk - 1) / (waves_per_chunk > 0 ? waves_per_chunk : 1);
        }
        const int64_t ncmax = (L + kKB - 1) / kKB;
        if (nc < 1) nc = 1;
        if (nc > ncmax) nc = ncmax;
        if (nc > 65535) nc = 65535;
        T = (L + nc - 1) / nc;
        T = (T + kKB - 1) / kKB * kKB;
    }
    p.NC = (L + T - 1) / T;
    p.T = (p.NC == 1) ? L : T;
    int64_t mt = (2 * s.d + 15) / 16;
    p.mtiles = mt <= 1 ? 1 : mt <= 2 ? 2 : mt <= 4 ? 4 : 8;
    size_t off = 0;
    if (p.NC > 1) {
        if (p.algo == kAlgoScan) {  // the matrix-core path gets its chunk states from its own sub-block tables
            const size_t frag = (size_t)s.H * p.mtiles * (p.T / 32) * kWave * 16;
            p.off_vand_hi = off;
            off = align256(off + frag);
            p.off_vand_lo = off;
            off = align256(off + frag);
        }
        p.off_lamT = off;
        off = align256(off + (size_t)s.H * s.d * 8);
        p.off_carry = off;
        off = align256(off + (size_t)p.NC * s.B * s.D * s.d * 8);
    }
    if (p.algo == kAlgoMfma) {
        p.off_mfma_tab = off;
        off = align256(off + mfma_table_bytes(s.H, s.d, s.act));
        p.off_mfma_lam = off;
        off = align256(off + mfma_lam_bytes(s.H, s.d));
    }
    p.bytes = off;
    return p;
}

// The matrix-core path streams 16-byte pieces of 8 channels: it needs aligned
// activation rows.
static bool mfma_aligned(const PrefillArgs &a) {
    const int esz = a.s.act == kBF16 ? 2 : 4;
    auto al16 = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; };
    return al16(a.q) && al16(a.k) && al16(a.v) && al16(a.y) && (a.ld_in * esz) % 16 == 0 &&
           (a.ld_y * esz) % 16 == 0;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
    const OpShape &s = a.s;
    const int64_t nstate = s.B * s.D * s.d;
    if (nstate == 0) return hipSuccess;
    if (a.plan.L == 0) {
        state_copy_kernel<<<dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, stream>>>(
            a.state_in, a.state_out, nstate);
        return hipGetLastError();
    }
    hipError_t err;
    const float2 *carry0 = a.state_in;
    const int esz = s.act == kBF16 ? 2 : 4;
    auto al16 = [](const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; };
    // 16-byte k, v pieces for the chunk-state passes
    const bool vec = (s.P % 8 == 0) && ((a.ld_in * esz) % 16 == 0) && al16(a.k) && al16(a.v);
    if (a.plan.algo == kAlgoMfma) {
        // Matrix-core plan.  Chunk states come from the state-only sub-block
        // pass (either load width); the full pass needs 16-byte-aligned rows
        // of q, k, v and y, else the lane scan runs from the same carries.
        const bool full = mfma_aligned(a);
        if (full || a.plan.NC > 1)
            if ((err = launch_mfma_tables(a, stream)) != hipSuccess) return err;
        if (a.plan.NC > 1) {
            if ((err = launch_chunk_mfma_state(a, vec, stream)) != hipSuccess) return err;
            carry_scan_kernel<<<dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, stream>>>(a);
            if ((err = hipGetLastError()) != hipSuccess) return err;
            carry0 = a.state_in ? reinterpret_cast<const float2 *>(a.ws + a.plan.off_carry) : nullptr;
        }
        if (full) return launch_chunk_mfma(a, carry0, stream);
        return s.act == kBF16 ? launch_scan<kBF16>(a, carry0, stream) : launch_scan<kF32>(a, carry0, stream);
    }
    if (a.plan.NC > 1) {
        const int64_t total = s.H * a.plan.mtiles * (a.plan.T / 32) * kWave;
        vand_tables_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream>>>(
            s, a.plan.T, a.plan.mtiles, reinterpret_cast<uint4 *>(a.ws + a.plan.off_vand_hi),
            reinterpret_cast<uint4 *>(a.ws + a.plan.off_vand_lo),
            reinterpret_cast<float2 *>(a.ws + a.plan.off_lamT));
        if ((err = hipGetLastError()) != hipSuccess) return err;
        err = s.act == kBF16 ? launch_chunk_state<kBF16>(a, vec, stream) : launch_chunk_state<kF32>(a, vec, stream);
        if (err != hipSuccess) return err;
        carry_scan_kernel<<<dim3((unsigned)((nstate + 255) / 256)), dim3(256), 0, stream>>>(a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        carry0 = a.state_in ? reinterpret_cast<const float2 *>(a.ws + a.plan.off_carry) : nullptr;
    }
    return s.act == kBF16 ? launch_scan<kBF16>(a, carry0, stream) : launch_scan<kF32>(a, carry0, stream);
}

}  // namespace hm
