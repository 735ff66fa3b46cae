// dense.hip -- the projections around the operator in a projected Hyena stack:
// per-row inverse RMS and a bf16 GEMM with an optional per-row scale.
//
//   inv_rms[m] = 1 / sqrt(mean_k x[m][k]^2 + eps)                (float32)
//   C[m][n]    = bf16( row_scale[m] * sum_k A[m][k] W[n][k] )      (float32 accumulation)
//
// A (activations) and W (weights, [N][K]) are both K-contiguous, which is the
// natural operand order of the matrix cores: a 16x16x32 bf16 MFMA fragment is
// 16 contiguous bytes of one row per lane (lane l: row l%16, k 8*(l/16)..+7).
//
// Two GEMM kernels:
//   * gemm_tiled  (large M): 256-thread workgroups on a BM x BN tile, K staged
//     64 at a time through double-buffered LDS (rows padded to 144 B so the
//     16-lane fragment reads hit distinct banks), 4 waves each owning a WM x WN
//     sub-tile of 16x16x32 MFMAs.  Tiles are ordered so each XCD walks a
//     contiguous range, grouped GM m-tiles at a time, to keep A and W in L2.
//   * gemm_skinny (M <= 64, the generation step): a workgroup owns BN columns
//     and all rows; its KW waves split K, stream W and A fragments straight from
//     memory (no LDS staging), and reduce their partial tiles through LDS.  The
//     step is bound by streaming W from HBM.
#include "hm_internal.hpp"

namespace hm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const uint4 a, const uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}

// ------------------------------------------------------------------ RMS

// One wave per row; lanes stride over the row in 16-byte (8 x bf16) pieces.
__global__ __launch_bounds__(256) void row_rms_kernel(RmsArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= a.M) return;
    const uint16_t *x = static_cast<const uint16_t *>(a.x) + row * a.ld;
    float s = 0.f;
    if (a.vec) {
        for (int64_t k = (int64_t)lane * 8; k < a.D; k += kWave * 8) {
            const uint4 w = *reinterpret_cast<const uint4 *>(x + k);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_lo(ws[e]), hi = bf16_hi(ws[e]);
                s = fmaf(lo, lo, s);
                s = fmaf(hi, hi, s);
            }
        }
    } else {
        for (int64_t k = lane; k < a.D; k += kWave) {
            const float v = __uint_as_float((uint32_t)x[k] << 16);
            s = fmaf(v, v, s);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) a.inv_rms[row] = 1.0f / sqrtf(s / (float)a.D + a.eps);
}

// ------------------------------------------------------------------ tiled GEMM

constexpr int kBK = 64;            // K per LDS stage
constexpr int kLdsK = kBK + 8;     // padded LDS row, bf16 elements (144 B)

template <int BM, int BN, int WM, int WN, int GM>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs g) {
    static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
    constexpr int MT = WM / 16, NT = WN / 16;
    constexpr int A_LOADS = BM * (kBK / 8) / 256;  // 16-byte pieces per thread per stage
    constexpr int W_LOADS = BN * (kBK / 8) / 256;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kLdsK];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * kLdsK];

    const int tiles_m = (int)((g.M + BM - 1) / BM), tiles_n = (int)((g.N + BN - 1) / BN);
    const int nwg = tiles_m * tiles_n;
    int id = blockIdx.x;
    if (nwg % 8 == 0) id = (id % 8) * (nwg / 8) + id / 8;  // contiguous tile range per XCD
    const int group = id / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = (tiles_m - first_m < GM) ? tiles_m - first_m : GM;
    const int in_group = id - group * GM * tiles_n;
    const int tm = first_m + in_group % gm, tn = in_group / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int wm = w % (BM / WM), wn = w / (BM / WM);

    // global -> register staging: piece p of a stage covers row p/8, 8 k-values at (p%8)*8
    uint4 ra[A_LOADS], rw[W_LOADS];
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);
    auto load_stage = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int p = tid + i * 256, r = p / 8, kk = (p % 8) * 8;
            const int64_t row = m0 + r;
            ra[i] = row < g.M ? *reinterpret_cast<const uint4 *>(A + row * g.lda + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) {
            const int p = tid + i * 256, r = p / 8, kk = (p % 8) * 8;
            const int64_t row = n0 + r;
            rw[i] = row < g.N ? *reinterpret_cast<const uint4 *>(W + row * g.ldw + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int p = tid + i * 256;
            *reinterpret_cast<uint4 *>(&As[buf][(p / 8) * kLdsK + (p % 8) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) {
            const int p = tid + i * 256;
            *reinterpret_cast<uint4 *>(&Ws[buf][(p / 8) * kLdsK + (p % 8) * 8]) = rw[i];
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)(g.K / kBK);
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kb = 0; kb < nk; ++kb) {
        const int buf = kb & 1;
        if (kb + 1 < nk) load_stage((int64_t)(kb + 1) * kBK);
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int ko = ks * 32 + 8 * (lane / 16);
            uint4 af[MT], bf[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                af[i] = *reinterpret_cast<const uint4 *>(&As[buf][(wm * WM + i * 16 + lane % 16) * kLdsK + ko]);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                bf[j] = *reinterpret_cast<const uint4 *>(&Ws[buf][(wn * WN + j * 16 + lane % 16) * kLdsK + ko]);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
        }
        if (kb + 1 < nk) store_stage(buf ^ 1);
        __syncthreads();
    }

    // epilogue: C-tile lane l holds rows 4*(l/16)..+3, column l%16
    uint16_t *C = static_cast<uint16_t *>(g.C);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane / 16) + r;
            if (row >= g.M) continue;
            const float sc = g.row_scale ? g.row_scale[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t col = n0 + wn * WN + j * 16 + lane % 16;
                if (col < g.N) C[row * g.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r] * sc);
            }
        }
    }
}

// ------------------------------------------------------------------ skinny GEMM

// Workgroup: KW waves, all M (<= 64) rows x BN columns.  Wave w accumulates the
// K range [w*K/KW, (w+1)*K/KW) with fragments loaded straight from memory, then
// the partial tiles are summed through LDS.
template <int BN, int KW>
__global__ __launch_bounds__(KW * 64) void gemm_skinny_kernel(GemmArgs g) {
    constexpr int NT = BN / 16;
    constexpr int UK = 4;  // 32-wide k steps per unrolled batch of loads
    __shared__ float part[KW][64 * BN];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t kspan = g.K / KW, kbeg = (int64_t)w * kspan;
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);
    const int ko = 8 * (lane / 16);

    f32x4 acc[4][NT];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t k = kbeg; k < kbeg + kspan; k += 32 * UK) {
        uint4 af[UK][4], bf[UK][NT];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = i * 16 + lane % 16;
                af[u][i] = row < g.M ? *reinterpret_cast<const uint4 *>(A + row * g.lda + k + 32 * u + ko)
                                     : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t col = n0 + j * 16 + lane % 16;
                bf[u][j] = col < g.N ? *reinterpret_cast<const uint4 *>(W + col * g.ldw + k + 32 * u + ko)
                                     : make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < UK; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[i][j] = mfma16(af[u][i], bf[u][j], acc[i][j]);
    }
    // partial tile of this wave -> LDS [row][col]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                part[w][(i * 16 + 4 * (lane / 16) + r) * BN + j * 16 + lane % 16] = acc[i][j][r];
    __syncthreads();
    uint16_t *C = static_cast<uint16_t *>(g.C);
    for (int e = threadIdx.x; e < 64 * BN; e += KW * 64) {
        const int row = e / BN, col = e % BN;
        if (row >= g.M || n0 + col >= g.N) continue;
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < KW; ++q) s += part[q][e];
        const float sc = g.row_scale ? g.row_scale[row] : 1.0f;
        C[row * g.ldc + n0 + col] = (uint16_t)f32_to_bf16(s * sc);
    }
}

template <int BM, int BN, int WM, int WN, int GM>
hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
    const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    gemm_tiled_kernel<BM, BN, WM, WN, GM><<<dim3((unsigned)tiles), dim3(256), 0, stream>>>(g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_row_rms(const RmsArgs &a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    row_rms_kernel<<<dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    if (g.M <= 64 && g.K % (8 * 32 * 4) == 0) {
        const int64_t bn = (g.N >= 4096) ? 32 : 16;
        if (bn == 32)
            gemm_skinny_kernel<32, 8><<<dim3((unsigned)((g.N + 31) / 32)), dim3(512), 0, stream>>>(g);
        else
            gemm_skinny_kernel<16, 8><<<dim3((unsigned)((g.N + 15) / 16)), dim3(512), 0, stream>>>(g);
        return hipGetLastError();
    }
    return launch_tiled<128, 256, 64, 128, 4>(g, stream);
}

}  // namespace hm
