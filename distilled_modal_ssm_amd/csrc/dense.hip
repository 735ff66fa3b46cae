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
// GEMM kernels (the split-K pair for M <= 64 is described with its code):
//   * gemm_tiled  (large M): workgroups on a BM x BN tile, K staged 64 at a
//     time through double-buffered LDS (rows padded to 144 B so the 16-lane
//     fragment reads hit distinct banks), (BM/WM) x (BN/WN) waves each owning a
//     WM x WN sub-tile of 16x16x32 MFMAs.  Tiles are ordered so each XCD walks
//     a contiguous range, grouped GM m-tiles at a time, to keep A and W in L2.
//   * gemm_stream_lds / gemm_skinny (M <= 64, the generation step).
//     gemm_stream_lds (K = 2048): a workgroup owns 16-48 columns and all 64
//     rows or one 32-row half (the two halves of a tile on one XCD, sharing
//     its weights through L2); it loads A and W as 128-byte row pieces a few
//     chunks ahead and stages them per wave through LDS, its K loop unrolled.
//     gemm_skinny: a workgroup owns 16 columns and all rows, contiguous A and
//     W slabs through double-buffered LDS.  Both sum their K parts through
//     LDS.  Every workgroup re-reads its rows of A, so these are bound by
//     L1->L2 request throughput as much as by the W stream.
//   * gemm_stream_dl (the generation step's out_proj: M in (32, 64], no fused
//     RMS): the 32-row, 16-column workgroups of gemm_stream_lds with K staged
//     by direct global -> LDS loads into wave-private chunk buffers.
//   * the fused generation step of a layer: gemm_stream_lds on in_proj
//     weights packed so a 48-column tile is q, k, v of 16 channels, whose
//     epilogue runs the modal decode step for them instead of storing C.
#include "hm_internal.hpp"

#include <type_traits>

namespace hm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const uint4 a, const uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1 in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Row sums of squares come from one extra MFMA per A fragment: the diagonal of
// A_tile A_tile^T is sum_k a[row][k]^2.  In a 16x16 C tile lane l holds rows
// 4*(l/16)..+3 of column l%16, so diagonal entry q sits in lane 16*(q/4) + q,
// register q % 4.  diag_of returns it for the lanes that hold one (others: 0)
// together with its row q.
__device__ __forceinline__ float diag_of(const f32x4 c, int lane, int &q) {
    q = lane % 16;
    const int r = q - 4 * (lane / 16);
    return (r >= 0 && r < 4) ? c[r] : 0.f;
}

__device__ __forceinline__ float rms_scale(float sumsq, int64_t K, float eps) {
    return 1.0f / sqrtf(sumsq / (float)K + eps);
}

// ------------------------------------------------------------------ RMS

// One wave per row; lanes stride over the row in 16-byte (8 x bf16) pieces,
// four pieces in flight per lane (a 2048-wide row in one round trip: with one
// piece at a time, measured on MI355X at M = 131072, D = 2048, the pass was
// bound by load latency).
__global__ __launch_bounds__(256) void row_rms_kernel(RmsArgs a) {
    const int64_t row = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (row >= a.M) return;
    const uint16_t *x = static_cast<const uint16_t *>(a.x) + row * a.ld;
    float s = 0.f;
    if (a.vec) {
#pragma unroll 4
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

template <int BM, int BN, int WM, int WN, int GM, bool RMS>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_tiled_kernel(GemmArgs g) {
    constexpr int NTHR = (BM / WM) * (BN / WN) * 64;
    constexpr int MT = WM / 16, NT = WN / 16;
    constexpr int A_LOADS = BM * (kBK / 8) / NTHR;  // 16-byte pieces per thread per stage
    constexpr int W_LOADS = BN * (kBK / 8) / NTHR;
    static_assert(A_LOADS * NTHR == BM * (kBK / 8) && W_LOADS * NTHR == BN * (kBK / 8), "staging");
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
            const int p = tid + i * NTHR, r = p / 8, kk = (p % 8) * 8;
            const int64_t row = m0 + r;
            ra[i] = row < g.M ? *reinterpret_cast<const uint4 *>(A + row * g.lda + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) {
            const int p = tid + i * NTHR, r = p / 8, kk = (p % 8) * 8;
            const int64_t row = n0 + r;
            rw[i] = row < g.N ? *reinterpret_cast<const uint4 *>(W + row * g.ldw + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int p = tid + i * NTHR;
            *reinterpret_cast<uint4 *>(&As[buf][(p / 8) * kLdsK + (p % 8) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < W_LOADS; ++i) {
            const int p = tid + i * NTHR;
            *reinterpret_cast<uint4 *>(&Ws[buf][(p / 8) * kLdsK + (p % 8) * 8]) = rw[i];
        }
    };

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // row sums of squares from the A pieces this thread stages (row p/8 of piece i)
    float ssq[RMS ? A_LOADS : 1];
#pragma unroll
    for (int i = 0; i < (RMS ? A_LOADS : 1); ++i) ssq[i] = 0.f;
    auto accumulate_squares = [&]() {
        if constexpr (RMS) {
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i) {
                const uint32_t wv[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_lo(wv[e]), hi = bf16_hi(wv[e]);
                    ssq[i] = fmaf(lo, lo, fmaf(hi, hi, ssq[i]));
                }
            }
        }
    };

    const int nk = (int)(g.K / kBK);
    load_stage(0);
    accumulate_squares();
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
        if (kb + 1 < nk) {
            accumulate_squares();
            store_stage(buf ^ 1);
        }
        __syncthreads();
    }
    // per-row scale: the 8 consecutive lanes that staged a row sum their parts
    __shared__ float rs[RMS ? BM : 1];
    if constexpr (RMS) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            float v = ssq[i];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            if ((tid & 7) == 0) rs[(tid + i * NTHR) / 8] = rms_scale(v, g.K, g.rms_eps);
        }
        __syncthreads();
    }

    // epilogue: C-tile lane l holds rows 4*(l/16)..+3, column l%16.  The row
    // scales are all loaded before the first store (the vector memory counter
    // counts stores and loads in order: a load between the stores would wait
    // for every store before it).
    float rsc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane / 16) + r;
            rsc[i][r] = (g.row_scale && row < g.M) ? g.row_scale[row] : 1.0f;
        }
    uint16_t *C = static_cast<uint16_t *>(g.C);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane / 16) + r;
            if (row >= g.M) continue;
            float sc = rsc[i][r];
            if constexpr (RMS) sc *= rs[wm * WM + i * 16 + 4 * (lane / 16) + r];
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t col = n0 + wn * WN + j * 16 + lane % 16;
                if (col < g.N) C[row * g.ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r] * sc);
            }
        }
    }
}

// ------------------------------------------------------------------ prompt GEMM, direct loads

// 256 x 256 tile, 8 waves of 64 x 128 (two per SIMD), K staged 32 at a time by
// direct global -> LDS loads into four stage buffers, each stage's loads issued
// four stages before its products: no staging registers and no LDS store
// instructions.  LDS rows are 64 bytes
// (32 bf16) with the 16-byte chunks XOR-swizzled by row / 2 ^ row / 8, so a
// fragment read (16 rows, one chunk each) covers all banks in every 8 lanes
// (128 bytes) and in all 16 (256 bytes).  The K loop is unrolled at compile
// time (NK stages) and each buffer is its own array, so every wait names
// exactly the loads it needs.  The workgroup barrier is a bare s_barrier after
// an explicit wait for the next stage's loads only (a __syncthreads would also
// wait for the loads of the stages further ahead).  Each stage's A fragments
// are read right after that barrier, before the previous stage's products;
// the B fragments of column tile j are re-read as soon as the products that
// use them are issued.  No fused RMS: with the sums of squares the kernel
// spills; a separate row pass (hyena_row_rms) plus the row scale is faster.
__device__ __forceinline__ int dl_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <int NK>
__global__ __launch_bounds__(512) void gemm_dl8_kernel(GemmArgs g) {
    constexpr int BM = 256, BN = 256, BK = 32, NB = 4;
    __shared__ __attribute__((aligned(16))) uint16_t A0[BM * BK], A1[BM * BK], A2[BM * BK], A3[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t W0[BN * BK], W1[BN * BK], W2[BN * BK], W3[BN * BK];

    const int tiles_m = (int)(g.M / BM), tiles_n = (int)(g.N / BN);
    const int nwg = tiles_m * tiles_n;
    constexpr int GM = 4;
    int id = blockIdx.x;
    if (nwg % 8 == 0) id = (id % 8) * (nwg / 8) + id / 8;  // contiguous tile range per XCD
    const int group = id / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = (tiles_m - first_m < GM) ? tiles_m - first_m : GM;
    const int in_group = id - group * GM * tiles_n;
    const int tm = first_m + in_group % gm, tn = in_group / gm;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = w % 4, wn = w / 4;  // the wave's 64 x 128 sub-tile
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);

    // direct loads: wave w stages row blocks 2 w and 2 w + 1 (16 rows each) of A and of W
    uint32_t offa[2], offw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int lr = 16 * (2 * w + h) + lane / 4;
        const int lc = (lane % 4) ^ dl_swz(lr);
        offa[h] = (uint32_t)(lr * g.lda + 8 * lc) * 2u;
        offw[h] = (uint32_t)(lr * g.ldw + 8 * lc) * 2u;
    }
    const char *Ab = reinterpret_cast<const char *>(A + m0 * g.lda);
    const char *Wb = reinterpret_cast<const char *>(W + n0 * g.ldw);
    auto bufs = [&](auto bc) {
        constexpr int b = decltype(bc)::value;
        uint16_t *a = b == 0 ? A0 : b == 1 ? A1 : b == 2 ? A2 : A3;
        uint16_t *ww = b == 0 ? W0 : b == 1 ? W1 : b == 2 ? W2 : W3;
        return std::make_pair(a, ww);
    };
    auto issue = [&](auto sc) {
        constexpr int st = decltype(sc)::value;
        const auto [as, ws] = bufs(std::integral_constant<int, st % NB>{});
        const int64_t k0 = (int64_t)st * BK;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(Ab + 2 * k0 + offa[h]),
                                             &as[16 * (2 * w + h) * BK], 16, 0, 0);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(Wb + 2 * k0 + offw[h]),
                                             &ws[16 * (2 * w + h) * BK], 16, 0, 0);
        }
    };
    auto frag = [&](const uint16_t *buf, int row0) {
        const int r = row0 + lane % 16, c = lane / 16;
        return *reinterpret_cast<const uint4 *>(&buf[r * BK + 8 * (c ^ dl_swz(r))]);
    };
    // A fragments double-buffered; B fragments single: column tile j's read for
    // the next stage follows the products that use tile j of this one
    uint4 af[2][4], bf[8];
    auto read_a = [&](auto sc) {
        constexpr int st = decltype(sc)::value;
        const auto [as, ws] = bufs(std::integral_constant<int, st % NB>{});
#pragma unroll
        for (int i = 0; i < 4; ++i) af[st % 2][i] = frag(as, 64 * wm + 16 * i);
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The products are taken with the W fragment as the first operand, so the
    // C tiles are held transposed: lane l holds row 16 i + l % 16 of the wave's
    // tile, columns 16 j + 4 (l / 16) .. + 3, four adjacent outputs that leave
    // as one 8-byte piece.  The row scales of the lane's 4 rows are loaded
    // during the last stage's products, before any output store (the vector
    // memory counter counts stores and loads in order: a scale loaded between
    // the stores would wait for every store issued before it).
    float rsc[4];
    auto load_scales = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) rsc[i] = g.row_scale ? g.row_scale[m0 + 64 * wm + 16 * i + lane % 16] : 1.0f;
    };

    // The stage barrier: this wave's wait (an s_waitcnt immediate: vmcnt in
    // bits 3:0, expcnt 6:4, lgkmcnt 11:8), then a bare s_barrier.  The signal
    // fences keep the compiler from moving LDS accesses across it (the barrier
    // builtin itself is not a memory operation to the compiler), the
    // scheduling barriers keep the machine scheduler from doing so.
    auto stage_barrier = [&](auto wc) {
        constexpr int wait = decltype(wc)::value;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    // stages in flight before stage st's barrier: up to st + NB - 1; the
    // barrier needs stage st + 1's loads (read right after it)
    static_for<0, (NK < NB ? NK : NB)>([&](auto sc) { issue(sc); });
    {
        constexpr int later = (NK < NB ? NK : NB) - 1;  // stages issued after stage 0
        stage_barrier(std::integral_constant<int, (4 * later) | (0x7 << 4)>{});
    }
    read_a(std::integral_constant<int, 0>{});
    {
        const auto [as, ws] = bufs(std::integral_constant<int, 0>{});
#pragma unroll
        for (int j = 0; j < 8; ++j) bf[j] = frag(ws, 128 * wn + 16 * j);
    }
    static_for<0, NK>([&](auto sc) {
        constexpr int st = decltype(sc)::value;
        if constexpr (st + 1 < NK) {
            // issued so far: stages .. min(st + NB - 1, NK - 1); wait for st + 1
            constexpr int last = (st + NB - 1 < NK - 1) ? st + NB - 1 : NK - 1;
            constexpr int after = last - (st + 1);
            stage_barrier(std::integral_constant<int, (4 * after) | (0x7 << 4)>{});  // vmcnt(4 after), lgkmcnt(0)
            if constexpr (st + NB < NK) issue(std::integral_constant<int, st + NB>{});
            read_a(std::integral_constant<int, st + 1>{});
        }
        const auto [nas, nws] = bufs(std::integral_constant<int, (st + 1) % NB>{});
        if constexpr (st + 1 == NK) load_scales();
        // a wave in its products outranks the other wave of its SIMD in the
        // barrier, load-issue and fragment-read part of a stage (measured on
        // MI355X, M = 131072, K = 2048: in_proj 2.87 -> 2.79 ms, out_proj
        // 1.01 -> 0.99 ms)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i][j] = mfma16(bf[j], af[st % 2][i], acc[i][j]);
            if constexpr (st + 1 < NK) bf[j] = frag(nws, 128 * wn + 16 * j);
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    });
    // Epilogue through LDS: each wave writes its 64 x 128 bf16 tile (16 KB)
    // into one of the eight stage arrays as 8-byte pieces, then reads it back
    // as whole 16-byte chunks, so each store instruction writes four complete
    // 256-byte row segments of C (2-byte stores of the MFMA layout wrote four
    // 32-byte pieces per instruction).  A row of the staged tile is 256 bytes,
    // sixteen 16-byte chunks, with chunk c stored at c ^ (row % 16): the
    // sixteen rows one piece-write instruction touches then fall on distinct
    // banks.  Each wave reads only what it wrote (its LDS operations complete
    // in order), so one barrier -- every wave done with the stage buffers --
    // is all the epilogue needs.
    __syncthreads();
    uint16_t *ob = w == 0 ? A0 : w == 1 ? A1 : w == 2 ? A2 : w == 3 ? A3 : w == 4 ? W0 : w == 5 ? W1 : w == 6 ? W2 : W3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * i + lane % 16;
        const float sc = rsc[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int chunk = 2 * j + (lane / 16) / 2;  // 16-byte chunk of the row holding the piece
            const uint2 piece = make_uint2(pack_bf16x2(acc[i][j][0] * sc, acc[i][j][1] * sc),
                                           pack_bf16x2(acc[i][j][2] * sc, acc[i][j][3] * sc));
            *reinterpret_cast<uint2 *>(&ob[row * 128 + 8 * (chunk ^ (row % 16)) + 4 * ((lane / 16) % 2)]) = piece;
        }
    }
    uint16_t *C = static_cast<uint16_t *>(g.C) + (m0 + 64 * wm) * g.ldc + n0 + 128 * wn;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int row = 4 * t + lane / 16, chunk = lane % 16;
        const uint4 v = *reinterpret_cast<const uint4 *>(&ob[row * 128 + 8 * (chunk ^ (row % 16))]);
        *reinterpret_cast<uint4 *>(C + (int64_t)row * g.ldc + 8 * chunk) = v;
    }
}

// ------------------------------------------------------------------ skinny GEMM

// Workgroup = 4 waves on all M <= 64 rows x BN columns.  K advances in slabs of
// kSkCK: the A slab [64][kSkCK] and the W slab [BN][kSkCK] are read with
// contiguous 16-byte pieces (whole 512-byte row runs, which HBM streams
// efficiently) into registers one slab ahead, then written to double-buffered
// LDS.  Wave w owns column tile w % NTB and K half-range w / NTB of the slab
// (NTB = BN / 16 column tiles, 4 / NTB K parts); the K parts are summed
// through LDS at the end.
constexpr int kSkCK = 256;            // K per slab
constexpr int kSkLd = kSkCK + 8;      // padded LDS row (bf16), 528 B

template <int BN, bool RMS>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmArgs g) {
    constexpr int NTB = BN / 16;          // column tiles
    constexpr int KP = 4 / NTB;           // K parts per slab
    constexpr int KPS = kSkCK / KP / 32;  // 32-wide k steps per wave per slab
    constexpr int A_P = 64 * (kSkCK / 8) / 256;  // 16-byte pieces per thread
    constexpr int W_P = BN * (kSkCK / 8) / 256;
    static_assert(NTB * KP == 4 && A_P * 256 == 64 * (kSkCK / 8) && W_P * 256 == BN * (kSkCK / 8), "shape");
    __shared__ __attribute__((aligned(16))) uint16_t As[2][64 * kSkLd];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * kSkLd];

    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int nt = w % NTB, kp = w / NTB;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);

    uint4 ra[A_P], rw[W_P];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < A_P; ++i) {
            const int p = tid + i * 256, r = p / (kSkCK / 8), kk = (p % (kSkCK / 8)) * 8;
            ra[i] = r < g.M ? *reinterpret_cast<const uint4 *>(A + r * g.lda + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W_P; ++i) {
            const int p = tid + i * 256, r = p / (kSkCK / 8), kk = (p % (kSkCK / 8)) * 8;
            const int64_t row = n0 + r;
            rw[i] = row < g.N ? *reinterpret_cast<const uint4 *>(W + row * g.ldw + k0 + kk) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_P; ++i) {
            const int p = tid + i * 256;
            *reinterpret_cast<uint4 *>(&As[buf][(p / (kSkCK / 8)) * kSkLd + (p % (kSkCK / 8)) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < W_P; ++i) {
            const int p = tid + i * 256;
            *reinterpret_cast<uint4 *>(&Ws[buf][(p / (kSkCK / 8)) * kSkLd + (p % (kSkCK / 8)) * 8]) = rw[i];
        }
    };

    f32x4 acc[4], ss[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = ss[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ns = (int)(g.K / kSkCK);
    load(0);
    store(0);
    __syncthreads();
    for (int sl = 0; sl < ns; ++sl) {
        const int buf = sl & 1;
        if (sl + 1 < ns) load((int64_t)(sl + 1) * kSkCK);
#pragma unroll
        for (int st = 0; st < KPS; ++st) {
            const int ko = (kp * KPS + st) * 32 + 8 * (lane / 16);
            const uint4 bf = *reinterpret_cast<const uint4 *>(&Ws[buf][(nt * 16 + lane % 16) * kSkLd + ko]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint4 af = *reinterpret_cast<const uint4 *>(&As[buf][(m * 16 + lane % 16) * kSkLd + ko]);
                acc[m] = mfma16(af, bf, acc[m]);
                if constexpr (RMS) {
                    if (nt == 0) ss[m] = mfma16(af, af, ss[m]);  // one column tile per K part is enough
                }
            }
        }
        if (sl + 1 < ns) store(buf ^ 1);
        __syncthreads();
    }

    // sum the K parts: C-tile lane l holds rows 16m + 4*(l/16) + r, column l%16
    float *red = reinterpret_cast<float *>(&As[0][0]);  // [KP][64][BN] floats fit in one A buffer
    float *red_ss = reinterpret_cast<float *>(&Ws[0][0]);  // [KP][64]
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(kp * 64 + m * 16 + 4 * (lane / 16) + r) * BN + nt * 16 + lane % 16] = acc[m][r];
    if constexpr (RMS) {
        if (nt == 0) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                int q;
                const float dg = diag_of(ss[m], lane, q);
                if (4 * (lane / 16) <= q && q < 4 * (lane / 16) + 4) red_ss[kp * 64 + m * 16 + q] = dg;
            }
        }
    }
    __syncthreads();
    uint16_t *C = static_cast<uint16_t *>(g.C);
    for (int e = tid; e < 64 * BN; e += 256) {
        const int row = e / BN, c = e % BN;
        const int64_t col = n0 + c;
        if (row >= g.M || col >= g.N) continue;
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < KP; ++q) sum += red[(q * 64 + row) * BN + c];
        float sc = g.row_scale ? g.row_scale[row] : 1.0f;
        if constexpr (RMS) {
            float s2 = 0.f;
#pragma unroll
            for (int q = 0; q < KP; ++q) s2 += red_ss[q * 64 + row];
            sc *= rms_scale(s2, g.K, g.rms_eps);
        }
        C[row * g.ldc + col] = (uint16_t)f32_to_bf16(sum * sc);
    }
}

// Weight-streaming GEMM for M <= 64 and K = 2048 (K loop fully unrolled).
// Workgroup = 4 waves on MR rows (64, or 32 = one half of the rows) x BN =
// 16 NTW columns; wave w takes K quarter w (8 chunks of 64).  Both operands are loaded as 128-byte row pieces
// (8 lanes per row, 8 rows per load instruction) -- measured on MI355X,
// fragment-shaped loads (64 bytes of 16 rows per instruction) stream W 15-40 %
// slower and double the requests for A, which every workgroup re-reads --
// into registers (A two chunks ahead, W SW chunks ahead), then written to
// wave-private LDS buffers (rows padded to 144 B) and read back as MFMA
// fragments.  The buffers are private to the wave, so no workgroup barrier is
// needed inside the K loop (LDS operations of one wave complete in order).
// The loop is unrolled at compile time, so every wait names exactly the load
// it needs.  The four K quarters are summed through LDS, reusing the A buffers.
constexpr int kAsLd = 72;  // bf16 per LDS row of the A chunk (64 + 8 pad)

// FDL > 0: the fused decode epilogue (d = FDL modes); FDL < 0: the gate
// epilogue of the deferred state, y = q (D u + rho), u_prev <- u.  PDD > 0: the
// workgroup has 8 waves, and waves 4..7 run the prepare of g.prep (d = PDD)
// while waves 0..3 stream the product: their loads wait on their own
// counters, so the state stream does not hold up the K loop.
template <int NTW, int SW, bool RMS, int MR, int FDL = 0, int PDD = 0>
__global__ __launch_bounds__(PDD > 0 ? 512 : 256) void gemm_stream_lds_kernel(GemmArgs g) {
    constexpr int MT = MR / 16, AL = MR / 8;  // m-tiles; A row-piece loads per chunk
    constexpr int BN = 16 * NTW, NCH = 8;  // K quarter: 8 chunks of 64
    constexpr int WPL = BN / 8;            // W row pieces per lane per chunk (8 rows per load)
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) uint16_t as[4][2][MR * kAsLd];
    __shared__ __attribute__((aligned(16))) uint16_t wsm[4][2][BN * kAsLd];
    __shared__ float red_ss[RMS ? 4 * MR : 1];
    static_assert(4 * MR * BN * sizeof(float) <= sizeof(as), "the K-part sums reuse the A buffers");
    __shared__ unsigned arrivals;  // product waves past each epilogue sync point (PDD > 0)
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    // MR = 32: the two row halves of a column tile sit 8 workgroups apart, on one XCD
    int64_t tile = blockIdx.x, m0 = 0;
    bool active = true;
    if constexpr (MR == 32) {
        const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
        m0 = 32 * (slot % 2);
        tile = (slot / 2) * 8 + xcd;
        active = !(tile * BN >= g.N || m0 >= g.M);
    }
    if constexpr (PDD > 0) {
        // Prepare waves: units of two channels, striding over the grid.  They
        // take no part in the product and end here (readfirstlane makes the
        // exit a wave-uniform branch).  A barrier counts every wave of the
        // workgroup that has not ended, so a barrier in the epilogue would wait
        // until the prepare waves end (measured on MI355X, B = 64, D = 2048,
        // d = 16: 2.2 us); the product waves synchronise through an LDS arrival
        // count instead (gemm_sync below).  The barrier here, before any wave
        // leaves, orders the count's initialisation.
        if (tid == 0) arrivals = 0;
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(w) >= 4) {
            const int64_t units = g.prep.B * (g.prep.D / 2);
            for (int64_t u = (int64_t)blockIdx.x * 256 + (tid - 256); u < units; u += (int64_t)gridDim.x * 256)
                prepare_unit<PDD>(g.prep, u);
            return;
        }
    }
    if (!active) return;  // the whole workgroup: no barrier is left behind
    const bool gemm_wave = (PDD == 0) || w < 4;
    const int64_t n0 = tile * BN;
    const int64_t kbeg = (int64_t)w * NCH * 64;
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);
    const int ko = 8 * (lane / 16);
    // row piece of lane l in a load: row 8 i + l / 8, 16-byte piece l % 8 of the chunk's 128 bytes
    const int prow = lane / 8, ppiece = lane % 8;
    const uint16_t *arow[AL], *wrow[WPL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
        const int64_t r = m0 + 8 * i + prow;
        arow[i] = A + (r < g.M ? r : 0) * g.lda + kbeg + 8 * ppiece;  // clamped rows are masked at the end
    }
#pragma unroll
    for (int i = 0; i < WPL; ++i) {
        const int64_t c = n0 + 8 * i + prow;
        wrow[i] = W + (c < g.N ? c : 0) * g.ldw + kbeg + 8 * ppiece;  // clamped columns are masked at the end
    }
    // A two chunks ahead, W SW chunks ahead, in registers (native vectors, so
    // they stay in registers); every index below is a compile-time constant
    u32x4 ra[2][AL], rw[SW][WPL];
    auto load_a = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
#pragma unroll
        for (int i = 0; i < AL; ++i) ra[c % 2][i] = *reinterpret_cast<const u32x4 *>(arow[i] + 64 * c);
    };
    auto load_w = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
#pragma unroll
        for (int i = 0; i < WPL; ++i) {
            // non-temporal for the 32-column form (measured on MI355X, 24 cold weights:
            // N = 6144 11.45 -> 11.02 us); the 16-column form measured slower with it
            // (N = 2048: 6.35 -> 7.85 us)
            const u32x4 *pw = reinterpret_cast<const u32x4 *>(wrow[i] + 64 * c);
            if constexpr (NTW >= 2)
                rw[c % SW][i] = __builtin_nontemporal_load(pw);
            else
                rw[c % SW][i] = *pw;
        }
    };
    // Fused decode step (FDL modes): thread = (row dr of the half, channel pair
    // dcp of the tile's 16 channels).  Its state is loaded only once the K loop
    // is done: loads retire in order, so state loads issued earlier would hold
    // up every later chunk wait (measured on MI355X, B = 64, D = 2048, d = 16:
    // 19.9 us with the loads at kernel start, 18.1 us at the epilogue).
    static_assert(FDL == 0 || (NTW == 3 && MR == 32 && RMS), "fused step: 48 columns = q, k, v of 16 channels");
    static_assert(PDD == 0 || (FDL < 0 && NTW == 3 && MR == 32 && RMS), "prepare waves ride with the gate");
    const int dr = tid / 8, dcp = tid % 8;
    const int64_t db = m0 + dr, dc = tile * 16 + 2 * dcp;
    const int64_t dg = FDL ? dc / g.P : 0;
    float2 *dst = nullptr;
    f32x4 xs[FDL > 0 ? FDL : 1];
    if constexpr (FDL > 0) {
        if (db < g.M) dst = g.state + ((db * g.H + dg) * FDL) * g.P + (dc - dg * g.P);
    }
    auto load_state = [&]() {
        if constexpr (FDL > 0) {
            if (db < g.M) {
#pragma unroll
                for (int n = 0; n < FDL; ++n) xs[n] = *reinterpret_cast<const f32x4 *>(dst + n * g.P);
            }
        }
    };
    f32x4 acc[MT][NTW], ss[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        ss[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NTW; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (gemm_wave) {
        static_for<0, SW>([&](auto cc) { load_w(cc); });
        static_for<0, 2>([&](auto cc) { load_a(cc); });
        __builtin_amdgcn_sched_barrier(0);
        // chunk c: its A and W pieces go to the wave's LDS buffers c % 2 (the
        // wave's LDS operations complete in order, so chunk c - 2's fragment reads
        // of those buffers are done), the loads for chunks c + 2 (A) and c + SW (W)
        // are issued into the freed registers, then two 32-wide MFMA steps
        static_for<0, NCH>([&](auto cc) {
            constexpr int c = decltype(cc)::value, buf = c % 2;
#pragma unroll
            for (int i = 0; i < AL; ++i)
                *reinterpret_cast<u32x4 *>(&as[w][buf][(8 * i + prow) * kAsLd + 8 * ppiece]) = ra[buf][i];
#pragma unroll
            for (int i = 0; i < WPL; ++i)
                *reinterpret_cast<u32x4 *>(&wsm[w][buf][(8 * i + prow) * kAsLd + 8 * ppiece]) = rw[c % SW][i];
            if constexpr (c + 2 < NCH) load_a(std::integral_constant<int, c + 2>{});
            if constexpr (c + SW < NCH) load_w(std::integral_constant<int, c + SW>{});
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint4 a[MT], b[NTW];
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    a[m] = *reinterpret_cast<const uint4 *>(&as[w][buf][(16 * m + lane % 16) * kAsLd + 32 * h + ko]);
#pragma unroll
                for (int j = 0; j < NTW; ++j)
                    b[j] = *reinterpret_cast<const uint4 *>(&wsm[w][buf][(16 * j + lane % 16) * kAsLd + 32 * h + ko]);
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int j = 0; j < NTW; ++j) acc[m][j] = mfma16(a[m], b[j], acc[m][j]);
                if constexpr (RMS) {
#pragma unroll
                    for (int m = 0; m < MT; ++m) ss[m] = mfma16(a[m], a[m], ss[m]);
                }
            }
        });
        if constexpr (RMS) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                int q;
                const float dg = diag_of(ss[m], lane, q);
                if (4 * (lane / 16) <= q && q < 4 * (lane / 16) + 4) red_ss[w * MR + m * 16 + q] = dg;
            }
        }
    }
    // Workgroup sync of the product waves.  With prepare waves (PDD > 0) it is
    // an LDS arrival count: lane 0 of each of the four product waves adds one
    // (release), then the wave waits for the count to reach `target` (acquire).
    // The four product waves of an active workgroup all reach both sync points.
    auto gemm_sync = [&](unsigned target) {
        if constexpr (PDD > 0) {
            if (lane == 0) __hip_atomic_fetch_add(&arrivals, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            while (__hip_atomic_load(&arrivals, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
                __builtin_amdgcn_s_sleep(1);
        } else {
            __syncthreads();
        }
    };
    load_state();
    gemm_sync(4);  // every wave is done with its A buffers, which now hold the K-part sums
    float *red = reinterpret_cast<float *>(&as[0][0][0]);
    if (gemm_wave) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int j = 0; j < NTW; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red[(w * MR + m * 16 + 4 * (lane / 16) + r) * BN + j * 16 + lane % 16] = acc[m][j][r];
    }
    gemm_sync(8);
    if constexpr (FDL != 0) {
        // Each thread's row dr and two channels: q, k, v straight from the
        // K-part sums, rounded to bf16 exactly as the projection stores them
        // (one inverse RMS per thread, all LDS reads in flight together; a
        // staging pass over the tile with a scale per element took 1.5 us of
        // the launch on MI355X), then the gate or the decode step.
        if (tid >= 256 || db >= g.M) return;
        const float sc = rms_scale(red_ss[dr] + red_ss[MR + dr] + red_ss[2 * MR + dr] + red_ss[3 * MR + dr], g.K,
                                   g.rms_eps);
        float qv[6];  // q, k, v of channels dc and dc + 1
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = 16 * j + 2 * dcp + h;
                const float sum = red[(0 * MR + dr) * BN + c] + red[(1 * MR + dr) * BN + c] +
                                  red[(2 * MR + dr) * BN + c] + red[(3 * MR + dr) * BN + c];
                qv[2 * j + h] = bf16_lo(f32_to_bf16(sum * sc));
            }
        const float q0 = qv[0], q1 = qv[1];
        const float u0 = qv[2] * qv[4], u1 = qv[3] * qv[5];
        if constexpr (FDL < 0) {
            // the gate of the deferred state: y = q (D u + rho), u_prev <- u
            const int64_t ldr = g.H * g.P;
            const float2 rr = *reinterpret_cast<const float2 *>(g.rho + db * ldr + dc);
            const float Dg = g.skip[dg];
            // y with a plain store: out_proj reads it next, and a streaming store
            // sends it past the caches it is read back through (measured on
            // MI355X, 24-layer stack at batch 64: 0.5152 -> 0.5128 ms per token)
            *reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(g.y) + db * g.ld_y + dc) =
                pack_bf16x2(q0 * fmaf(Dg, u0, rr.x), q1 * fmaf(Dg, u1, rr.y));
            *reinterpret_cast<float2 *>(g.u_prev + db * ldr + dc) = make_float2(u0, u1);
            return;
        }
        // the decode step with the arithmetic of decode_step_fixed (two
        // channels per lane): y = q (D u + Re sum R x), x <- lambda x + u
        // the head's poles and residues are read before the first state store:
        // the vector memory counter counts stores and loads in order, so a load
        // issued after a store is waited for together with the store
        constexpr int NM = FDL > 0 ? FDL : 1;
        const float2 *lam = g.poles + dg * NM, *res = g.residues + dg * NM;
        float2 lv[NM], rv[NM];
#pragma unroll
        for (int n = 0; n < NM; ++n) {
            lv[n] = lam[n];
            rv[n] = res[n];
        }
        const float Dg = g.skip[dg];
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int n = 0; n < (FDL > 0 ? FDL : 0); ++n) {
            const float2 l = lv[n], r = rv[n];
            const f32x4 xo = xs[n];
            acc0 = fmaf(r.x, xo[0], acc0);
            acc0 = fmaf(-r.y, xo[1], acc0);
            acc1 = fmaf(r.x, xo[2], acc1);
            acc1 = fmaf(-r.y, xo[3], acc1);
            const f32x4 xn = {fmaf(l.x, xo[0], fmaf(-l.y, xo[1], u0)), fmaf(l.x, xo[1], l.y * xo[0]),
                              fmaf(l.x, xo[2], fmaf(-l.y, xo[3], u1)), fmaf(l.x, xo[3], l.y * xo[2])};
            __builtin_nontemporal_store(xn, reinterpret_cast<f32x4 *>(dst + n * g.P));
        }
        __builtin_nontemporal_store(pack_bf16x2(q0 * fmaf(Dg, u0, acc0), q1 * fmaf(Dg, u1, acc1)),
                                    reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(g.y) + db * g.ld_y + dc));
        return;
    }
    uint16_t *C = static_cast<uint16_t *>(g.C);
    // each thread two adjacent columns of a row, one 4-byte store where C's
    // layout allows (ldc even, C 4-byte aligned; wave-uniform)
    const bool pairs = g.ldc % 2 == 0 && reinterpret_cast<uintptr_t>(g.C) % 4 == 0;
    for (int e = tid; e < MR * BN / 2 && tid < 256; e += 256) {
        const int lr = e / (BN / 2), c = 2 * (e % (BN / 2));
        const int64_t row = m0 + lr, col = n0 + c;
        if (row >= g.M || col >= g.N) continue;
        float2 sum = make_float2(0.f, 0.f);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float2 part = *reinterpret_cast<const float2 *>(&red[(q * MR + lr) * BN + c]);
            sum.x += part.x;
            sum.y += part.y;
        }
        float sc = g.row_scale ? g.row_scale[row] : 1.0f;
        if constexpr (RMS)
            sc *= rms_scale(red_ss[lr] + red_ss[MR + lr] + red_ss[2 * MR + lr] + red_ss[3 * MR + lr], g.K, g.rms_eps);
        if (pairs && col + 1 < g.N) {
            *reinterpret_cast<uint32_t *>(&C[row * g.ldc + col]) = pack_bf16x2(sum.x * sc, sum.y * sc);
        } else {
            C[row * g.ldc + col] = (uint16_t)f32_to_bf16(sum.x * sc);
            if (col + 1 < g.N) C[row * g.ldc + col + 1] = (uint16_t)f32_to_bf16(sum.y * sc);
        }
    }
}

// out_proj-shaped streaming GEMM: M in (32, 64], K = 2048, no fused RMS; a
// workgroup owns 16 columns and one 32-row half (the two halves of a column
// tile on one XCD, as in gemm_stream_lds), wave w K quarter w in 8 chunks of
// 64.  K is staged by direct global -> LDS loads into NB wave-private chunk
// buffers, NB - 1 chunks ahead: no staging registers and no LDS stores.  A
// buffer row is 128 bytes (64 bf16), eight 16-byte pieces; piece p of row r
// sits in slot p ^ (r % 8), so the 16 rows of a fragment read spread over
// the banks.  A load instruction covers 8 rows (8 lanes per row, each lane
// the piece that belongs in its slot), and each buffer is its own array, so
// every wait names exactly the loads it needs.  The four K quarters are
// summed through LDS as in gemm_stream_lds.
template <int NB>
__global__ __launch_bounds__(256) void gemm_stream_dl_kernel(GemmArgs g) {
    constexpr int MR = 32, BN = 16, NCH = 8, LPC = MR / 8 + BN / 8;  // load instructions per chunk
    static_assert(NB >= 3 && NB <= 6, "chunk buffers");
    __shared__ __attribute__((aligned(16))) uint16_t A0[4][MR * 64], A1[4][MR * 64], A2[4][MR * 64],
        A3[NB > 3 ? 4 : 1][MR * 64], A4[NB > 4 ? 4 : 1][MR * 64], A5[NB > 5 ? 4 : 1][MR * 64];
    __shared__ __attribute__((aligned(16))) uint16_t W0[4][BN * 64], W1[4][BN * 64], W2[4][BN * 64],
        W3[NB > 3 ? 4 : 1][BN * 64], W4[NB > 4 ? 4 : 1][BN * 64], W5[NB > 5 ? 4 : 1][BN * 64];
    static_assert(4 * MR * BN * sizeof(float) <= sizeof(A0), "the K-part sums reuse the first A buffer");
    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int64_t m0 = 32 * (slot % 2), tile = (slot / 2) * 8 + xcd;
    if (tile * BN >= g.N || m0 >= g.M) return;  // the whole workgroup
    const int64_t n0 = tile * BN, kbeg = (int64_t)w * NCH * 64;
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);
    // lane l loads row 8 i + l / 8 of instruction i, the piece for slot l % 8
    const int lrow = lane / 8, lpiece = (lane % 8) ^ (lane / 8);
    const uint16_t *arow[MR / 8], *wrow[BN / 8];
#pragma unroll
    for (int i = 0; i < MR / 8; ++i) {
        const int64_t r = m0 + 8 * i + lrow;
        arow[i] = A + (r < g.M ? r : 0) * g.lda + kbeg + 8 * lpiece;  // clamped rows are masked at the end
    }
#pragma unroll
    for (int i = 0; i < BN / 8; ++i) {
        const int64_t c = n0 + 8 * i + lrow;
        wrow[i] = W + (c < g.N ? c : 0) * g.ldw + kbeg + 8 * lpiece;  // clamped columns are masked at the end
    }
    auto bufs = [&](auto bc) {
        constexpr int b = decltype(bc)::value;
        uint16_t *a = b == 0 ? A0[w] : b == 1 ? A1[w] : b == 2 ? A2[w] : b == 3 ? A3[NB > 3 ? w : 0]
                    : b == 4 ? A4[NB > 4 ? w : 0] : A5[NB > 5 ? w : 0];
        uint16_t *ww = b == 0 ? W0[w] : b == 1 ? W1[w] : b == 2 ? W2[w] : b == 3 ? W3[NB > 3 ? w : 0]
                     : b == 4 ? W4[NB > 4 ? w : 0] : W5[NB > 5 ? w : 0];
        return std::make_pair(a, ww);
    };
    auto issue = [&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const auto [ab, wb] = bufs(std::integral_constant<int, c % NB>{});
#pragma unroll
        for (int i = 0; i < MR / 8; ++i)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(arow[i] + 64 * c), &ab[8 * i * 64], 16, 0, 0);
#pragma unroll
        for (int i = 0; i < BN / 8; ++i)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(wrow[i] + 64 * c), &wb[8 * i * 64], 16, 0, 0);
    };
    auto frag = [&](const uint16_t *buf, int r, int q) {
        return *reinterpret_cast<const uint4 *>(&buf[r * 64 + 8 * (q ^ (r % 8))]);
    };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    static_for<0, NB>([&](auto cc) { issue(cc); });
    static_for<0, NCH>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        // chunks issued so far: 0 .. min(c + NB - 1, NCH - 1); wait for chunk c
        // (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8 = 0)
        constexpr int later = ((c + NB - 1 < NCH - 1) ? c + NB - 1 : NCH - 1) - c;
        constexpr int vm = LPC * later;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4));
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const auto [ab, wb] = bufs(std::integral_constant<int, c % NB>{});
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 b = frag(wb, lane % 16, 4 * h + lane / 16);
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[m] = mfma16(frag(ab, 16 * m + lane % 16, 4 * h + lane / 16), b, acc[m]);
        }
        if constexpr (c + NB < NCH) {
            // this chunk's fragment reads are done (the products above used
            // them) before its buffer takes chunk c + NB
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            issue(std::integral_constant<int, c + NB>{});
        }
    });
    __syncthreads();  // every wave is done with its buffers; the sums reuse A0
    float *red = reinterpret_cast<float *>(&A0[0][0]);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(w * MR + m * 16 + 4 * (lane / 16) + r) * BN + lane % 16] = acc[m][r];
    __syncthreads();
    uint16_t *C = static_cast<uint16_t *>(g.C);
    const bool pairs = g.ldc % 2 == 0 && reinterpret_cast<uintptr_t>(g.C) % 4 == 0;
    {
        const int e = tid;  // MR * BN / 2 = 256 pairs, one per thread
        const int lr = e / (BN / 2), c = 2 * (e % (BN / 2));
        const int64_t row = m0 + lr, col = n0 + c;
        if (row < g.M && col < g.N) {
            float2 sum = make_float2(0.f, 0.f);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 part = *reinterpret_cast<const float2 *>(&red[(q * MR + lr) * BN + c]);
                sum.x += part.x;
                sum.y += part.y;
            }
            const float sc = g.row_scale ? g.row_scale[row] : 1.0f;
            if (pairs && col + 1 < g.N) {
                *reinterpret_cast<uint32_t *>(&C[row * g.ldc + col]) = pack_bf16x2(sum.x * sc, sum.y * sc);
            } else {
                C[row * g.ldc + col] = (uint16_t)f32_to_bf16(sum.x * sc);
                if (col + 1 < g.N) C[row * g.ldc + col + 1] = (uint16_t)f32_to_bf16(sum.y * sc);
            }
        }
    }
}

// ------------------------------------------------------------------ split-K GEMM (M <= 64)

// Pass 1.  Workgroup = (64-column tile nt, 256-wide K slice sl), 4 waves; wave
// w covers k in [sl*256 + 64w, +64) for all 64 rows and 64 columns: its A and
// W fragments (16 x 16 bytes per lane) are all loaded at once, straight into
// the MFMA operand registers, so every workgroup has its whole 64 KB in
// flight.  The four waves' C tiles are summed through LDS into one fp32
// partial per (tile, slice), stored in C-fragment order, plus (fused RMS) the
// slice's row sums of squares.
template <bool RMS>
__global__ __launch_bounds__(256) void gemm_splitk_kernel(GemmArgs g, int nsl) {
    __shared__ __attribute__((aligned(16))) float red[4][16][kWave][4];  // wave, C tile, lane, register
    __shared__ float ssq_l[4][64];
    const int nt = blockIdx.x, sl = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int r16 = lane % 16, kg = lane / 16;
    const int64_t n0 = (int64_t)nt * kSplitBN, k0 = (int64_t)sl * kSplitKS + 64 * w;
    const uint16_t *A = static_cast<const uint16_t *>(g.A);
    const uint16_t *W = static_cast<const uint16_t *>(g.W);
    const int64_t tiles = (g.N + kSplitBN - 1) / kSplitBN;
    float *part = reinterpret_cast<float *>(g.ws);
    float *ssq_part = part + tiles * nsl * 4096;

    uint4 a[4][2], b[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int64_t k = k0 + 32 * ks + 8 * kg;
            const int64_t row = 16 * i + r16, col = n0 + 16 * i + r16;
            a[i][ks] = row < g.M ? *reinterpret_cast<const uint4 *>(A + row * g.lda + k) : make_uint4(0, 0, 0, 0);
            b[i][ks] = col < g.N ? *reinterpret_cast<const uint4 *>(W + col * g.ldw + k) : make_uint4(0, 0, 0, 0);
        }
    f32x4 acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = mfma16(a[mi][ks], b[nj][ks], acc[mi][nj]);
    if constexpr (RMS) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            float s = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint32_t wv[4] = {a[mi][ks].x, a[mi][ks].y, a[mi][ks].z, a[mi][ks].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_lo(wv[e]), hi = bf16_hi(wv[e]);
                    s = fmaf(lo, lo, fmaf(hi, hi, s));
                }
            }
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            if (kg == 0) ssq_l[w][16 * mi + r16] = s;
        }
    }
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj)
            *reinterpret_cast<f32x4 *>(&red[w][mi * 4 + nj][lane][0]) = acc[mi][nj];
    __syncthreads();

    // partial of this slice, C-fragment order: float4 q = tile * 64 + lane
    float *mine = part + ((int64_t)nt * nsl + sl) * 4096;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + 256 * i;
        const float *r0 = &red[0][q / kWave][q % kWave][0];
        f32x4 v = *reinterpret_cast<const f32x4 *>(r0);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) v += *reinterpret_cast<const f32x4 *>(r0 + ww * 16 * kWave * 4);
        *reinterpret_cast<f32x4 *>(mine + 4 * q) = v;
    }
    if (RMS && tid < 64)
        ssq_part[((int64_t)nt * nsl + sl) * 64 + tid] = ssq_l[0][tid] + ssq_l[1][tid] + ssq_l[2][tid] + ssq_l[3][tid];
}

// Pass 2.  Four workgroups per column tile, one float4 of the tile's C
// fragments per thread: sums the slices' partials (all loads in flight),
// scales (row scale, or the inverse RMS from the slices' sums of squares) and
// writes bf16 C.
template <bool RMS, int NSL>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
    __shared__ float scale[64];
    const int nt = blockIdx.x / 4, quarter = blockIdx.x % 4, tid = threadIdx.x;
    const int64_t n0 = (int64_t)nt * kSplitBN;
    const int64_t tiles = (g.N + kSplitBN - 1) / kSplitBN;
    const float *part = reinterpret_cast<const float *>(g.ws) + (int64_t)nt * NSL * 4096;
    const float *ssq_part = reinterpret_cast<const float *>(g.ws) + tiles * NSL * 4096 + (int64_t)nt * NSL * 64;
    const int q = quarter * 256 + tid, tile = q / kWave, ln = q % kWave;
    f32x4 p[NSL];
#pragma unroll
    for (int s = 0; s < NSL; ++s) p[s] = *reinterpret_cast<const f32x4 *>(part + (int64_t)s * 4096 + 4 * q);
    if (tid < 64) {
        float sc = (g.row_scale && tid < g.M) ? g.row_scale[tid] : 1.0f;
        if constexpr (RMS) {
            float tot = 0.f;
#pragma unroll
            for (int s = 0; s < NSL; ++s) tot += ssq_part[s * 64 + tid];
            sc *= rms_scale(tot, g.K, g.rms_eps);
        }
        scale[tid] = sc;
    }
    __syncthreads();
    f32x4 v = p[0];
#pragma unroll
    for (int s = 1; s < NSL; ++s) v += p[s];
    uint16_t *C = static_cast<uint16_t *>(g.C);
    const int64_t col = n0 + 16 * (tile % 4) + ln % 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * (tile / 4) + 4 * (ln / 16) + r;
        if (row < g.M && col < g.N) C[row * g.ldc + col] = (uint16_t)f32_to_bf16(v[r] * scale[row]);
    }
}

template <bool RMS>
hipError_t launch_splitk(const GemmArgs &g, hipStream_t stream) {
    const int nsl = (int)(g.K / kSplitKS);
    const unsigned tiles = (unsigned)((g.N + kSplitBN - 1) / kSplitBN);
    gemm_splitk_kernel<RMS><<<dim3(tiles, (unsigned)nsl), dim3(256), 0, stream>>>(g, nsl);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid(tiles * 4), block(256);
    switch (nsl) {
        case 2: splitk_reduce_kernel<RMS, 2><<<grid, block, 0, stream>>>(g); break;
        case 4: splitk_reduce_kernel<RMS, 4><<<grid, block, 0, stream>>>(g); break;
        case 16: splitk_reduce_kernel<RMS, 16><<<grid, block, 0, stream>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <bool RMS, int BM, int BN, int WM, int WN, int GM>
hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
    const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    gemm_tiled_kernel<BM, BN, WM, WN, GM, RMS>
        <<<dim3((unsigned)tiles), dim3((BM / WM) * (BN / WN) * 64), 0, stream>>>(g);
    return hipGetLastError();
}

template <bool RMS>
hipError_t launch_gemm_t(const GemmArgs &g, hipStream_t stream) {
    if (g.M <= 64 && g.K == 2048) {
        // M > 32: each workgroup takes 32 rows, so a column tile is two
        // workgroups on one XCD that share its weights through L2, and every
        // workgroup reads half of A.  48 columns for wide outputs and 16 for
        // narrow ones give 256 workgroups (one per CU) at N = 6144 and N = 2048.
        // Measured on MI355X at M = 64 (graph-replayed, 24 distinct weights),
        // against 64-row workgroups of 32 / 16 columns: N = 6144 with the fused
        // RMS 12.2 -> 10.7 us, N = 2048 6.3 -> 5.0 us; 32-row workgroups of 32
        // columns (384 of them) 13.0 us.  The 64-row form measured ahead of
        // split-K (9.1 us at N = 2048) and of the skinny kernel (10.6 us).
        if (g.M > 32) {
            if (g.N >= 4096) {
                const int64_t tiles = (g.N + 47) / 48;
                gemm_stream_lds_kernel<3, 2, RMS, 32><<<dim3((unsigned)(((tiles + 7) / 8) * 16)), dim3(256), 0, stream>>>(g);
            } else {
                const int64_t tiles = (g.N + 15) / 16;
                const dim3 grid((unsigned)(((tiles + 7) / 8) * 16));
                // out_proj (no fused RMS) stages K by direct loads, five chunks
                // ahead (measured on MI355X in the 24-layer stack at batch 64,
                // token 0.4956 ms with the register-staged kernel, 0.4940 /
                // 0.4920 / 0.4899 ms with 3 / 4 / 6 chunk buffers)
                if constexpr (!RMS)
                    gemm_stream_dl_kernel<6><<<grid, dim3(256), 0, stream>>>(g);
                else
                    gemm_stream_lds_kernel<1, 2, RMS, 32><<<grid, dim3(256), 0, stream>>>(g);
            }
        } else if (g.N >= 4096)
            gemm_stream_lds_kernel<2, 2, RMS, 64><<<dim3((unsigned)((g.N + 31) / 32)), dim3(256), 0, stream>>>(g);
        else
            gemm_stream_lds_kernel<1, 2, RMS, 64><<<dim3((unsigned)((g.N + 15) / 16)), dim3(256), 0, stream>>>(g);
        return hipGetLastError();
    }
    const size_t ws_need = splitk_workspace_bytes(g.M, g.N, g.K);
    if (g.ws && ws_need > 0 && g.ws_bytes >= ws_need) return launch_splitk<RMS>(g, stream);
    if (g.M <= 64 && g.K % kSkCK == 0) {
        gemm_skinny_kernel<16, RMS><<<dim3((unsigned)((g.N + 15) / 16)), dim3(256), 0, stream>>>(g);
        return hipGetLastError();
    }
    // Plain products (no fused RMS) of whole 256 x 256 tiles with K = 2048:
    // measured on MI355X at M = 131072 (in_proj N = 6144 with a row scale,
    // out_proj N = 2048) 2.87 and 1.00 ms against 3.27 and 1.10 ms for the
    // tiled kernel below.
    if (!RMS && g.M % 256 == 0 && g.N % 256 == 0 && g.K == 2048 && g.lda % 8 == 0 && g.ldw % 8 == 0 &&
        g.ldc % 8 == 0 && reinterpret_cast<uintptr_t>(g.C) % 16 == 0 && g.lda < (1 << 20) && g.ldw < (1 << 20)) {
        gemm_dl8_kernel<64><<<dim3((unsigned)((g.M / 256) * (g.N / 256))), dim3(512), 0, stream>>>(g);
        return hipGetLastError();
    }
    // 256 x 256 tile, 16 waves of 64 x 64 (4 per SIMD): measured on MI355X at
    // M = 131072, K = 2048 ahead of 4 waves of 128 x 128 (1.3-1.6x) and of
    // 8 waves of 64 x 128.
    return launch_tiled<RMS, 256, 256, 64, 64, 4>(g, stream);
}

}  // namespace

size_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    // M <= 64 and N <= 4096 with K in {512, 1024, 4096}; K = 2048 always takes
    // the streaming kernel, which is faster than split-K there (measured on
    // MI355X at M = 64: 6.9 vs 9.1 us for N = 2048), so it needs no workspace.
    if (M < 1 || M > 64 || N < 1 || N > 4096 || K % kSplitKS != 0 || K == 2048) return 0;
    const int64_t nsl = K / kSplitKS;
    if (nsl != 2 && nsl != 4 && nsl != 16) return 0;
    const size_t tiles = (size_t)((N + kSplitBN - 1) / kSplitBN);
    return tiles * nsl * (4096 + 64) * sizeof(float);
}

hipError_t launch_row_rms(const RmsArgs &a, hipStream_t stream) {
    if (a.M == 0) return hipSuccess;
    row_rms_kernel<<<dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream) {
    if (g.M == 0 || g.N == 0) return hipSuccess;
    return g.rms ? launch_gemm_t<true>(g, stream) : launch_gemm_t<false>(g, stream);
}

hipError_t launch_layer_step(const GemmArgs &g, int d, hipStream_t stream) {
    if (g.M == 0) return hipSuccess;
    // column tiles of 48 = 16 channels; the two 32-row halves of a tile 8 workgroups apart
    const int64_t tiles = g.N / 48;
    const dim3 grid((unsigned)(((tiles + 7) / 8) * 16)), block(256);
    switch (d) {
        case 8: gemm_stream_lds_kernel<3, 2, true, 32, 8><<<grid, block, 0, stream>>>(g); break;
        case 16: gemm_stream_lds_kernel<3, 2, true, 32, 16><<<grid, block, 0, stream>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_layer_gate(const GemmArgs &g, hipStream_t stream) {
    if (g.M == 0) return hipSuccess;
    // Weights one chunk ahead (SW = 1), not two: measured on MI355X in the
    // 24-layer stack at batch 64, 0.5134 -> 0.5063 ms per token; the state
    // stream of the ride-along prepare gains more than the product loses.
    // Two and more chunks of weights ahead, or the layer input one chunk
    // ahead instead of two, or temporal weight loads, measured slower.
    const int64_t tiles = g.N / 48;
    const dim3 grid((unsigned)(((tiles + 7) / 8) * 16));
    switch (g.prep.B > 0 ? g.prep.d : 0) {
        case 0: gemm_stream_lds_kernel<3, 1, true, 32, -1, 0><<<grid, dim3(256), 0, stream>>>(g); break;
        case 8: gemm_stream_lds_kernel<3, 1, true, 32, -1, 8><<<grid, dim3(512), 0, stream>>>(g); break;
        case 16: gemm_stream_lds_kernel<3, 1, true, 32, -1, 16><<<grid, dim3(512), 0, stream>>>(g); break;
        case 32: gemm_stream_lds_kernel<3, 1, true, 32, -1, 32><<<grid, dim3(512), 0, stream>>>(g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

namespace {
// One workgroup per packed row: row 48 G + 16 j + i is in_proj row j D + 16 G + i.
__global__ __launch_bounds__(256) void pack_in_proj_kernel(int64_t D, int64_t K, const uint16_t *w, int64_t ldw,
                                                           uint16_t *out) {
    const int64_t r = blockIdx.x, grp = r / 48, j = (r % 48) / 16, i = r % 16;
    const uint16_t *src = w + (j * D + 16 * grp + i) * ldw;
    uint16_t *dst = out + r * K;
    for (int64_t k = threadIdx.x * 8; k < K; k += 256 * 8)
        *reinterpret_cast<uint4 *>(dst + k) = *reinterpret_cast<const uint4 *>(src + k);
}
}  // namespace

hipError_t launch_pack_in_proj(int64_t D, int64_t K, const void *w, int64_t ldw, void *out, hipStream_t stream) {
    if (D == 0) return hipSuccess;
    pack_in_proj_kernel<<<dim3((unsigned)(3 * D)), dim3(256), 0, stream>>>(D, K, static_cast<const uint16_t *>(w), ldw,
                                                                          static_cast<uint16_t *>(out));
    return hipGetLastError();
}

}  // namespace hm
