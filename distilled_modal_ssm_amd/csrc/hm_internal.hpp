// Internal declarations of the gfx950 modal-SSM Hyena library: argument blocks
// passed to the kernel launchers, and device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hm {

constexpr int kWave = 64;
constexpr int kMaxModes = 64;  // largest supported number of modes d

enum ActType : int { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two float32 -> a packed bfloat16 pair (a in the low half), round to nearest
// even, in one v_cvt_pk_bf16_f32.
typedef __bf16 hm_bf16x2 __attribute__((ext_vector_type(2)));
typedef float hm_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(hm_f32x2{a, b}, hm_bf16x2));
}

// lambda^e (e >= 0) in float64 by binary powering: at most 2 log2(e) complex
// products, relative error ~1e-15 even for e ~ 64k and |lambda| ~ 0.9999.
__device__ inline void complex_pow(double lr, double li, int64_t e, double &pr, double &pi) {
    pr = 1.0;
    pi = 0.0;
    double br = lr, bi = li;
    while (e != 0) {
        if (e & 1) {
            const double nr = pr * br - pi * bi;
            pi = pr * bi + pi * br;
            pr = nr;
        }
        const double nb = br * br - bi * bi;
        bi = 2.0 * br * bi;
        br = nb;
        e >>= 1;
    }
}

// Activation element access for float32 (ACT = kF32) or bfloat16 bit patterns.
template <int ACT> struct Act;

template <> struct Act<kF32> {
    using T = float;
    static constexpr int kBytes = 4;
    __device__ static float ld(const T *p) { return *p; }
    __device__ static float2 ld2(const T *p) { return *reinterpret_cast<const float2 *>(p); }
    __device__ static void st(T *p, float x) { *p = x; }
    __device__ static void st2(T *p, float a, float b) {
        *reinterpret_cast<float2 *>(p) = make_float2(a, b);
    }
};

template <> struct Act<kBF16> {
    using T = uint16_t;
    static constexpr int kBytes = 2;
    __device__ static float ld(const T *p) { return __uint_as_float((uint32_t)*p << 16); }
    __device__ static float2 ld2(const T *p) {
        uint32_t w = *reinterpret_cast<const uint32_t *>(p);
        return make_float2(bf16_lo(w), bf16_hi(w));
    }
    __device__ static void st(T *p, float x) { *p = (uint16_t)f32_to_bf16(x); }
    __device__ static void st2(T *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
};

// Raw-buffer access to activations: a wave-uniform descriptor over one region,
// a per-lane 32-bit byte offset and a wave-uniform (scalar) byte offset, so the
// address arithmetic stays off the vector ALUs.  Every access must lie inside
// the region given to make_region.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_region(const void *base, uint32_t bytes) {
    // dword 3 = 0x00020000: 32-bit data format, the value the gfx9 family expects
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

template <int ACT> struct BufAct;

template <> struct BufAct<kF32> {
    __device__ static float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    }
    __device__ static void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
    }
};

template <> struct BufAct<kBF16> {
    __device__ static float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0) << 16);
    }
    __device__ static void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16(x), r, voff, soff, 0);
    }
};

// ---------------------------------------------------------------- argument blocks

struct OpShape {
    int64_t B, D, H, d, P;
    int act;
    const float2 *poles;    // [H][d]
    const float2 *residues; // [H][d]
    const float *skip;      // [H]
};

struct DecodeArgs {
    OpShape s;
    const void *q, *k, *v;
    int64_t ld_in;
    void *y;
    int64_t ld_y;
    float2 *state; // [B][H][d][P]
};

struct FilterArgs {
    OpShape s;
    int64_t L;
    float *h; // [H][L]
};

// In-chunk algorithms of prefill.
enum PrefillAlgo : int { kAlgoAuto = 0, kAlgoScan = 1, kAlgoMfma = 2 };

// Chunked prefill plan: NC chunks of T steps (the last one may be shorter).
struct PrefillPlan {
    int64_t L, T, NC;
    int algo;            // kAlgoScan or kAlgoMfma (resolved)
    int64_t mtiles;      // 16-row tiles of the 2d Vandermonde rows (chunk states)
    size_t off_vand_hi;  // bf16 A-operand fragments, [H][mtiles][T/32][64 lanes][8]
    size_t off_vand_lo;
    size_t off_lamT;     // float2 [H][d]: lambda^T
    size_t off_carry;    // float2 [NC][B][H][d][P]: state entering each chunk
    size_t off_mfma_tab; // sub-block tables (matrix-core path)
    size_t off_mfma_lam; // float2 [H][D2/2]: lambda^64
    size_t bytes;        // total workspace
};

// Geometry of the matrix-core prefill for d modes: D2 = mode rows (Re/Im of
// each mode, padded to at least 32), fragment counts of the per-head tables.
constexpr int kSubBlock = 64;  // steps per sub-block
template <int DD> struct MfmaGeom {
    static constexpr int D2 = (2 * DD < 32) ? 32 : 2 * DD;
    static constexpr int KC = D2 / 32;   // 32-wide k steps of C X
    static constexpr int MTS = D2 / 16;  // 16-row tiles of V U
    static constexpr int NFRAG = 8 + 4 * KC + 2 * MTS;  // T + C + V fragments
};

struct PrefillArgs {
    OpShape s;
    PrefillPlan plan;
    const void *q, *k, *v;
    int64_t ld_in;
    void *y;
    int64_t ld_y;
    const float2 *state_in; // nullable
    float2 *state_out;
    unsigned char *ws;
};

struct RmsArgs {
    const void *x;  // bf16 [M][ld]
    int64_t M, D, ld;
    float eps;
    float *inv_rms;  // [M]
    bool vec;        // rows 16-byte aligned and D % 8 == 0
};

// Deferred state of a generated token (the stack's generation step).  The
// state of a layer is kept one input behind: s = x - u_prev, where x is the
// modal state of the recurrence and u_prev the layer's last input u (real, so
// it adds to the real part of every mode).  "Prepare" turns s and u_prev into
// the readout of the coming token and the next deferred state,
//     x = s + u_prev;  rho = Re sum_n R_n x_n;  s <- lambda x,
// which needs nothing from the coming token; its gate is then
//     y = q (D u + rho),  u_prev <- u.
struct PrepArgs {
    int64_t B = 0, D = 0, H = 0, P = 0, d = 0;  // B = 0: no prepare
    float2 *state = nullptr;                    // s, [B][H][d][P] complex, in/out
    const float *u_prev = nullptr;              // [B][D]
    float *rho = nullptr;                       // [B][D] out
    const float2 *poles = nullptr, *residues = nullptr;  // [H][d]
};

// Prepare of one unit: batch row b, channels c and c + 1 (c even, one head;
// D / H even), unit = b D/2 + c/2.  16-byte state accesses, non-temporal (the
// state is streamed once per token).  The modes go in four quarters, each
// loaded whole, then updated and stored, so the state's stores start after a
// quarter of its loads.  Measured on MI355X riding in the 24-layer stack's
// gate at batch 64, d = 16, with the gate's weights one chunk ahead: 0.495 ms
// per token against 0.503 ms for halves, 0.514 ms for eighths and 0.533 ms for
// one mode at a time (with the weights two chunks ahead, halves had measured
// ahead of quarters).
template <int DD>
__device__ __forceinline__ void prepare_unit(const PrepArgs &p, int64_t unit) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int HB = DD / 4;
    const int64_t half = p.D / 2, b = unit / half, c = 2 * (unit - b * half), g = c / p.P;
    f4 *st = reinterpret_cast<f4 *>(p.state + ((b * p.H + g) * DD) * p.P + (c - g * p.P));
    const float2 up = *reinterpret_cast<const float2 *>(p.u_prev + b * p.D + c);
    const float2 *lam = p.poles + g * DD, *res = p.residues + g * DD;
    float r0 = 0.f, r1 = 0.f;
#pragma unroll
    for (int h0 = 0; h0 < DD; h0 += HB) {
        f4 v[HB];
#pragma unroll
        for (int n = 0; n < HB; ++n) v[n] = __builtin_nontemporal_load(st + (h0 + n) * (p.P / 2));
#pragma unroll
        for (int n = 0; n < HB; ++n) {
            const float2 l = lam[h0 + n], r = res[h0 + n];
            const float ar = v[n][0] + up.x, ai = v[n][1], br = v[n][2] + up.y, bi = v[n][3];
            r0 = fmaf(r.x, ar, fmaf(-r.y, ai, r0));
            r1 = fmaf(r.x, br, fmaf(-r.y, bi, r1));
            __builtin_nontemporal_store(f4{fmaf(l.x, ar, -l.y * ai), fmaf(l.x, ai, l.y * ar), fmaf(l.x, br, -l.y * bi),
                                           fmaf(l.x, bi, l.y * br)},
                                        st + (h0 + n) * (p.P / 2));
        }
    }
    *reinterpret_cast<float2 *>(p.rho + b * p.D + c) = make_float2(r0, r1);
}

struct GemmArgs {
    int64_t M, N, K;
    const void *A;  // bf16 [M][lda]
    int64_t lda;
    const void *W;  // bf16 [N][ldw]
    int64_t ldw;
    const float *row_scale;  // [M] or null
    void *C;                 // bf16 [M][ldc]
    int64_t ldc;
    bool rms;                // also scale row m by 1/sqrt(mean_k A[m][k]^2 + rms_eps)
    float rms_eps;
    unsigned char *ws = nullptr;  // split-K workspace (M <= 64), or null
    size_t ws_bytes = 0;
    // Fused generation step of a projected layer (launch_layer_step only): W is
    // the packed in_proj, and the epilogue runs the decode step on the columns
    // instead of storing C.
    float2 *state = nullptr;                      // [M][H][d][P] complex, in/out
    const float2 *poles = nullptr, *residues = nullptr;  // [H][d]
    const float *skip = nullptr;                  // [H]
    int64_t P = 0, H = 0;
    void *y = nullptr;                            // bf16 [M][ld_y]
    int64_t ld_y = 0;
    // Gate of a generated token with the deferred state (launch_layer_gate only):
    // the epilogue computes y = q (D u + rho), u_prev <- u for its columns, and
    // four extra waves per workgroup run the prepare `prep` of another layer.
    const float *rho = nullptr;   // [M][H*P]
    float *u_prev = nullptr;      // [M][H*P] out
    PrepArgs prep;
};

bool prepare_supported(int64_t d);
hipError_t launch_prepare(const PrepArgs &p, hipStream_t stream);
hipError_t launch_layer_gate(const GemmArgs &g, hipStream_t stream);

// Split-K path of the small-M GEMM: 64-column tiles x 256-wide K slices write
// fp32 partials, a second pass sums them per tile.  Workspace: partials
// [tiles][slices][64*64] fp32, then row sums of squares [tiles][slices][64]
// fp32.  0 bytes when the shape does not take this path.
constexpr int kSplitBN = 64, kSplitKS = 256;
size_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);

// Explicit-filter (non-distilled) decode step and its u cache.
struct FirArgs {
    OpShape s;
    const float *h;     // [H][h_len] taps
    int64_t h_len;
    int64_t t;          // position of the token being generated
    int64_t lo;         // first cached row in the window
    int R;              // row ranges of pass 1
    const void *q, *k, *v;
    int64_t ld_in;
    void *y;
    int64_t ld_y;
    void *cache;        // [B][cache_len][D] activation dtype
    int64_t cache_len;
    float *part;        // [R][B][D] fp32
    int loads = 0;      // cache loads: 0 by window size, 1 plain, 2 non-temporal
};
int fir_ranges(int64_t B, int64_t D);
hipError_t launch_fir_decode(const FirArgs &a, hipStream_t stream);
hipError_t launch_fir_fill(const FirArgs &a, int64_t L, hipStream_t stream);

// FFT prefill (the convolution through transforms of length N = 2^logn >= 2L).
struct FftArgs {
    OpShape s;
    int64_t L;
    int logn;
    int np;             // channel pairs per workgroup
    const void *q, *k, *v;
    int64_t ld_in;
    void *y;
    int64_t ld_y;
    float *h;           // [H][L] taps (workspace)
    float2 *tw;         // [N/2] twiddles (workspace)
    float2 *spec;       // [H][N] filter spectra (workspace)
    float2 *z;          // [B][N][D/2] transform of the channel pairs, multi-pass path only (workspace)
};
constexpr int kFftMaxLogN = 13;      // N <= 8192: one transform in one workgroup's LDS (prompts up to 4096)
constexpr int kFftMaxLogNLong = 18;  // N <= 262144 in three passes over HBM (prompts up to 131072)
int fft_log_n(int64_t L);
int fft_pairs_per_group(int64_t P, int logn);
size_t fft_lds_bytes(int logn, int np);
hipError_t launch_fft_prefill(const FftArgs &a, hipStream_t stream);

// Distillation objective: filter discrepancy against target taps, its gradient,
// and an Adam step on the modal parameters.
struct DistillArgs {
    OpShape s;
    int64_t L;
    const float *target;  // [H][L]
    double *e;            // [H][L] residual hhat - target
    double *loss_part;    // [H][tiles]
    double *grad_part;    // [H*d][chunks][4]
    int tiles, chunks;
    float *loss, *g_poles, *g_res, *g_skip;
};
constexpr int kDistillTile = 8192;  // taps per gradient workgroup
int distill_tiles(int64_t L, int64_t d);  // residual workgroups per head
hipError_t launch_distill_grad(const DistillArgs &a, hipStream_t stream);
struct AdamArgs {
    int64_t H, d;
    float *poles, *residues, *skip;
    const float *g_poles, *g_res, *g_skip;
    float *m, *v;  // [H*d*4 + H]: poles (2/mode), residues (2/mode), skip
    float lr, beta1, beta2, eps, r_max, bc1, bc2;
};
hipError_t launch_distill_adam(const AdamArgs &a, hipStream_t stream);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; none synchronises.

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_filter(const FilterArgs &a, hipStream_t stream);
PrefillPlan make_prefill_plan(const OpShape &s, int64_t L, int64_t chunk, int algo);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);
// matrix-core prefill (prefill_mfma.hip)
int mfma_channel_tile(const OpShape &s);  // channels per workgroup, 0 = not eligible
size_t mfma_table_bytes(int64_t H, int64_t d, int act);
size_t mfma_lam_bytes(int64_t H, int64_t d);
// per-head tables; also lambda^T (carry scan) when the prompt is chunked
hipError_t launch_mfma_tables(const PrefillArgs &a, hipStream_t stream);
hipError_t launch_chunk_mfma(const PrefillArgs &a, const float2 *carry0, hipStream_t stream);
// chunk end states S_c of chunks 0 .. NC-2 into carry slots 1 .. NC-1 (vec: 16-byte k, v pieces)
hipError_t launch_chunk_mfma_state(const PrefillArgs &a, bool vec, hipStream_t stream);
hipError_t launch_row_rms(const RmsArgs &a, hipStream_t stream);
hipError_t launch_gemm(const GemmArgs &g, hipStream_t stream);
// Generation step of a projected layer: packed in_proj (fused RMS) + decode step
// in one launch; M <= 64, K = 2048, N = 3 * channels, d in {8, 16}.
hipError_t launch_layer_step(const GemmArgs &g, int d, hipStream_t stream);
// in_proj weights [3D][K] -> packed rows: 48 G + 16 j + i <- j D + 16 G + i.
hipError_t launch_pack_in_proj(int64_t D, int64_t K, const void *w, int64_t ldw, void *out, hipStream_t stream);

}  // namespace hm
