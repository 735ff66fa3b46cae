// prefill_mfma.hip -- prompt processing of the modal Hyena operator on the
// matrix cores (gfx950 MFMA), in sub-blocks of 64 steps.
//
// For a sub-block of 64 steps entering with state X (complex, d modes per
// channel), with u_j = k_j v_j:
//     y_i = q_i ( sum_{j<=i} h[i-j] u_j + Re sum_n R_n lambda_n^i X_n )      i < 64
//     X'  = lambda^64 X + sum_j lambda^(63-j) u_j
// (h[0] = D, h[m] = Re sum_n R_n lambda_n^(m-1)).  This is the causal long
// convolution y = q (h conv (k v)) of the StripedHyena article ("Hyena層次結構")
// cut at sub-block boundaries: the part inside the sub-block is a 64x64 causal
// Toeplitz product, the part from before it reaches the sub-block through the
// modal state.  Per head, all three matrices -- T (64x64 Toeplitz of h), C
// (64 x 2d readout rows Re/-Im of R lambda^i) and V (2d x 64 Vandermonde rows
// Re/Im of lambda^(63-j)) -- are shared by every channel and batch row (weight
// tying, Laughing Hyena Distillery review, "提出的方法"), so
//     Y = T U + C X,      S = V U,      X' = lambda^64 (.) X + S
// are dense GEMMs with N = channels.  They run as bf16 16x16x32 MFMAs with every
// operand split into bfloat16 parts and float32 accumulation:
//   bfloat16 activations: high and low part (hi*hi + hi*lo + lo*hi, about 16
//     significant bits per product; u = k v of two bfloat16 values is exact in
//     the two parts);
//   float32 activations: high, middle and low part, the six products down to
//     2^-16 of the leading one (hi*hi + hi*mid + mid*hi + hi*lo + lo*hi +
//     mid*mid), which keeps about 24 significant bits, float32 precision: the
//     "bf16x6" splitting of Henry, Tang and Heinecke ("Leveraging the bfloat16
//     artificial intelligence datatype for higher-precision computations",
//     ARITH 2019).
// The state stays in float32 registers from sub-block to sub-block.
//
// Work per element: 2*(64 + 4*D2) flops on the matrix cores (x3 or x6 for the
// split); the kernel is bound by streaming q, k, v and y through HBM.
//
// Workgroup: one (batch row, head, tile of PT = 64 or 128 channels, chunk),
// PT/16 waves of 16 channels each.  Per sub-block: q, k, v for 64 steps x PT
// channels are loaded one sub-block ahead (contiguous 16-byte pieces), u = k v
// is split and transposed into LDS ([channel][step], the MFMA B operand), q
// stays in the loading thread's registers, the Y accumulators go to an LDS
// tile that the loading threads read back to gate (y = q Y) and write out as
// whole row pieces.  Per-head table fragments (in A-operand lane order) sit in
// LDS.
//
// A prompt cut into chunks (when there are too few (row, head, tile) triples
// to fill the GPU) first runs the same kernel in state-only form over every
// chunk but the last: from a zero state it loads only k and v, does only
// S = V U and X' = lambda^64 X + S, and writes the chunk's end state S_c.  A
// carry scan then forms the state entering each chunk, which the full pass
// starts from.
#include "hm_internal.hpp"

#include <type_traits>

namespace hm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const uint4 a, const uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                    c, 0, 0, 0);
}

// Split products.  NP = 2: a = {hi, lo}: hi*hi + hi*lo + lo*hi.  NP = 3:
// a = {hi, mid, lo}: the small terms first (lo*hi, hi*lo, mid*mid, mid*hi,
// hi*mid), the leading hi*hi last.
template <int NP>
__device__ __forceinline__ f32x4 mfma_split(const uint4 (&a)[NP], const uint4 (&b)[NP], f32x4 c) {
    if constexpr (NP == 2) {
        c = mfma(a[0], b[0], c);
        c = mfma(a[0], b[1], c);
        return mfma(a[1], b[0], c);
    } else {
        c = mfma(a[2], b[0], c);
        c = mfma(a[0], b[2], c);
        c = mfma(a[1], b[1], c);
        c = mfma(a[1], b[0], c);
        c = mfma(a[0], b[1], c);
        return mfma(a[0], b[0], c);
    }
}

// bfloat16 parts of the table entries and of float32 operands
constexpr int parts_of(int act) { return act == kF32 ? 3 : 2; }

__device__ __forceinline__ uint32_t bf16_bits(float x) { return f32_to_bf16(x); }
__device__ __forceinline__ float bf16_val(uint32_t b) { return __uint_as_float(b << 16); }

constexpr int kTabThreads = 512;  // threads of a tables workgroup (one head)

// lambda^e in float64 from the polar form
__device__ inline void polar_pow(double lr, double li, double e, double &re, double &im) {
    if (e == 0.0) {
        re = 1.0;
        im = 0.0;
        return;
    }
    const double mag = exp(e * log(hypot(lr, li)));
    double s, c;
    sincos(e * atan2(li, lr), &s, &c);
    re = mag * c;
    im = mag * s;
}

// ------------------------------------------------------------------ tables

// One workgroup of 512 threads per head (every power below takes one pass),
// with the head's poles and residues staged in LDS.  Fragment f of the head,
// lane l, holds the eight
// A-operand values of that lane (row l%16 of the tile, k 8*(l/16)..+7):
//   f in [0, 8)            T tile (mt = f/2, kk = f%2): T[i][j] = h[i-j], j <= i
//   f in [8, 8+4KC)        C tile (mt, kc): C[i][2n] = Re(R_n lam_n^i), C[i][2n+1] = -Im(R_n lam_n^i)
//   f in [8+4KC, NFRAG)    V tile (ms, kk): V[2n][j] = Re lam_n^(63-j), V[2n+1][j] = Im lam_n^(63-j)
// stored as [head][f][part][lane] uint4 with NP parts (hi, lo or hi, mid, lo);
// also lam64[head][D2/2] = lambda^64.
template <int DD, int NP>
__global__ __launch_bounds__(kTabThreads) void mfma_tables_kernel(OpShape s, uint4 *frag, float2 *lam64,
                                                                  int64_t T, float2 *lamT) {
    using G = MfmaGeom<DD>;
    constexpr int D2 = G::D2, KC = G::KC, NFRAG = G::NFRAG;
    __shared__ double pr[65 * DD], pi[65 * DD];  // lambda_n^i, i <= 64
    __shared__ double hh[kSubBlock];
    __shared__ float2 pole[DD], res[DD];
    const int g = blockIdx.x, tid = threadIdx.x;
    if (tid < DD) {
        pole[tid] = s.poles[(int64_t)g * DD + tid];
        res[tid] = s.residues[(int64_t)g * DD + tid];
    }
    __syncthreads();
    // lambda^i for i = 4 seg .. 4 seg + 3: the first from the polar form, the
    // rest by float64 complex products (relative error ~1e-16 per product)
    for (int idx = tid; idx < 17 * DD; idx += kTabThreads) {
        const int seg = idx / DD, n = idx % DD;
        const float2 l = pole[n];
        const double lr = l.x, li = l.y;
        double re, im;
        polar_pow(lr, li, (double)(4 * seg), re, im);
        for (int k = 0; k < 4 && 4 * seg + k <= 64; ++k) {
            pr[(4 * seg + k) * DD + n] = re;
            pi[(4 * seg + k) * DD + n] = im;
            const double nr = re * lr - im * li;
            im = re * li + im * lr;
            re = nr;
        }
    }
    __syncthreads();
    for (int m = tid; m < kSubBlock; m += kTabThreads) {
        double acc = 0.0;
        if (m == 0) {
            acc = s.skip[g];
        } else {
            for (int n = 0; n < DD; ++n) {
                const float2 r = res[n];
                acc += (double)r.x * pr[(m - 1) * DD + n] - (double)r.y * pi[(m - 1) * DD + n];
            }
        }
        hh[m] = acc;
    }
    if (tid < D2 / 2)
        lam64[g * (D2 / 2) + tid] =
            tid < DD ? make_float2((float)pr[64 * DD + tid], (float)pi[64 * DD + tid]) : make_float2(0.f, 0.f);
    if (lamT && tid < DD) {  // lambda^T for the carry scan of a chunked prompt
        const float2 l = pole[tid];
        double re, im;
        polar_pow(l.x, l.y, (double)T, re, im);
        lamT[(int64_t)g * DD + tid] = make_float2((float)re, (float)im);
    }
    __syncthreads();
    for (int idx = tid; idx < NFRAG * kWave; idx += kTabThreads) {
        const int f = idx / kWave, l = idx % kWave;
        const int r16 = l % 16, k8 = 8 * (l / 16);
        uint32_t pt[NP][8];
        for (int e = 0; e < 8; ++e) {
            double v = 0.0;
            if (f < 8) {
                const int i = 16 * (f / 2) + r16, j = 32 * (f % 2) + k8 + e;
                v = (j <= i) ? hh[i - j] : 0.0;
            } else if (f < 8 + 4 * KC) {
                const int f2 = f - 8, i = 16 * (f2 / KC) + r16, k = 32 * (f2 % KC) + k8 + e, n = k / 2;
                if (n < DD) {
                    const float2 r = res[n];
                    const double a = pr[i * DD + n], b = pi[i * DD + n];
                    v = (k % 2 == 0) ? ((double)r.x * a - (double)r.y * b) : -((double)r.x * b + (double)r.y * a);
                }
            } else {
                const int f3 = f - 8 - 4 * KC, row = 16 * (f3 / 2) + r16, j = 32 * (f3 % 2) + k8 + e, n = row / 2;
                if (n < DD) v = (row % 2 == 0) ? pr[(63 - j) * DD + n] : pi[(63 - j) * DD + n];
            }
            if constexpr (NP == 2) {
                const float vf = (float)v;
                pt[0][e] = bf16_bits(vf);
                pt[1][e] = bf16_bits(vf - bf16_val(pt[0][e]));
            } else {
                // parts of the float64 value: each remainder is exact in float64
                pt[0][e] = bf16_bits((float)v);
                const double r1 = v - (double)bf16_val(pt[0][e]);
                pt[1][e] = bf16_bits((float)r1);
                pt[2][e] = bf16_bits((float)(r1 - (double)bf16_val(pt[1][e])));
            }
        }
        uint4 *o = frag + ((int64_t)(g * NFRAG + f) * NP) * kWave + l;
#pragma unroll
        for (int q = 0; q < NP; ++q)
            o[q * kWave] = make_uint4(pt[q][0] | pt[q][1] << 16, pt[q][2] | pt[q][3] << 16,
                                      pt[q][4] | pt[q][5] << 16, pt[q][6] | pt[q][7] << 16);
    }
}

// ------------------------------------------------------------------ sub-block kernel

// One thread's 8 channels of one row: channels e = 0..3 at the piece's
// address, e = 4..7 at SPLIT elements further.  bf16 rows use one 16-byte piece
// (SPLIT = 4), so consecutive lanes read consecutive 16 bytes.  float32 rows put
// the two 16-byte halves half a channel tile apart (SPLIT = PT/2), so each load
// instruction of a lane group still covers whole 128-byte lines.  The loads and
// stores are non-temporal: every element is read or written exactly once.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32v4 __attribute__((ext_vector_type(4)));
template <int ACT, int SPLIT> struct Piece;
template <int SPLIT> struct Piece<kBF16, SPLIT> {
    static_assert(SPLIT == 4, "bf16 pieces are 8 consecutive channels");
    u32x4 w;
    __device__ void load(const void *p) { w = __builtin_nontemporal_load(static_cast<const u32x4 *>(p)); }
    __device__ float get(int e) const { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); }
};
template <int SPLIT> struct Piece<kF32, SPLIT> {
    f32v4 a, b;
    __device__ void load(const void *p) {
        const float *f = static_cast<const float *>(p);
        a = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(f));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32v4 *>(f + SPLIT));
    }
    __device__ float get(int e) const { return (e < 4) ? a[e] : b[e - 4]; }
};
// The same 8 channels read one element at a time (rows not 16-byte aligned).
template <int ACT, int SPLIT> struct PieceScalar {
    float v[8];
    __device__ void load(const void *p) {
        const typename Act<ACT>::T *t = static_cast<const typename Act<ACT>::T *>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Act<ACT>::ld(t + (e & 3) + SPLIT * (e >> 2));
    }
    __device__ float get(int e) const { return v[e]; }
};

template <int SPLIT> __device__ __forceinline__ void store8(uint16_t *p, const float *v) {
    static_assert(SPLIT == 4, "bf16 pieces are 8 consecutive channels");
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}
template <int SPLIT> __device__ __forceinline__ void store8(float *p, const float *v) {
    __builtin_nontemporal_store(f32v4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32v4 *>(p));
    __builtin_nontemporal_store(f32v4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32v4 *>(p + SPLIT));
}

// LDS row of u for one channel: 64 steps in 16-byte units of 8 steps, the unit
// order XOR-permuted by (ch ^ ch/8) mod 8.  With it neither the transposing
// stores (8 channel groups x 8 step pairs per instruction) nor the MFMA operand
// reads (16 consecutive channels per instruction) meet a bank conflict on the
// 32 four-byte LDS banks.
constexpr int kLU = kSubBlock;
__device__ __forceinline__ int u_index(int ch, int t) {
    return ch * kLU + ((((t >> 3) ^ ((ch ^ (ch >> 3)) & 7))) << 3) + (t & 7);
}

// Y tile [step][channel] (float, row stride PT + 4): channels 32..63 of a row
// swap the halves of each 8-channel group, so the gating phase's 16-byte reads
// (8 channel groups of one row per 8 lanes) fall on disjoint banks.
__device__ __forceinline__ int yt_index(int row, int col, int ld) { return row * ld + (col ^ (((col >> 5) & 1) << 2)); }

// SO (state only): chunks 0 .. NC-2 of a chunked prompt, from a zero state,
// reading k and v only; writes S_c to carry slot c + 1.  VEC: 16-byte row
// pieces (else element loads, for rows that are not 16-byte aligned; the full
// pass always needs them aligned).
// PF: sub-blocks of q, k, v loads kept in flight (1 or 2).
// RS: row parts per sub-block (1 or 2).  With RS = 2 the workgroup has twice
// the waves: part 0 (the first PT / 16 waves) stages u, computes Y rows 0..31
// and the first half of the state modes, and gates and stores y; part 1
// computes Y rows 32..63 and the other half of the modes.  Both share the LDS
// tables and the u and x tiles, and pass the same two barriers per sub-block.
template <int DD, int PT, int ACT, bool SO, bool VEC, int PF, int RS>
__global__ __launch_bounds__(4 * PT * RS) void chunk_mfma_kernel(PrefillArgs a, const float2 *carry0) {
    using G = MfmaGeom<DD>;
    using T = typename Act<ACT>::T;
    // a thread's channels: CGW * cg + (e & 3) + SPLIT * (e >> 2), e = 0..7
    constexpr int SPLIT = (ACT == kF32) ? PT / 2 : 4, CGW = (ACT == kF32) ? 4 : 8;
    using PC = typename std::conditional<VEC, Piece<ACT, SPLIT>, PieceScalar<ACT, SPLIT>>::type;
    constexpr int D2 = G::D2, KC = G::KC, MTS = G::MTS, NFRAG = G::NFRAG;
    constexpr int NP = parts_of(ACT);          // bfloat16 parts per operand
    constexpr int NTHR = 4 * PT * RS;          // PT / 16 waves per row part
    constexpr int NSTG = 4 * PT;               // staging threads: row part 0
    constexpr int CW = 16, NTW = 1;            // channels and 16-wide tiles per wave
    constexpr int RG = 2;                      // staging rows per thread (two steps per 32-bit LDS word)
    constexpr int CG = PT / 8;                 // 8-channel groups per row
    constexpr int LX = D2 + 8;                 // LDS row of x (bf16), per channel
    constexpr int LQ = PT + 4;                 // LDS row of the Y tile (float), per step
    static_assert(PT == 64 || PT == 128, "channel tile");
    static_assert((64 / RG) * CG == NSTG, "one staging piece group per staging thread");
    static_assert(VEC || SO, "the full pass loads 16-byte pieces");
    static_assert(PF == 1 || PF == 2, "prefetch depth");
    static_assert(RS == 1 || (RS == 2 && MTS % 2 == 0), "row parts");

    __shared__ uint4 tab[NFRAG * NP * kWave];
    __shared__ __attribute__((aligned(16))) uint16_t ub[NP][PT * kLU];          // u parts, [channel][step]
    __shared__ __attribute__((aligned(16))) uint16_t xb[NP][SO ? 8 : PT * LX];  // state parts, [channel][row]
    __shared__ __attribute__((aligned(16))) float yt[SO ? 4 : kSubBlock * LQ];
    __shared__ float2 lamT[D2 / 2];
    static_assert(sizeof(tab) + sizeof(ub) + sizeof(xb) + sizeof(yt) + sizeof(lamT) <= 160 * 1024,
                  "LDS of one workgroup");

    const OpShape &s = a.s;
    const int64_t P = s.P, H = s.H, L = a.plan.L, Tc = a.plan.T;
    const int ntile = (int)(P / PT);
    const int g = blockIdx.x / ntile, ct = blockIdx.x % ntile;
    const int64_t c = blockIdx.y, b = blockIdx.z;
    const int64_t p0 = (int64_t)ct * PT;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int cw = (w % (PT / 16)) * CW;  // first local channel of this wave

    // per-head tables -> LDS
    {
        const uint4 *gt = reinterpret_cast<const uint4 *>(a.ws + a.plan.off_mfma_tab) + (int64_t)g * NFRAG * NP * kWave;
        for (int i = tid; i < NFRAG * NP * kWave; i += NTHR) tab[i] = gt[i];
        if (tid < D2 / 2)
            lamT[tid] = reinterpret_cast<const float2 *>(a.ws + a.plan.off_mfma_lam)[(int64_t)g * (D2 / 2) + tid];
    }

    const int64_t t_begin = c * Tc;
    const int nsteps = (int)(((L - t_begin) < Tc) ? (L - t_begin) : Tc);
    const int nsb = (nsteps + kSubBlock - 1) / kSubBlock;

    // The whole walk for row part HF: its Y rows [MT0, MT1), its state mode
    // tiles [MS0, MS0 + MSN); part 0 also stages and gates.
    auto walk = [&](auto hc) {
        constexpr int HF = decltype(hc)::value;
        constexpr bool STAGE = HF == 0;
        constexpr int MT0 = RS == 1 ? 0 : 2 * HF, MT1 = RS == 1 ? 4 : 2 * HF + 2;
        constexpr int MSN = MTS / RS, MS0 = HF * MSN;

        // entering state in C-tile layout: Xr[i][j] holds mode rows 16ms + 4(l/16) + 0..3
        // (modes 8ms + 2(l/16) and +1, Re/Im interleaved), ms = MS0 + i, of channel cw + 16j + l%16
        f32x4 Xr[MSN][NTW];
        {
            const float2 *src = SO ? nullptr : (c == 0) ? carry0
                                         : reinterpret_cast<const float2 *>(a.ws + a.plan.off_carry) +
                                               c * (s.B * H * DD * P);
#pragma unroll
            for (int i = 0; i < MSN; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int64_t p = p0 + cw + 16 * j + lane % 16;
                    const int n0 = 8 * (MS0 + i) + 2 * (lane / 16);
                    float2 x0 = make_float2(0.f, 0.f), x1 = make_float2(0.f, 0.f);
                    if (src && n0 < DD) x0 = src[((b * H + g) * DD + n0) * P + p];
                    if (src && n0 + 1 < DD) x1 = src[((b * H + g) * DD + n0 + 1) * P + p];
                    Xr[i][j] = f32x4{x0.x, x0.y, x1.x, x1.y};
                }
        }
        auto write_x = [&]() {
#pragma unroll
            for (int i = 0; i < MSN; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    f32x4 x = Xr[i][j];
                    const int o = (cw + 16 * j + lane % 16) * LX + 16 * (MS0 + i) + 4 * (lane / 16);
#pragma unroll
                    for (int q = 0; q < NP; ++q) {
                        // each part is x rounded to bfloat16, then x minus that part (exact)
                        const uint32_t p01 = pack_bf16x2(x[0], x[1]), p23 = pack_bf16x2(x[2], x[3]);
                        *reinterpret_cast<uint2 *>(&xb[q][o]) = make_uint2(p01, p23);
                        x = f32x4{x[0] - bf16_lo(p01), x[1] - bf16_hi(p01), x[2] - bf16_lo(p23), x[3] - bf16_hi(p23)};
                    }
                }
        };
        if constexpr (!SO) write_x();

        // staging role (row part 0): RG rows x 8 channels
        const int cg = tid % CG, rg = tid / CG;
        const int64_t ch0 = (int64_t)g * P + p0 + CGW * cg;  // global channel of the piece's element 0
        const T *qb = static_cast<const T *>(a.q) + (b * L + t_begin) * a.ld_in + ch0;
        const T *kb = static_cast<const T *>(a.k) + (b * L + t_begin) * a.ld_in + ch0;
        const T *vb = static_cast<const T *>(a.v) + (b * L + t_begin) * a.ld_in + ch0;
        T *yb = static_cast<T *>(a.y) + (b * L + t_begin) * a.ld_y + ch0;

        // q, k, v pieces of one sub-block: RG rows x 8 channels per thread
        struct Buf {
            PC q[RG], k[RG], v[RG];
        };
        auto load = [&](int sb, Buf &bf) {
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                int row = sb * kSubBlock + rg * RG + r;
                row = row < nsteps ? row : nsteps - 1;  // clamped; rows past the prompt are masked in staging
                const int64_t o = (int64_t)row * a.ld_in;
                if constexpr (!SO) bf.q[r].load(qb + o);
                bf.k[r].load(kb + o);
                bf.v[r].load(vb + o);
            }
        };

        // Two barriers per sub-block.  Between the second barrier of one sub-block
        // and the first of the next, threads read the Y tile (written before the
        // second) and write the u tiles (last read before the second), so the two
        // phases touch disjoint LDS.  With two row parts the x tiles are written
        // in that phase as well (both parts read all of x before the second).
        // One sub-block.  Its pieces are in `cur`; once staged, `cur` takes the
        // loads of sub-block sb + PF, so PF sub-blocks of loads stay in flight.
        auto sub_block = [&](int sb, Buf &cur) {
            const int nv = (nsteps - sb * kSubBlock < kSubBlock) ? nsteps - sb * kSubBlock : kSubBlock;
            // ---- stage: u = k v split into parts, transposed to [channel][step]; q stays in registers
            PC cq[RG];
            if constexpr (STAGE) {
                if constexpr (!SO) {
#pragma unroll
                    for (int r = 0; r < RG; ++r) cq[r] = cur.q[r];
                }
                float uu[RG][8];
#pragma unroll
                for (int r = 0; r < RG; ++r) {
                    const bool valid = rg * RG + r < nv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) uu[r][e] = valid ? cur.k[r].get(e) * cur.v[r].get(e) : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int o = u_index(CGW * cg + (e & 3) + SPLIT * (e >> 2), rg * RG);
                    float u0 = uu[0][e], u1 = uu[1][e];
#pragma unroll
                    for (int q = 0; q < NP; ++q) {
                        const uint32_t w2 = pack_bf16x2(u0, u1);
                        *reinterpret_cast<uint32_t *>(&ub[q][o]) = w2;
                        u0 -= bf16_lo(w2);
                        u1 -= bf16_hi(w2);
                    }
                }
                if (sb + PF < nsb) load(sb + PF, cur);  // PF sub-blocks ahead stay in flight during the products
            }
            __syncthreads();

            // ---- products
            f32x4 Y[MT1 - MT0][NTW], S[MSN][NTW];
#pragma unroll
            for (int i = 0; i < MT1 - MT0; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) Y[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < MSN; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) S[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            auto afrag = [&](int f, uint4 (&av)[NP]) {
#pragma unroll
                for (int q = 0; q < NP; ++q) av[q] = tab[(f * NP + q) * kWave + lane];
            };
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 bv[NTW][NP];
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int o = u_index(cw + 16 * j + lane % 16, 32 * kk + 8 * (lane / 16));
#pragma unroll
                    for (int q = 0; q < NP; ++q) bv[j][q] = *reinterpret_cast<const uint4 *>(&ub[q][o]);
                }
                if constexpr (!SO) {
#pragma unroll
                    for (int mt = MT0; mt < MT1; ++mt) {
                        // T is causal: rows 0..31 against steps 32..63 are all zero
                        if (kk == 1 && mt < 2) continue;
                        uint4 av[NP];
                        afrag(mt * 2 + kk, av);
#pragma unroll
                        for (int j = 0; j < NTW; ++j) Y[mt - MT0][j] = mfma_split<NP>(av, bv[j], Y[mt - MT0][j]);
                    }
                }
#pragma unroll
                for (int i = 0; i < MSN; ++i) {
                    uint4 av[NP];
                    afrag(8 + 4 * KC + (MS0 + i) * 2 + kk, av);
#pragma unroll
                    for (int j = 0; j < NTW; ++j) S[i][j] = mfma_split<NP>(av, bv[j], S[i][j]);
                }
            }
#pragma unroll
            for (int kc = 0; kc < (SO ? 0 : KC); ++kc) {
                uint4 xv[NTW][NP];
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int o = (cw + 16 * j + lane % 16) * LX + 32 * kc + 8 * (lane / 16);
#pragma unroll
                    for (int q = 0; q < NP; ++q) xv[j][q] = *reinterpret_cast<const uint4 *>(&xb[q][o]);
                }
#pragma unroll
                for (int mt = MT0; mt < MT1; ++mt) {
                    uint4 av[NP];
                    afrag(8 + mt * KC + kc, av);
#pragma unroll
                    for (int j = 0; j < NTW; ++j) Y[mt - MT0][j] = mfma_split<NP>(av, xv[j], Y[mt - MT0][j]);
                }
            }

            // ---- Y tile -> LDS ([step][channel])
            if constexpr (!SO) {
#pragma unroll
                for (int mt = MT0; mt < MT1; ++mt)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            yt[yt_index(16 * mt + 4 * (lane / 16) + r, cw + 16 * j + lane % 16, LQ)] = Y[mt - MT0][j][r];
            }

            // ---- state hand-off
            if (nv == kSubBlock) {
#pragma unroll
                for (int i = 0; i < MSN; ++i)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int q2 = 0; q2 < 2; ++q2) {
                            const float2 lt = lamT[8 * (MS0 + i) + 2 * (lane / 16) + q2];
                            const float xr = Xr[i][j][2 * q2], xi = Xr[i][j][2 * q2 + 1];
                            Xr[i][j][2 * q2] = fmaf(lt.x, xr, fmaf(-lt.y, xi, S[i][j][2 * q2]));
                            Xr[i][j][2 * q2 + 1] = fmaf(lt.x, xi, fmaf(lt.y, xr, S[i][j][2 * q2 + 1]));
                        }
                // with two row parts the other part may still be reading the
                // entering x (its C X products): the next x goes to LDS after
                // the barrier below
                if constexpr (!SO && RS == 1) write_x();
            } else {
                // ragged final sub-block (end of the prompt): step the recurrence
                // over its nv steps on the vector ALUs, from u = the sum of its parts in LDS
#pragma unroll
                for (int i = 0; i < MSN; ++i)
#pragma unroll
                    for (int j = 0; j < NTW; ++j)
#pragma unroll
                        for (int q2 = 0; q2 < 2; ++q2) {
                            const int n = 8 * (MS0 + i) + 2 * (lane / 16) + q2;
                            if (n >= DD) continue;
                            const float2 l = s.poles[(int64_t)g * DD + n];
                            float xr = Xr[i][j][2 * q2], xi = Xr[i][j][2 * q2 + 1];
                            const int ch = cw + 16 * j + lane % 16;
                            for (int t = 0; t < nv; ++t) {
                                const int o = u_index(ch, t);
                                float u = 0.f;
#pragma unroll
                                for (int q = NP - 1; q >= 0; --q) u += bf16_val(ub[q][o]);
                                const float nr = fmaf(l.x, xr, fmaf(-l.y, xi, u));
                                xi = fmaf(l.x, xi, l.y * xr);
                                xr = nr;
                            }
                            Xr[i][j][2 * q2] = xr;
                            Xr[i][j][2 * q2 + 1] = xi;
                        }
            }
            __syncthreads();
            if constexpr (!SO && RS == 2) {
                if (nv == kSubBlock) write_x();
            }

            // ---- gate y = q Y and store whole 8-channel pieces of valid rows
            if constexpr (STAGE) {
#pragma unroll
                for (int r = 0; r < (SO ? 0 : RG); ++r) {
                    const int row = rg * RG + r;
                    if (row < nv) {
                        const float4 y0 = *reinterpret_cast<const float4 *>(&yt[yt_index(row, CGW * cg, LQ)]);
                        const float4 y1 = *reinterpret_cast<const float4 *>(&yt[yt_index(row, CGW * cg + SPLIT, LQ)]);
                        const float yy[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = cq[r].get(e) * yy[e];
                        store8<SPLIT>(reinterpret_cast<T *>(yb + (int64_t)(sb * kSubBlock + row) * a.ld_y), v);
                    }
                }
            }
        };
        Buf b0, b1;
        if constexpr (STAGE) load(0, b0);
        if constexpr (PF == 2) {
            if constexpr (STAGE) {
                if (nsb > 1) load(1, b1);
            }
            for (int sb = 0; sb < nsb; sb += 2) {
                sub_block(sb, b0);
                if (sb + 1 < nsb) sub_block(sb + 1, b1);
            }
        } else {
            for (int sb = 0; sb < nsb; ++sb) sub_block(sb, b0);
        }

        if (SO || c == a.plan.NC - 1) {
            float2 *const base = SO ? reinterpret_cast<float2 *>(a.ws + a.plan.off_carry) + (c + 1) * (s.B * H * DD * P)
                                    : a.state_out;
#pragma unroll
            for (int i = 0; i < MSN; ++i)
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    const int64_t p = p0 + cw + 16 * j + lane % 16;
                    const int n0 = 8 * (MS0 + i) + 2 * (lane / 16);
                    float2 *dst = base + ((b * H + g) * DD) * P + p;
                    if (n0 < DD) dst[(int64_t)n0 * P] = make_float2(Xr[i][j][0], Xr[i][j][1]);
                    if (n0 + 1 < DD) dst[(int64_t)(n0 + 1) * P] = make_float2(Xr[i][j][2], Xr[i][j][3]);
                }
        }
    };
    if constexpr (RS == 1) {
        walk(std::integral_constant<int, 0>{});
    } else {
        // the row part is wave-uniform; readfirstlane makes the branch scalar, so
        // each wave runs only its own part (and its own two barriers per sub-block)
        if (__builtin_amdgcn_readfirstlane(w / (PT / 16)) == 0)
            walk(std::integral_constant<int, 0>{});
        else
            walk(std::integral_constant<int, 1>{});
    }
}

// Load prefetch depth in sub-blocks.  float32 sub-blocks do twice the matrix-core
// work of bfloat16 ones (six split products instead of three), which a single
// sub-block of loads in flight no longer covers at one wave per SIMD.
constexpr int kPfBF16 = 1, kPfF32 = 2;
// Row parts of the full pass (the state-only pass keeps one): two for float32
// 64-channel tiles, whose three-part tables hold the workgroup to four waves
// per CU otherwise (at 128 channels, 16 waves would spill).
constexpr int kRsBF16 = 1;
template <int PT> constexpr int rs_f32() { return PT == 64 ? 2 : 1; }

// float32 tiles of 128 channels take three bfloat16 parts of every operand and
// do not fit the LDS at d = 32: the channel tile is 64 there.
template <int DD, int PT> constexpr bool f32_tile_fits() { return !(DD == 32 && PT == 128); }

template <int DD, int PT>
hipError_t launch_dd(const PrefillArgs &a, const float2 *carry0, hipStream_t stream) {
    const dim3 grid((unsigned)(a.s.H * (a.s.P / PT)), (unsigned)a.plan.NC, (unsigned)a.s.B);
    if (a.s.act == kBF16) {
        chunk_mfma_kernel<DD, PT, kBF16, false, true, kPfBF16, kRsBF16><<<grid, dim3(4 * PT * kRsBF16), 0, stream>>>(
            a, carry0);
    } else {
        if constexpr (f32_tile_fits<DD, PT>())
            chunk_mfma_kernel<DD, PT, kF32, false, true, kPfF32, rs_f32<PT>()>
                <<<grid, dim3(4 * PT * rs_f32<PT>()), 0, stream>>>(a, carry0);
        else
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DD, int PT>
hipError_t launch_dd_state(const PrefillArgs &a, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)(a.s.H * (a.s.P / PT)), (unsigned)(a.plan.NC - 1), (unsigned)a.s.B), block(4 * PT);
    if (a.s.act == kBF16) {
        if (vec) chunk_mfma_kernel<DD, PT, kBF16, true, true, kPfBF16, 1><<<grid, block, 0, stream>>>(a, nullptr);
        else chunk_mfma_kernel<DD, PT, kBF16, true, false, kPfBF16, 1><<<grid, block, 0, stream>>>(a, nullptr);
    } else {
        if constexpr (f32_tile_fits<DD, PT>()) {
            if (vec) chunk_mfma_kernel<DD, PT, kF32, true, true, kPfF32, 1><<<grid, block, 0, stream>>>(a, nullptr);
            else chunk_mfma_kernel<DD, PT, kF32, true, false, kPfF32, 1><<<grid, block, 0, stream>>>(a, nullptr);
        } else {
            return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int PT>
hipError_t launch_pt(const PrefillArgs &a, const float2 *carry0, bool state_only, bool vec, hipStream_t stream) {
    switch (a.s.d) {
        case 8: return state_only ? launch_dd_state<8, PT>(a, vec, stream) : launch_dd<8, PT>(a, carry0, stream);
        case 16: return state_only ? launch_dd_state<16, PT>(a, vec, stream) : launch_dd<16, PT>(a, carry0, stream);
        case 32: return state_only ? launch_dd_state<32, PT>(a, vec, stream) : launch_dd<32, PT>(a, carry0, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Channel tile: 128 channels (8 waves, 256-byte row pieces) when that still
// gives one workgroup per CU without cutting the prompt into chunks (measured
// on MI355X: 2.8 % faster at B = 16, D = 2048 and 3.6 % at B = 256 than two
// 64-channel workgroups per CU), else 64.
int mfma_channel_tile(const OpShape &s) {
    if (s.d != 8 && s.d != 16 && s.d != 32) return 0;
    const bool wide_fits = !(s.act == kF32 && s.d == 32);
    if (wide_fits && s.P % 128 == 0 && s.B * s.H * (s.P / 128) >= 256) return 128;
    return (s.P % 64 == 0) ? 64 : 0;
}

size_t mfma_table_bytes(int64_t H, int64_t d, int act) {
    const size_t np = (size_t)parts_of(act);
    switch (d) {
        case 8: return (size_t)H * MfmaGeom<8>::NFRAG * np * kWave * 16;
        case 16: return (size_t)H * MfmaGeom<16>::NFRAG * np * kWave * 16;
        case 32: return (size_t)H * MfmaGeom<32>::NFRAG * np * kWave * 16;
        default: return 0;
    }
}

size_t mfma_lam_bytes(int64_t H, int64_t d) {
    const int64_t d2 = (2 * d < 32) ? 32 : 2 * d;
    return (size_t)H * (d2 / 2) * sizeof(float2);
}

hipError_t launch_mfma_tables(const PrefillArgs &a, hipStream_t stream) {
    uint4 *frag = reinterpret_cast<uint4 *>(a.ws + a.plan.off_mfma_tab);
    float2 *lam = reinterpret_cast<float2 *>(a.ws + a.plan.off_mfma_lam);
    float2 *lamT = a.plan.NC > 1 ? reinterpret_cast<float2 *>(a.ws + a.plan.off_lamT) : nullptr;
    const dim3 grid((unsigned)a.s.H), block(kTabThreads);
    const bool f32 = a.s.act == kF32;
    switch (a.s.d) {
        case 8:
            if (f32) mfma_tables_kernel<8, 3><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            else mfma_tables_kernel<8, 2><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            break;
        case 16:
            if (f32) mfma_tables_kernel<16, 3><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            else mfma_tables_kernel<16, 2><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            break;
        case 32:
            if (f32) mfma_tables_kernel<32, 3><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            else mfma_tables_kernel<32, 2><<<grid, block, 0, stream>>>(a.s, frag, lam, a.plan.T, lamT);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_chunk_mfma(const PrefillArgs &a, const float2 *carry0, hipStream_t stream) {
    const int pt = mfma_channel_tile(a.s);
    if (pt == 128) return launch_pt<128>(a, carry0, false, true, stream);
    if (pt == 64) return launch_pt<64>(a, carry0, false, true, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_mfma_state(const PrefillArgs &a, bool vec, hipStream_t stream) {
    if (a.plan.NC < 2) return hipSuccess;
    const int pt = mfma_channel_tile(a.s);
    if (pt == 128) return launch_pt<128>(a, nullptr, true, vec, stream);
    if (pt == 64) return launch_pt<64>(a, nullptr, true, vec, stream);
    return hipErrorInvalidValue;
}

}  // namespace hm
