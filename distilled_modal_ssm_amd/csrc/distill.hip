// distill.hip -- the distillation objective on the GPU: how far a modal
// filter is from a given long filter, its gradient, and an optimiser step.
//
// Distillation replaces each head's long convolution filter h by a d-mode
// modal filter hhat (Laughing Hyena Distillery review, 提出的方法: the filters
// are fitted under a filter-discrepancy objective, then decoded as a
// recurrence).  Here the discrepancy is the squared distance over L taps,
//     J_g = sum_{t<L} (hhat_g[t] - h_g[t])^2,
//     hhat_g[0] = D_g,  hhat_g[t] = Re sum_n R_gn lambda_gn^(t-1),
// with e = hhat - h and p_t = lambda^(t-1):
//     dJ/dD = 2 e[0],  dJ/dR_n = 2 sum_t e[t] (Re p_t, -Im p_t),
//     dJ/dlambda_n = 2 sum_t e[t] (Re c_t, -Im c_t),  c_t = R_n (t-1) lambda_n^(t-2),
// (hhat is the real part of a function holomorphic in lambda and R).
//
// Kernels, all float64 inside: (1) residual -- one thread per (head, mode,
// 32-tap run) evaluates R lambda^(t-1) by binary powering and a walk, the
// workgroup sums the modes per tap in LDS, writes e and a partial sum of e^2;
// (2) gradient -- per (head, mode, 8192-tap chunk), each thread walks
// lambda^(t-2) and lambda^(t-1) over every 256th tap against e (coalesced
// reads) and the workgroup reduces four sums; (3) finish
// -- sums the partials into float32 loss and gradients.  The Adam step keeps
// every |lambda| <= r_max < 1 (a stable recurrence).
#include "hm_internal.hpp"

namespace hm {
namespace {

constexpr int kRun = 32;

template <int DPAD>
__global__ __launch_bounds__(256) void distill_residual_kernel(DistillArgs a) {
    constexpr int RPB = 256 / DPAD, TPB = RPB * kRun, LP = kRun + 1;
    __shared__ double part[RPB * DPAD * LP];
    __shared__ double red[256];
    const int64_t L = a.L, d = a.s.d;
    const int64_t tiles = (L + TPB - 1) / TPB;
    const int64_t g = blockIdx.x / tiles, tile = blockIdx.x - g * tiles;
    const int n = threadIdx.x % DPAD, rl = threadIdx.x / DPAD;
    const int64_t t0 = tile * TPB + (int64_t)rl * kRun;
    double acc[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) acc[j] = 0.0;
    if (n < d && t0 < L) {
        const float2 lf = a.s.poles[g * d + n], rf = a.s.residues[g * d + n];
        const double lr = lf.x, li = lf.y, rr = rf.x, ri = rf.y;
        double pr, pi;
        complex_pow(lr, li, (t0 == 0) ? 0 : t0 - 1, pr, pi);
        const int first = (t0 == 0) ? 1 : 0;
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            if (j >= first) {
                acc[j] = rr * pr - ri * pi;
                const double nr = lr * pr - li * pi;
                pi = lr * pi + li * pr;
                pr = nr;
            }
        }
    }
    double *row = part + (rl * DPAD + n) * LP;
#pragma unroll
    for (int j = 0; j < kRun; ++j) row[j] = acc[j];
    __syncthreads();
    double sq = 0.0;
    for (int tau = threadIdx.x; tau < TPB; tau += 256) {
        const int64_t t = tile * TPB + tau;
        if (t >= L) break;
        const int run = tau / kRun, j = tau % kRun;
        double hh = 0.0;
        for (int m = 0; m < d; ++m) hh += part[(run * DPAD + m) * LP + j];
        if (t == 0) hh = a.s.skip[g];
        const double e = hh - (double)a.target[g * L + t];
        a.e[g * L + t] = e;
        sq += e * e;
    }
    red[threadIdx.x] = sq;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.loss_part[g * a.tiles + tile] = red[0];
}

// Workgroup = (head g, mode n, chunk of 8192 taps).  Thread i takes the taps
// chunk start + i + 256 j (j < 32), so a wave reads 64 consecutive residuals
// per step; lambda^(t-1) and lambda^(t-2) advance by lambda^256 (binary
// powering once per thread).
__global__ __launch_bounds__(256) void distill_grad_kernel(DistillArgs a) {
    __shared__ double red[4][256];
    __shared__ double2 shared_pow[2];  // lambda^256, lambda^B
    const int64_t L = a.L, d = a.s.d;
    // workgroups go round-robin over the 8 XCDs: map them so that the d modes of
    // a head (which all read that head's residual) run on one XCD and share it in L2
    const int64_t nx = gridDim.x;
    const int64_t gn = (nx % 8 == 0) ? (int64_t)(blockIdx.x % 8) * (nx / 8) + blockIdx.x / 8 : blockIdx.x;
    const int64_t chunk = blockIdx.y;
    const int64_t g = gn / d;
    const int64_t tf = chunk * kDistillTile + threadIdx.x;  // this thread's first tap
    // lambda^(t - 2) at the thread's first walked tap t = lambda^B * lambda^e, with
    // B = chunk start - 2 (chunk > 0) or 0 and the thread's offset e < 512: the long
    // powerings (and lambda^256) once per workgroup (measured on MI355X, H = 32,
    // d = 32, L = 65536: 97 -> 80 us with the XCD mapping above)
    const int64_t B = chunk > 0 ? chunk * kDistillTile - 2 : 0;
    if (threadIdx.x == 0) {
        const float2 lf = a.s.poles[gn];
        double wr, wi, br, bi;
        complex_pow(lf.x, lf.y, 256, wr, wi);
        complex_pow(lf.x, lf.y, B, br, bi);
        shared_pow[0] = make_double2(wr, wi);
        shared_pow[1] = make_double2(br, bi);
    }
    __syncthreads();
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    if (tf < L) {
        const float2 lf = a.s.poles[gn], rf = a.s.residues[gn];
        const double lr = lf.x, li = lf.y, rr = rf.x, ri = rf.y;
        const double *e = a.e + g * L;
        int j0 = 0;
        if (tf < 2) {  // tap 0 has no modal part; tap 1 has lambda^0 = 1 and no lambda^(t-2) term
            if (tf == 1) s[0] += e[1];
            j0 = 1;
        }
        const int64_t ts = tf + 256 * j0;
        if (ts < L) {
            const double2 w2 = shared_pow[0], b2 = shared_pow[1];
            const double wr = w2.x, wi = w2.y;
            double er, ei;
            complex_pow(lr, li, ts - 2 - B, er, ei);
            double qr = b2.x * er - b2.y * ei, qi = b2.x * ei + b2.y * er;  // lambda^(t-2), t >= 2
            double pr = qr * lr - qi * li, pi = qr * li + qi * lr;           // lambda^(t-1)
            for (int j = j0; j < kDistillTile / 256; ++j) {
                const int64_t t = tf + 256 * (int64_t)j;
                if (t >= L) break;
                const double ev = e[t], k = (double)(t - 1);
                s[0] += ev * pr;
                s[1] += ev * pi;
                s[2] += ev * k * (rr * qr - ri * qi);
                s[3] += ev * k * (rr * qi + ri * qr);
                double nr = pr * wr - pi * wi;
                pi = pr * wi + pi * wr;
                pr = nr;
                nr = qr * wr - qi * wi;
                qi = qr * wi + qi * wr;
                qr = nr;
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) red[c][threadIdx.x] = s[c];
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (threadIdx.x < w)
#pragma unroll
            for (int c = 0; c < 4; ++c) red[c][threadIdx.x] += red[c][threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x < 4) a.grad_part[(gn * a.chunks + chunk) * 4 + threadIdx.x] = red[threadIdx.x][0];
}

// Threads sum each (head, mode)'s chunk partials into the gradients; wave w of
// workgroup b sums head 4 b + w's loss partials (lanes stride over the tiles,
// then a butterfly across the wave).
__global__ __launch_bounds__(256) void distill_finish_kernel(DistillArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t H = a.s.H, d = a.s.d;
    if (i < H * d) {
        double s[4] = {0.0, 0.0, 0.0, 0.0};
        for (int c = 0; c < a.chunks; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k) s[k] += a.grad_part[(i * a.chunks + c) * 4 + k];
        a.g_res[2 * i] = (float)(2.0 * s[0]);
        a.g_res[2 * i + 1] = (float)(-2.0 * s[1]);
        a.g_poles[2 * i] = (float)(2.0 * s[2]);
        a.g_poles[2 * i + 1] = (float)(-2.0 * s[3]);
    }
    const int lane = threadIdx.x % kWave;
    const int64_t g = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (g < H) {
        double l = 0.0;
        for (int t = lane; t < a.tiles; t += kWave) l += a.loss_part[g * a.tiles + t];
#pragma unroll
        for (int m = kWave / 2; m > 0; m >>= 1) l += __shfl_xor(l, m);
        if (lane == 0) {
            a.loss[g] = (float)l;
            a.g_skip[g] = (float)(2.0 * a.e[g * a.L]);
        }
    }
}

__device__ inline float adam_update(float p, float g, float &m, float &v, const AdamArgs &a) {
    m = a.beta1 * m + (1.f - a.beta1) * g;
    v = a.beta2 * v + (1.f - a.beta2) * g * g;
    const float mh = m / a.bc1, vh = v / a.bc2;
    return p - a.lr * mh / (sqrtf(vh) + a.eps);
}

__global__ __launch_bounds__(256) void distill_adam_kernel(AdamArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nm = a.H * a.d;
    if (i < nm) {
        float *m = a.m + 4 * i, *v = a.v + 4 * i;
        float lr = adam_update(a.poles[2 * i], a.g_poles[2 * i], m[0], v[0], a);
        float li = adam_update(a.poles[2 * i + 1], a.g_poles[2 * i + 1], m[1], v[1], a);
        const float r = sqrtf(lr * lr + li * li);
        if (r > a.r_max) {  // keep the recurrence stable
            lr *= a.r_max / r;
            li *= a.r_max / r;
        }
        a.poles[2 * i] = lr;
        a.poles[2 * i + 1] = li;
        a.residues[2 * i] = adam_update(a.residues[2 * i], a.g_res[2 * i], m[2], v[2], a);
        a.residues[2 * i + 1] = adam_update(a.residues[2 * i + 1], a.g_res[2 * i + 1], m[3], v[3], a);
    }
    if (i < a.H) {
        float *m = a.m + 4 * nm + i, *v = a.v + 4 * nm + i;
        a.skip[i] = adam_update(a.skip[i], a.g_skip[i], *m, *v, a);
    }
}

template <int DPAD>
hipError_t launch_residual(const DistillArgs &a, hipStream_t stream) {
    constexpr int TPB = (256 / DPAD) * kRun;
    const int64_t blocks = a.s.H * ((a.L + TPB - 1) / TPB);
    distill_residual_kernel<DPAD><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace

int distill_tiles(int64_t L, int64_t d) {
    int dpad = 1;
    while (dpad < d) dpad <<= 1;
    const int64_t tpb = (256 / dpad) * kRun;
    return (int)((L + tpb - 1) / tpb);
}

hipError_t launch_distill_grad(const DistillArgs &a, hipStream_t stream) {
    const int64_t d = a.s.d;
    hipError_t err;
    if (d <= 1) err = launch_residual<1>(a, stream);
    else if (d <= 2) err = launch_residual<2>(a, stream);
    else if (d <= 4) err = launch_residual<4>(a, stream);
    else if (d <= 8) err = launch_residual<8>(a, stream);
    else if (d <= 16) err = launch_residual<16>(a, stream);
    else if (d <= 32) err = launch_residual<32>(a, stream);
    else err = launch_residual<64>(a, stream);
    if (err != hipSuccess) return err;
    distill_grad_kernel<<<dim3((unsigned)(a.s.H * d), (unsigned)a.chunks), dim3(256), 0, stream>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t nb_grad = (a.s.H * d + 255) / 256, nb_loss = (a.s.H + 3) / 4;  // 4 waves per workgroup
    distill_finish_kernel<<<dim3((unsigned)(nb_grad > nb_loss ? nb_grad : nb_loss)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_distill_adam(const AdamArgs &a, hipStream_t stream) {
    const int64_t n = a.H * a.d > a.H ? a.H * a.d : a.H;
    distill_adam_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace hm
