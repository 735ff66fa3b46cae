// hm_api.cpp -- the C ABI declared in include/hyena_modal.h.
//
// Every entry point validates its arguments on the host first (sizes, pointers,
// alignment, workspace) and returns a status without touching the GPU when they
// are wrong.  Valid calls build an argument block and enqueue kernels on the
// caller's stream; nothing here allocates, frees or synchronises.
#include "hyena_modal.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "hm_internal.hpp"

// Device scratch of hyena_modal_prefill_noalloc: the prefill workspace for
// callers that cannot allocate.  Each GPU the library runs on holds its own
// copy of this array (HM_NOALLOC_SCRATCH_BYTES) from module load until the
// process ends.  Host code never passes its name to a kernel: the name is a
// host-side stand-in, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[HM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the current device, looked up once per device
// (with that device current) and kept.  No allocation happens here.
hm_status scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return HM_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return HM_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;  // guard against int64 overflow in offsets

bool aligned(const void *p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) % m) == 0; }

hm_status check_desc(const hm_desc *desc) {
    if (!desc) return HM_ERR_INVALID_ARG;
    if (desc->abi_version != HM_ABI_VERSION) return HM_ERR_INVALID_ARG;
    if (desc->act_dtype != HM_F32 && desc->act_dtype != HM_BF16) return HM_ERR_UNSUPPORTED;
    if (desc->batch < 0 || desc->channels < 1 || desc->heads < 1 || desc->modes < 1)
        return HM_ERR_INVALID_ARG;
    if (desc->channels % desc->heads != 0) return HM_ERR_INVALID_ARG;
    if (desc->modes > HM_MAX_MODES) return HM_ERR_UNSUPPORTED;
    if (!desc->poles || !desc->residues || !desc->skip) return HM_ERR_INVALID_ARG;
    if (!aligned(desc->poles, 8) || !aligned(desc->residues, 8) || !aligned(desc->skip, 4))
        return HM_ERR_UNSUPPORTED;
    if (desc->batch > kMaxElems / desc->channels) return HM_ERR_INVALID_ARG;
    if (desc->batch * desc->channels > kMaxElems / desc->modes) return HM_ERR_INVALID_ARG;
    return HM_OK;
}

hm::OpShape shape_of(const hm_desc *desc) {
    hm::OpShape s;
    s.B = desc->batch;
    s.D = desc->channels;
    s.H = desc->heads;
    s.d = desc->modes;
    s.P = desc->channels / desc->heads;
    s.act = desc->act_dtype == HM_BF16 ? hm::kBF16 : hm::kF32;
    s.poles = reinterpret_cast<const float2 *>(desc->poles);
    s.residues = reinterpret_cast<const float2 *>(desc->residues);
    s.skip = desc->skip;
    return s;
}

int elem_bytes(const hm_desc *desc) { return desc->act_dtype == HM_BF16 ? 2 : 4; }

hm_status check_act(const hm_desc *desc, const void *p) {
    if (!p) return HM_ERR_INVALID_ARG;
    if (!aligned(p, (uintptr_t)elem_bytes(desc))) return HM_ERR_UNSUPPORTED;
    return HM_OK;
}

hm_status check_chunk(int64_t chunk) {
    if (chunk < 0) return HM_ERR_INVALID_ARG;
    if (chunk > 0 && chunk % 64 != 0) return HM_ERR_UNSUPPORTED;
    return HM_OK;
}

hm_status check_opts(const hm_prefill_opts *opts, int64_t *chunk, int *algo) {
    *chunk = 0;
    *algo = hm::kAlgoAuto;
    if (!opts) return HM_OK;
    hm_status st = check_chunk(opts->chunk);
    if (st != HM_OK) return st;
    if (opts->algo != HM_PREFILL_AUTO && opts->algo != HM_PREFILL_SCAN && opts->algo != HM_PREFILL_MFMA)
        return HM_ERR_INVALID_ARG;
    *chunk = opts->chunk;
    *algo = opts->algo == HM_PREFILL_SCAN ? hm::kAlgoScan : opts->algo == HM_PREFILL_MFMA ? hm::kAlgoMfma
                                                                                              : hm::kAlgoAuto;
    return HM_OK;
}

// use_scratch: take the workspace from the per-device `scratch` array instead
// of the caller (workspace and ws_bytes are then ignored).
hm_status prefill_impl(const hm_desc *desc, int64_t L, const void *q, const void *k, const void *v,
                       int64_t ld_in, void *y, int64_t ld_y, const float *state_in, float *state_out,
                       void *workspace, size_t ws_bytes, void *stream, const hm_prefill_opts *opts,
                       bool use_scratch = false) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    int64_t chunk;
    int algo;
    if ((st = check_opts(opts, &chunk, &algo)) != HM_OK) return st;
    if (L < 0 || L > kMaxElems) return HM_ERR_INVALID_ARG;
    const hm::OpShape s = shape_of(desc);
    if (s.B > 0 && L > 0) {
        if ((st = check_act(desc, q)) != HM_OK || (st = check_act(desc, k)) != HM_OK ||
            (st = check_act(desc, v)) != HM_OK || (st = check_act(desc, y)) != HM_OK)
            return st;
        if (ld_in < s.D || ld_y < s.D) return HM_ERR_INVALID_ARG;
        if (s.B * L > kMaxElems / ld_in || s.B * L > kMaxElems / ld_y) return HM_ERR_INVALID_ARG;
    }
    if (s.B > 0) {
        if (!state_out) return HM_ERR_INVALID_ARG;
        if (!aligned(state_out, 8) || (state_in && !aligned(state_in, 8))) return HM_ERR_UNSUPPORTED;
    }
    const hm::PrefillPlan plan = hm::make_prefill_plan(s, L, chunk, algo);
    // grid limits: batch rows and chunks map to the y/z launch dimensions
    if (s.B > 65535 || plan.NC > 65535) return HM_ERR_UNSUPPORTED;
    if (algo == hm::kAlgoMfma && s.B > 0 && L > 0) {
        // the matrix-core path was asked for explicitly: shape and alignment must allow it
        const int esz = elem_bytes(desc);
        if (plan.algo != hm::kAlgoMfma || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
            !aligned(y, 16) || (ld_in * esz) % 16 != 0 || (ld_y * esz) % 16 != 0)
            return HM_ERR_UNSUPPORTED;
    }
    if (use_scratch) {
        if (s.B > 0 && plan.bytes > (size_t)HM_NOALLOC_SCRATCH_BYTES) return HM_ERR_WORKSPACE;
    } else if (s.B > 0 && plan.bytes > 0) {
        if (!workspace || ws_bytes < plan.bytes) return HM_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return HM_ERR_UNSUPPORTED;
    }
    if (s.B == 0) return HM_OK;
    if (use_scratch && (st = scratch_for_current_device(&workspace)) != HM_OK) return st;
    hm::PrefillArgs a;
    a.s = s;
    a.plan = plan;
    a.q = q;
    a.k = k;
    a.v = v;
    a.ld_in = ld_in;
    a.y = y;
    a.ld_y = ld_y;
    a.state_in = reinterpret_cast<const float2 *>(state_in);
    a.state_out = reinterpret_cast<float2 *>(state_out);
    a.ws = static_cast<unsigned char *>(workspace);
    const hipError_t err = hm::launch_prefill(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status workspace_impl(const hm_desc *desc, int64_t L, const hm_prefill_opts *opts, size_t *bytes) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    int64_t chunk;
    int algo;
    if ((st = check_opts(opts, &chunk, &algo)) != HM_OK) return st;
    if (!bytes || L < 0 || L > kMaxElems) return HM_ERR_INVALID_ARG;
    *bytes = desc->batch > 0 ? hm::make_prefill_plan(shape_of(desc), L, chunk, algo).bytes : 0;
    return HM_OK;
}

hm_status plan_impl(const hm_desc *desc, int64_t L, const hm_prefill_opts *opts, hm_prefill_info *info) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    int64_t chunk;
    int algo;
    if ((st = check_opts(opts, &chunk, &algo)) != HM_OK) return st;
    if (!info || L < 0 || L > kMaxElems) return HM_ERR_INVALID_ARG;
    const hm::PrefillPlan plan = hm::make_prefill_plan(shape_of(desc), L, chunk, algo);
    if (algo == hm::kAlgoMfma && plan.algo != hm::kAlgoMfma) return HM_ERR_UNSUPPORTED;
    info->algo = plan.algo == hm::kAlgoMfma ? HM_PREFILL_MFMA : HM_PREFILL_SCAN;
    info->channel_tile = plan.algo == hm::kAlgoMfma ? hm::mfma_channel_tile(shape_of(desc)) : 0;
    info->chunk = plan.T;
    info->n_chunks = plan.NC;
    info->workspace_bytes = desc->batch > 0 ? plan.bytes : 0;
    return HM_OK;
}

}  // namespace

extern "C" {

int hm_abi_version(void) { return HM_ABI_VERSION; }

const char *hm_status_string(hm_status status) {
    switch (status) {
        case HM_OK: return "HM_OK";
        case HM_ERR_INVALID_ARG: return "HM_ERR_INVALID_ARG: invalid argument";
        case HM_ERR_UNSUPPORTED: return "HM_ERR_UNSUPPORTED: unsupported dtype, size or alignment";
        case HM_ERR_WORKSPACE: return "HM_ERR_WORKSPACE: workspace missing or too small";
        case HM_ERR_HIP: return "HM_ERR_HIP: kernel launch failed";
    }
    return "unknown hm_status";
}

hm_status hyena_modal_prefill_workspace(const hm_desc *desc, int64_t L, size_t *bytes) {
    return workspace_impl(desc, L, nullptr, bytes);
}

hm_status hyena_modal_prefill_workspace_ex(const hm_desc *desc, int64_t L, const hm_prefill_opts *opts,
                                           size_t *bytes) {
    return workspace_impl(desc, L, opts, bytes);
}

hm_status hyena_modal_prefill_plan(const hm_desc *desc, int64_t L, const hm_prefill_opts *opts,
                                   hm_prefill_info *info) {
    return plan_impl(desc, L, opts, info);
}

hm_status hyena_modal_prefill(const hm_desc *desc, int64_t L, const void *q, const void *k,
                              const void *v, int64_t ld_in, void *y, int64_t ld_y,
                              const float *state_in, float *state_out, void *workspace,
                              size_t ws_bytes, void *stream) {
    return prefill_impl(desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out, workspace, ws_bytes,
                        stream, nullptr);
}

hm_status hyena_modal_prefill_ex(const hm_desc *desc, int64_t L, const void *q, const void *k,
                                 const void *v, int64_t ld_in, void *y, int64_t ld_y,
                                 const float *state_in, float *state_out, void *workspace,
                                 size_t ws_bytes, const hm_prefill_opts *opts, void *stream) {
    return prefill_impl(desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out, workspace, ws_bytes,
                        stream, opts);
}

hm_status hyena_modal_prefill_noalloc(const hm_desc *desc, int64_t L, const void *q, const void *k,
                                      const void *v, int64_t ld_in, void *y, int64_t ld_y,
                                      const float *state_in, float *state_out,
                                      const hm_prefill_opts *opts, void *stream) {
    return prefill_impl(desc, L, q, k, v, ld_in, y, ld_y, state_in, state_out, nullptr, 0, stream, opts,
                        /*use_scratch=*/true);
}

hm_status hyena_modal_decode_step(const hm_desc *desc, const void *q, const void *k, const void *v,
                                  int64_t ld_in, void *y, int64_t ld_y, float *state, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    const hm::OpShape s = shape_of(desc);
    if (s.B == 0) return HM_OK;
    if ((st = check_act(desc, q)) != HM_OK || (st = check_act(desc, k)) != HM_OK ||
        (st = check_act(desc, v)) != HM_OK || (st = check_act(desc, y)) != HM_OK)
        return st;
    if (!state) return HM_ERR_INVALID_ARG;
    if (!aligned(state, 8)) return HM_ERR_UNSUPPORTED;
    if (ld_in < s.D || ld_y < s.D) return HM_ERR_INVALID_ARG;
    if (s.B > kMaxElems / ld_in || s.B > kMaxElems / ld_y) return HM_ERR_INVALID_ARG;
    if (s.B > 65535 || s.D * 4 > INT32_MAX) return HM_ERR_UNSUPPORTED;  // grid limits
    hm::DecodeArgs a;
    a.s = s;
    a.q = q;
    a.k = k;
    a.v = v;
    a.ld_in = ld_in;
    a.y = y;
    a.ld_y = ld_y;
    a.state = reinterpret_cast<float2 *>(state);
    const hipError_t err = hm::launch_decode_step(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_filter_materialize(const hm_desc *desc, int64_t L, float *h_out, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (L < 0 || L > kMaxElems / desc->heads) return HM_ERR_INVALID_ARG;
    if (L == 0) return HM_OK;
    // grid limit: one workgroup per head and (at least) 128 taps
    if ((L + 127) / 128 > (int64_t)INT32_MAX / desc->heads) return HM_ERR_UNSUPPORTED;
    if (!h_out) return HM_ERR_INVALID_ARG;
    if (!aligned(h_out, 4)) return HM_ERR_UNSUPPORTED;
    hm::FilterArgs a;
    a.s = shape_of(desc);
    a.L = L;
    a.h = h_out;
    const hipError_t err = hm::launch_filter(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

static hm_status fir_check(const hm_desc *desc, const void *cache, int64_t cache_len) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (cache_len < 1 || desc->batch > kMaxElems / cache_len || desc->batch * cache_len > kMaxElems / desc->channels)
        return HM_ERR_INVALID_ARG;
    if (desc->batch > 0 && !cache) return HM_ERR_INVALID_ARG;
    if (desc->channels % 8 != 0 || (desc->channels / desc->heads) % 8 != 0) return HM_ERR_UNSUPPORTED;
    if (desc->batch > 0 && !aligned(cache, 16)) return HM_ERR_UNSUPPORTED;
    return HM_OK;
}

hm_status hyena_fir_workspace(const hm_desc *desc, size_t *bytes) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!bytes) return HM_ERR_INVALID_ARG;
    *bytes = (size_t)hm::fir_ranges(desc->batch, desc->channels) * desc->batch * desc->channels * sizeof(float);
    return HM_OK;
}

hm_status hyena_fir_cache_fill(const hm_desc *desc, int64_t L, const void *k, const void *v, int64_t ld_in,
                               void *u_cache, int64_t cache_len, void *stream) {
    hm_status st = fir_check(desc, u_cache, cache_len);
    if (st != HM_OK) return st;
    if (L < 0 || L > cache_len) return HM_ERR_INVALID_ARG;
    if (desc->batch == 0 || L == 0) return HM_OK;
    if ((st = check_act(desc, k)) != HM_OK || (st = check_act(desc, v)) != HM_OK) return st;
    if (ld_in < desc->channels || desc->batch * L > kMaxElems / ld_in) return HM_ERR_INVALID_ARG;
    hm::FirArgs a{};
    a.s = shape_of(desc);
    a.k = k;
    a.v = v;
    a.ld_in = ld_in;
    a.cache = u_cache;
    a.cache_len = cache_len;
    const hipError_t err = hm::launch_fir_fill(a, L, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

static hm_status fir_decode_impl(const hm_desc *desc, const float *h, int64_t h_len, int64_t window, int64_t t,
                                 const void *q, const void *k, const void *v, int64_t ld_in, void *y,
                                 int64_t ld_y, void *u_cache, int64_t cache_len, void *workspace,
                                 size_t ws_bytes, int32_t loads, void *stream) {
    hm_status st = fir_check(desc, u_cache, cache_len);
    if (st != HM_OK) return st;
    if (loads < 0 || loads > 2) return HM_ERR_INVALID_ARG;
    // float32 non-temporal loads need the 512-channel block split
    if (loads == 2 && desc->act_dtype == HM_F32 && desc->channels % 512 != 0) return HM_ERR_UNSUPPORTED;
    if (t < 0 || t >= cache_len || window < 0) return HM_ERR_INVALID_ARG;
    const int64_t taps = (window == 0 || window > t + 1) ? t + 1 : window;
    if (!h || h_len < taps || h_len > kMaxElems / desc->heads) return HM_ERR_INVALID_ARG;
    if (!aligned(h, 4)) return HM_ERR_UNSUPPORTED;
    if (desc->batch == 0) return HM_OK;
    if ((st = check_act(desc, q)) != HM_OK || (st = check_act(desc, k)) != HM_OK ||
        (st = check_act(desc, v)) != HM_OK || (st = check_act(desc, y)) != HM_OK)
        return st;
    if (ld_in < desc->channels || ld_y < desc->channels) return HM_ERR_INVALID_ARG;
    if (desc->batch > kMaxElems / ld_in || desc->batch > kMaxElems / ld_y) return HM_ERR_INVALID_ARG;
    if (desc->batch > 65535) return HM_ERR_UNSUPPORTED;  // grid z
    const int R = hm::fir_ranges(desc->batch, desc->channels);
    const size_t need = (size_t)R * desc->batch * desc->channels * sizeof(float);
    if (!workspace || ws_bytes < need) return HM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HM_ERR_UNSUPPORTED;
    hm::FirArgs a{};
    a.s = shape_of(desc);
    a.h = h;
    a.h_len = h_len;
    a.t = t;
    a.lo = t + 1 - taps;
    a.R = R;
    a.q = q;
    a.k = k;
    a.v = v;
    a.ld_in = ld_in;
    a.y = y;
    a.ld_y = ld_y;
    a.cache = u_cache;
    a.cache_len = cache_len;
    a.part = static_cast<float *>(workspace);
    a.loads = loads;
    const hipError_t err = hm::launch_fir_decode(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_fir_decode_step(const hm_desc *desc, const float *h, int64_t h_len, int64_t window, int64_t t,
                                const void *q, const void *k, const void *v, int64_t ld_in, void *y,
                                int64_t ld_y, void *u_cache, int64_t cache_len, void *workspace,
                                size_t ws_bytes, void *stream) {
    return fir_decode_impl(desc, h, h_len, window, t, q, k, v, ld_in, y, ld_y, u_cache, cache_len, workspace,
                           ws_bytes, HM_FIR_LOADS_AUTO, stream);
}

hm_status hyena_fir_decode_step_ex(const hm_desc *desc, const float *h, int64_t h_len, int64_t window, int64_t t,
                                   const void *q, const void *k, const void *v, int64_t ld_in, void *y,
                                   int64_t ld_y, void *u_cache, int64_t cache_len, void *workspace,
                                   size_t ws_bytes, int32_t loads, void *stream) {
    return fir_decode_impl(desc, h, h_len, window, t, q, k, v, ld_in, y, ld_y, u_cache, cache_len, workspace,
                           ws_bytes, loads, stream);
}

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// FFT-prefill workspace: taps [H][L] fp32 | twiddles [N/2] | spectra [H][N] (complex fp32)
// | past N = 8192, the multi-pass work buffer [B][N][D/2] (complex fp32).
static size_t fft_workspace_bytes(const hm_desc *desc, int64_t L, size_t *off_tw, size_t *off_spec,
                                  size_t *off_z) {
    const int logn = hm::fft_log_n(L);
    const size_t N = size_t(1) << logn;
    *off_tw = align_up((size_t)desc->heads * L * sizeof(float));
    *off_spec = align_up(*off_tw + N / 2 * 8);
    *off_z = align_up(*off_spec + (size_t)desc->heads * N * 8);
    if (logn <= hm::kFftMaxLogN) return *off_z;
    return *off_z + (size_t)desc->batch * N * (size_t)(desc->channels / 2) * 8;
}

static constexpr int64_t kFftMaxL = int64_t(1) << (hm::kFftMaxLogNLong - 1);

// the multi-pass work buffer (B x N x D/2 complex) must stay addressable
static bool fft_long_fits(const hm_desc *desc, int64_t L) {
    const int logn = hm::fft_log_n(L);
    if (logn <= hm::kFftMaxLogN) return true;
    return desc->batch * (desc->channels / 2) <= kMaxElems / (int64_t(1) << logn);
}

hm_status hyena_fft_prefill_workspace(const hm_desc *desc, int64_t L, size_t *bytes) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!bytes || L < 0) return HM_ERR_INVALID_ARG;
    if (L > kFftMaxL || (L > 0 && !fft_long_fits(desc, L))) return HM_ERR_UNSUPPORTED;
    size_t a, b, c;
    *bytes = L == 0 ? 0 : fft_workspace_bytes(desc, L, &a, &b, &c);
    return HM_OK;
}

hm_status hyena_fft_prefill(const hm_desc *desc, int64_t L, const void *q, const void *k, const void *v,
                            int64_t ld_in, void *y, int64_t ld_y, void *workspace, size_t ws_bytes, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (L < 0) return HM_ERR_INVALID_ARG;
    if (L > kFftMaxL) return HM_ERR_UNSUPPORTED;
    if (desc->batch == 0 || L == 0) return HM_OK;
    if (!fft_long_fits(desc, L)) return HM_ERR_UNSUPPORTED;
    if ((desc->channels / desc->heads) % 2 != 0) return HM_ERR_UNSUPPORTED;  // channel pairs within a head
    if (desc->batch > 65535 || desc->channels / 2 > INT32_MAX) return HM_ERR_UNSUPPORTED;
    if ((st = check_act(desc, q)) != HM_OK || (st = check_act(desc, k)) != HM_OK ||
        (st = check_act(desc, v)) != HM_OK || (st = check_act(desc, y)) != HM_OK)
        return st;
    if (ld_in < desc->channels || ld_y < desc->channels) return HM_ERR_INVALID_ARG;
    if (desc->batch * L > kMaxElems / ld_in || desc->batch * L > kMaxElems / ld_y) return HM_ERR_INVALID_ARG;
    size_t off_tw, off_spec, off_z;
    const size_t need = fft_workspace_bytes(desc, L, &off_tw, &off_spec, &off_z);
    if (!workspace || ws_bytes < need) return HM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HM_ERR_UNSUPPORTED;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    hm::FftArgs a{};
    a.s = shape_of(desc);
    a.L = L;
    a.logn = hm::fft_log_n(L);
    a.np = hm::fft_pairs_per_group(a.s.P, a.logn);
    a.q = q;
    a.k = k;
    a.v = v;
    a.ld_in = ld_in;
    a.y = y;
    a.ld_y = ld_y;
    a.h = reinterpret_cast<float *>(ws);
    a.tw = reinterpret_cast<float2 *>(ws + off_tw);
    a.spec = reinterpret_cast<float2 *>(ws + off_spec);
    a.z = a.logn > hm::kFftMaxLogN ? reinterpret_cast<float2 *>(ws + off_z) : nullptr;
    hm::FilterArgs f;
    f.s = a.s;
    f.L = L;
    f.h = a.h;
    hipError_t err = hm::launch_filter(f, static_cast<hipStream_t>(stream));
    if (err == hipSuccess) err = hm::launch_fft_prefill(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

// Distillation workspace: residual [H][L] f64 | loss partials [H][tiles] f64 | gradient partials [H*d][chunks][4] f64.
static size_t distill_layout(const hm_desc *desc, int64_t L, size_t *off_loss, size_t *off_grad, int *tiles,
                             int *chunks) {
    *tiles = hm::distill_tiles(L, desc->modes);
    *chunks = (int)((L + hm::kDistillTile - 1) / hm::kDistillTile);
    *off_loss = align_up((size_t)desc->heads * L * sizeof(double));
    *off_grad = align_up(*off_loss + (size_t)desc->heads * *tiles * sizeof(double));
    return *off_grad + (size_t)desc->heads * desc->modes * *chunks * 4 * sizeof(double);
}

static bool distill_l_ok(const hm_desc *desc, int64_t L) {
    return L >= 1 && L <= kMaxElems / desc->heads && (L + hm::kDistillTile - 1) / hm::kDistillTile <= 65535 &&
           (int64_t)desc->heads * ((L + 127) / 128) <= INT32_MAX;
}

hm_status hyena_distill_workspace(const hm_desc *desc, int64_t L, size_t *bytes) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!bytes || !distill_l_ok(desc, L)) return HM_ERR_INVALID_ARG;
    size_t a, b;
    int t, c;
    *bytes = distill_layout(desc, L, &a, &b, &t, &c);
    return HM_OK;
}

hm_status hyena_distill_grad(const hm_desc *desc, int64_t L, const float *h_target, float *loss, float *g_poles,
                             float *g_res, float *g_skip, void *workspace, size_t ws_bytes, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!distill_l_ok(desc, L)) return HM_ERR_INVALID_ARG;
    if (!h_target || !loss || !g_poles || !g_res || !g_skip) return HM_ERR_INVALID_ARG;
    if (!aligned(h_target, 4) || !aligned(loss, 4) || !aligned(g_poles, 4) || !aligned(g_res, 4) ||
        !aligned(g_skip, 4))
        return HM_ERR_UNSUPPORTED;
    hm::DistillArgs a{};
    size_t off_loss, off_grad;
    const size_t need = distill_layout(desc, L, &off_loss, &off_grad, &a.tiles, &a.chunks);
    if (!workspace || ws_bytes < need) return HM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HM_ERR_UNSUPPORTED;
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    a.s = shape_of(desc);
    a.L = L;
    a.target = h_target;
    a.e = reinterpret_cast<double *>(ws);
    a.loss_part = reinterpret_cast<double *>(ws + off_loss);
    a.grad_part = reinterpret_cast<double *>(ws + off_grad);
    a.loss = loss;
    a.g_poles = g_poles;
    a.g_res = g_res;
    a.g_skip = g_skip;
    const hipError_t err = hm::launch_distill_grad(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_distill_adam_step(int64_t H, int64_t d, float *poles, float *residues, float *skip,
                                  const float *g_poles, const float *g_res, const float *g_skip, float *m, float *v,
                                  int64_t step, float lr, float beta1, float beta2, float eps, float r_max,
                                  void *stream) {
    if (H < 1 || d < 1 || d > HM_MAX_MODES || H > INT32_MAX / 64) return HM_ERR_INVALID_ARG;
    if (!poles || !residues || !skip || !g_poles || !g_res || !g_skip || !m || !v) return HM_ERR_INVALID_ARG;
    if (step < 1 || !(lr > 0.f) || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f) ||
        !(eps > 0.f) || !(r_max > 0.f && r_max < 1.f))
        return HM_ERR_INVALID_ARG;
    for (const void *p : {(const void *)poles, (const void *)residues, (const void *)skip, (const void *)g_poles,
                          (const void *)g_res, (const void *)g_skip, (const void *)m, (const void *)v})
        if (!aligned(p, 4)) return HM_ERR_UNSUPPORTED;
    hm::AdamArgs a;
    a.H = H;
    a.d = d;
    a.poles = poles;
    a.residues = residues;
    a.skip = skip;
    a.g_poles = g_poles;
    a.g_res = g_res;
    a.g_skip = g_skip;
    a.m = m;
    a.v = v;
    a.lr = lr;
    a.beta1 = beta1;
    a.beta2 = beta2;
    a.eps = eps;
    a.r_max = r_max;
    a.bc1 = (float)(1.0 - std::pow((double)beta1, (double)step));
    a.bc2 = (float)(1.0 - std::pow((double)beta2, (double)step));
    const hipError_t err = hm::launch_distill_adam(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_row_rms(const void *x, int64_t M, int64_t D, int64_t ld, float eps, float *inv_rms,
                        void *stream) {
    if (M < 0 || D < 1 || ld < D || M > kMaxElems / ld || !(eps >= 0.0f)) return HM_ERR_INVALID_ARG;
    if (M == 0) return HM_OK;
    if (!x || !inv_rms) return HM_ERR_INVALID_ARG;
    if (!aligned(x, 2) || !aligned(inv_rms, 4)) return HM_ERR_UNSUPPORTED;
    if (M > int64_t(UINT32_MAX) * 4) return HM_ERR_UNSUPPORTED;
    hm::RmsArgs a;
    a.x = x;
    a.M = M;
    a.D = D;
    a.ld = ld;
    a.eps = eps;
    a.inv_rms = inv_rms;
    a.vec = aligned(x, 16) && D % 8 == 0 && ld % 8 == 0;
    const hipError_t err = hm::launch_row_rms(a, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

static hm_status dense_impl(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *W, int64_t ldw,
                     const float *row_scale, bool rms, float eps, void *C, int64_t ldc, void *workspace,
                     size_t ws_bytes, void *stream) {
    if (M < 0 || N < 0 || K < 1) return HM_ERR_INVALID_ARG;
    if (lda < K || ldw < K || ldc < N) return HM_ERR_INVALID_ARG;
    if (M > kMaxElems / lda || N > kMaxElems / ldw || M > kMaxElems / (ldc > 0 ? ldc : 1))
        return HM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return HM_OK;
    if (!A || !W || !C) return HM_ERR_INVALID_ARG;
    if (K % 64 != 0 || lda % 8 != 0 || ldw % 8 != 0) return HM_ERR_UNSUPPORTED;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(C, 2) || (row_scale && !aligned(row_scale, 4)))
        return HM_ERR_UNSUPPORTED;
    if (((M + 127) / 128) * ((N + 255) / 256) > INT32_MAX) return HM_ERR_UNSUPPORTED;
    const size_t ws_need = hm::splitk_workspace_bytes(M, N, K);
    if (workspace && ws_need > 0) {
        if (ws_bytes < ws_need) return HM_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return HM_ERR_UNSUPPORTED;
    }
    hm::GemmArgs g;
    g.M = M;
    g.N = N;
    g.K = K;
    g.A = A;
    g.lda = lda;
    g.W = W;
    g.ldw = ldw;
    g.row_scale = row_scale;
    g.C = C;
    g.ldc = ldc;
    g.rms = rms;
    g.rms_eps = eps;
    g.ws = (workspace && ws_need > 0) ? static_cast<unsigned char *>(workspace) : nullptr;
    g.ws_bytes = ws_bytes;
    const hipError_t err = hm::launch_gemm(g, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_dense_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *W,
                           int64_t ldw, const float *row_scale, void *C, int64_t ldc, void *stream) {
    return dense_impl(M, N, K, A, lda, W, ldw, row_scale, false, 0.0f, C, ldc, nullptr, 0, stream);
}

hm_status hyena_dense_rms_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *W,
                               int64_t ldw, float eps, void *C, int64_t ldc, void *stream) {
    if (!(eps >= 0.0f)) return HM_ERR_INVALID_ARG;
    return dense_impl(M, N, K, A, lda, W, ldw, nullptr, true, eps, C, ldc, nullptr, 0, stream);
}

hm_status hyena_dense_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes) {
    if (!bytes || M < 0 || N < 0 || K < 1) return HM_ERR_INVALID_ARG;
    *bytes = hm::splitk_workspace_bytes(M, N, K);
    return HM_OK;
}

hm_status hyena_dense_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *W,
                              int64_t ldw, const float *row_scale, void *C, int64_t ldc, void *workspace,
                              size_t ws_bytes, void *stream) {
    return dense_impl(M, N, K, A, lda, W, ldw, row_scale, false, 0.0f, C, ldc, workspace, ws_bytes, stream);
}

hm_status hyena_dense_rms_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *W,
                                  int64_t ldw, float eps, void *C, int64_t ldc, void *workspace, size_t ws_bytes,
                                  void *stream) {
    if (!(eps >= 0.0f)) return HM_ERR_INVALID_ARG;
    return dense_impl(M, N, K, A, lda, W, ldw, nullptr, true, eps, C, ldc, workspace, ws_bytes, stream);
}

hm_status hyena_pack_in_proj_bf16(int64_t D, int64_t K, const void *w_in, int64_t ldw, void *w_packed,
                                  void *stream) {
    if (D < 0 || K < 1 || ldw < K) return HM_ERR_INVALID_ARG;
    if (D == 0) return HM_OK;
    if (!w_in || !w_packed) return HM_ERR_INVALID_ARG;
    if (D % 16 != 0 || K % 8 != 0 || ldw % 8 != 0) return HM_ERR_UNSUPPORTED;
    if (!aligned(w_in, 16) || !aligned(w_packed, 16)) return HM_ERR_UNSUPPORTED;
    if (3 * D > INT32_MAX || 3 * D > kMaxElems / ldw) return HM_ERR_INVALID_ARG;
    const hipError_t err = hm::launch_pack_in_proj(D, K, w_in, ldw, w_packed, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

// ------------------------------------------------------------------ generation step, deferred state

static hm_status prep_of(const hm_desc *desc, float *state, const float *u_prev, float *rho, hm::PrepArgs *p) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    const hm::OpShape s = shape_of(desc);
    if (s.B > 0 && (!state || !u_prev || !rho)) return HM_ERR_INVALID_ARG;
    if (!hm::prepare_supported(s.d) || s.P % 2 != 0) return HM_ERR_UNSUPPORTED;
    if (s.B > 0 && (!aligned(state, 16) || !aligned(u_prev, 8) || !aligned(rho, 8))) return HM_ERR_UNSUPPORTED;
    p->B = s.B;
    p->D = s.D;
    p->H = s.H;
    p->P = s.P;
    p->d = s.d;
    p->state = reinterpret_cast<float2 *>(state);
    p->u_prev = u_prev;
    p->rho = rho;
    p->poles = s.poles;
    p->residues = s.residues;
    return HM_OK;
}

hm_status hyena_decode_prepare(const hm_desc *desc, float *state, const float *u_prev, float *rho, void *stream) {
    hm::PrepArgs p;
    hm_status st = prep_of(desc, state, u_prev, rho, &p);
    if (st != HM_OK) return st;
    if (p.B == 0) return HM_OK;
    const hipError_t err = hm::launch_prepare(p, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_layer_gate_bf16(const hm_desc *desc, const void *x, int64_t ldx, const void *w_packed, float eps,
                                const float *rho, float *u_prev, void *y, int64_t ld_y, const hm_desc *next,
                                float *next_state, const float *next_u_prev, float *next_rho, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!(eps >= 0.0f)) return HM_ERR_INVALID_ARG;
    hm::GemmArgs g;
    if (next && (st = prep_of(next, next_state, next_u_prev, next_rho, &g.prep)) != HM_OK) return st;
    const hm::OpShape s = shape_of(desc);
    if (s.B == 0) {
        if (g.prep.B == 0) return HM_OK;
        const hipError_t err = hm::launch_prepare(g.prep, static_cast<hipStream_t>(stream));
        return err == hipSuccess ? HM_OK : HM_ERR_HIP;
    }
    if (!x || !w_packed || !rho || !u_prev || !y) return HM_ERR_INVALID_ARG;
    if (ldx < s.D || ld_y < s.D) return HM_ERR_INVALID_ARG;
    if (s.act != hm::kBF16 || s.B > 64 || s.D != 2048 || s.P % 16 != 0) return HM_ERR_UNSUPPORTED;
    if (ldx % 8 != 0 || ld_y % 2 != 0) return HM_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 4) || !aligned(rho, 8) || !aligned(u_prev, 8))
        return HM_ERR_UNSUPPORTED;
    g.M = s.B;
    g.N = 3 * s.D;
    g.K = s.D;
    g.A = x;
    g.lda = ldx;
    g.W = w_packed;
    g.ldw = s.D;
    g.row_scale = nullptr;
    g.C = nullptr;
    g.ldc = 0;
    g.rms = true;
    g.rms_eps = eps;
    g.skip = s.skip;
    g.P = s.P;
    g.H = s.H;
    g.y = y;
    g.ld_y = ld_y;
    g.rho = rho;
    g.u_prev = u_prev;
    const hipError_t err = hm::launch_layer_gate(g, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

hm_status hyena_layer_step_bf16(const hm_desc *desc, const void *x, int64_t ldx, const void *w_packed, float eps,
                                float *state, void *y, int64_t ld_y, void *stream) {
    hm_status st = check_desc(desc);
    if (st != HM_OK) return st;
    if (!(eps >= 0.0f)) return HM_ERR_INVALID_ARG;
    const hm::OpShape s = shape_of(desc);
    if (s.B == 0) return HM_OK;
    if (!x || !w_packed || !state || !y) return HM_ERR_INVALID_ARG;
    if (ldx < s.D || ld_y < s.D) return HM_ERR_INVALID_ARG;
    if (s.act != hm::kBF16 || s.B > 64 || s.D != 2048 || (s.d != 8 && s.d != 16) || s.P % 16 != 0)
        return HM_ERR_UNSUPPORTED;
    if (ldx % 8 != 0 || ld_y % 2 != 0) return HM_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(state, 16) || !aligned(y, 4))
        return HM_ERR_UNSUPPORTED;
    hm::GemmArgs g;
    g.M = s.B;
    g.N = 3 * s.D;
    g.K = s.D;
    g.A = x;
    g.lda = ldx;
    g.W = w_packed;
    g.ldw = s.D;
    g.row_scale = nullptr;
    g.C = nullptr;
    g.ldc = 0;
    g.rms = true;
    g.rms_eps = eps;
    g.state = reinterpret_cast<float2 *>(state);
    g.poles = s.poles;
    g.residues = s.residues;
    g.skip = s.skip;
    g.P = s.P;
    g.H = s.H;
    g.y = y;
    g.ld_y = ld_y;
    const hipError_t err = hm::launch_layer_step(g, (int)s.d, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? HM_OK : HM_ERR_HIP;
}

}  // extern "C"
