// Drives the library's host side -- descriptor and argument validation, the
// prefill plan, every workspace query -- for a build whose host code carries
// AddressSanitizer and UndefinedBehaviorSanitizer.  Only calls that end before
// any HIP launch are made (invalid arguments, size queries, empty problems),
// so no GPU is needed.  Exit status 0 when every call returns the status its
// header documents.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hyena_modal.h"

static int failures = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        const hm_status got_ = (call);                                                      \
        if (got_ != (want)) {                                                               \
            std::printf("line %d: %s -> %d, want %d\n", __LINE__, #call, (int)got_, (int)(want)); \
            ++failures;                                                                     \
        }                                                                                   \
    } while (0)

alignas(256) static unsigned char arena[1 << 16];

int main() {
    float poles[64 * 2 * 4] = {}, res[64 * 2 * 4] = {}, skip[4] = {};
    hm_desc ok{HM_ABI_VERSION, HM_F32, 2, 256, 2, 16, poles, res, skip};
    void *const P = arena;  // stand-in device pointer, 256-byte aligned; never dereferenced here
    size_t n = 0;

    if (hm_abi_version() != HM_ABI_VERSION) ++failures;
    for (int s = 0; s <= 5; ++s)
        if (!hm_status_string(static_cast<hm_status>(s)) || !*hm_status_string(static_cast<hm_status>(s))) ++failures;

    // descriptors
    hm_desc bad = ok;
    EXPECT(hyena_modal_prefill_workspace(nullptr, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.abi_version = 99;  EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.act_dtype = 7;     EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_UNSUPPORTED);
    bad = ok; bad.channels = 255;    EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.modes = 0;         EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.modes = 65;        EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_UNSUPPORTED);
    bad = ok; bad.batch = -1;        EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.poles = nullptr;   EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);
    bad = ok; bad.residues = reinterpret_cast<const float *>(arena + 1);
    EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_UNSUPPORTED);
    bad = ok; bad.batch = int64_t(1) << 40; bad.channels = int64_t(1) << 20; bad.heads = 1;
    EXPECT(hyena_modal_prefill_workspace(&bad, 64, &n), HM_ERR_INVALID_ARG);  // B * D overflows the element limit

    // prefill: workspace, plan, argument checks
    EXPECT(hyena_modal_prefill_workspace(&ok, 0, &n), HM_OK);
    EXPECT(hyena_modal_prefill_workspace(&ok, -1, &n), HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_prefill_workspace(&ok, 4096, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_prefill_workspace(&ok, int64_t(1) << 50, &n), HM_ERR_INVALID_ARG);
    size_t need = 0;
    EXPECT(hyena_modal_prefill_workspace(&ok, 65536, &need), HM_OK);
    hm_prefill_opts o{};
    hm_prefill_info info{};
    for (int algo = 0; algo <= 2; ++algo)
        for (int64_t chunk : {int64_t(0), int64_t(64), int64_t(4096)}) {
            o.chunk = chunk;
            o.algo = algo;
            EXPECT(hyena_modal_prefill_plan(&ok, 65536, &o, &info), HM_OK);
            EXPECT(hyena_modal_prefill_workspace_ex(&ok, 65536, &o, &n), HM_OK);
            if (n != info.workspace_bytes) ++failures;
        }
    o.chunk = 100; o.algo = 0;  // not a multiple of 64
    EXPECT(hyena_modal_prefill_plan(&ok, 4096, &o, &info), HM_ERR_UNSUPPORTED);
    o.chunk = -64;
    EXPECT(hyena_modal_prefill_plan(&ok, 4096, &o, &info), HM_ERR_INVALID_ARG);
    o.chunk = 0; o.algo = 5;
    EXPECT(hyena_modal_prefill_plan(&ok, 4096, &o, &info), HM_ERR_INVALID_ARG);
    bad = ok; bad.modes = 12; o.algo = HM_PREFILL_MFMA;
    EXPECT(hyena_modal_prefill_plan(&bad, 4096, &o, &info), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_modal_prefill_plan(&ok, 4096, nullptr, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_prefill(&ok, 64, nullptr, P, P, 256, P, 256, nullptr, (float *)P, P, need, nullptr),
           HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_prefill(&ok, 64, P, P, P, 255, P, 256, nullptr, (float *)P, P, need, nullptr),
           HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_prefill(&ok, 65536, P, P, P, 256, P, 256, nullptr, (float *)P, P, need - 1, nullptr),
           HM_ERR_WORKSPACE);
    EXPECT(hyena_modal_prefill(&ok, 65536, P, P, P, 256, P, 256, nullptr, (float *)P, arena + 16, need, nullptr),
           HM_ERR_UNSUPPORTED);

    // decode, filter
    EXPECT(hyena_modal_decode_step(&ok, P, P, P, 256, nullptr, 256, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_modal_decode_step(&ok, P, P, P, 100, P, 256, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    bad = ok; bad.batch = 65536;
    EXPECT(hyena_modal_decode_step(&bad, P, P, P, 256, P, 256, (float *)P, nullptr), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_filter_materialize(&ok, -1, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_filter_materialize(&ok, 64, nullptr, nullptr), HM_ERR_INVALID_ARG);

    // projections
    EXPECT(hyena_row_rms(P, -1, 64, 64, 1e-6f, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_row_rms(P, 4, 64, 32, 1e-6f, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_row_rms(P, 4, 64, 64, -1.0f, (float *)P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_dense_bf16(0, 128, 256, P, 256, P, 256, nullptr, P, 128, nullptr), HM_OK);  // empty: no launch
    EXPECT(hyena_dense_bf16(64, 128, 96, P, 96, P, 96, nullptr, P, 128, nullptr), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_dense_bf16(64, 128, 256, arena + 2, 256, P, 256, nullptr, P, 128, nullptr), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_dense_rms_bf16(64, 128, 256, P, 256, P, 256, -1.0f, P, 128, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_dense_workspace(64, 2048, 1024, &n), HM_OK);
    if (n != size_t(32) * 4 * (4096 + 64) * 4) ++failures;
    EXPECT(hyena_dense_workspace(64, 2048, 2048, &n), HM_OK);
    if (n != 0) ++failures;
    EXPECT(hyena_dense_workspace(-1, 8, 256, &n), HM_ERR_INVALID_ARG);
    EXPECT(hyena_dense_bf16_ex(64, 2048, 1024, P, 1024, P, 1024, nullptr, P, 2048, P, 16, nullptr), HM_ERR_WORKSPACE);

    // explicit-filter baseline, FFT prefill, distillation
    hm_desc fir = ok;
    fir.channels = 64;
    fir.heads = 4;
    EXPECT(hyena_fir_workspace(&fir, &n), HM_OK);
    EXPECT(hyena_fir_workspace(&fir, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_fir_decode_step(&fir, (const float *)P, 100, 0, 200, P, P, P, 64, P, 64, P, 200, P, n, nullptr),
           HM_ERR_INVALID_ARG);  // t >= cache_len
    EXPECT(hyena_fft_prefill_workspace(&fir, 2048, &n), HM_OK);
    if (n != size_t(4) * 2048 * 4 + 2048 * 8 + 4 * 4096 * 8) ++failures;
    EXPECT(hyena_fft_prefill_workspace(&fir, 131072, &n), HM_OK);
    EXPECT(hyena_fft_prefill_workspace(&fir, 131073, &n), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_fft_prefill(&fir, 0, P, P, P, 64, P, 64, P, 0, nullptr), HM_OK);  // nothing to do
    EXPECT(hyena_fft_prefill(&fir, 4097, P, P, P, 64, P, 64, P, 4096, nullptr), HM_ERR_WORKSPACE);
    hm_desc dd = ok;
    dd.batch = 0;
    dd.channels = 4;
    dd.heads = 4;
    dd.modes = 8;
    EXPECT(hyena_distill_workspace(&dd, 1000, &n), HM_OK);
    EXPECT(hyena_distill_workspace(&dd, 0, &n), HM_ERR_INVALID_ARG);
    EXPECT(hyena_distill_adam_step(0, 8, (float *)P, (float *)P, (float *)P, (const float *)P, (const float *)P,
                                   (const float *)P, (float *)P, (float *)P, 1, 1e-2f, 0.9f, 0.999f, 1e-8f, 0.99f,
                                   nullptr),
           HM_ERR_INVALID_ARG);
    EXPECT(hyena_distill_adam_step(4, 8, (float *)P, (float *)P, (float *)P, (const float *)P, (const float *)P,
                                   (const float *)P, (float *)P, (float *)P, 1, 1e-2f, 0.9f, 0.999f, 1e-8f, 1.5f,
                                   nullptr),
           HM_ERR_INVALID_ARG);

    // fused generation step and its weight packing
    hm_desc ls = ok;
    ls.act_dtype = HM_BF16;
    ls.batch = 64;
    ls.channels = 2048;
    ls.heads = 16;
    ls.modes = 16;
    EXPECT(hyena_layer_step_bf16(&ls, P, 2048, P, -1.0f, (float *)P, P, 2048, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_layer_step_bf16(&ls, nullptr, 2048, P, 1e-6f, (float *)P, P, 2048, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_layer_step_bf16(&ls, P, 100, P, 1e-6f, (float *)P, P, 2048, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_layer_step_bf16(&ls, P, 2052, P, 1e-6f, (float *)P, P, 2048, nullptr), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_layer_step_bf16(&ls, P, 2048, P, 1e-6f, (float *)(arena + 8), P, 2048, nullptr), HM_ERR_UNSUPPORTED);
    hm_desc ls32 = ls;
    ls32.modes = 32;
    EXPECT(hyena_layer_step_bf16(&ls32, P, 2048, P, 1e-6f, (float *)P, P, 2048, nullptr), HM_ERR_UNSUPPORTED);
    hm_desc ls0 = ls;
    ls0.batch = 0;
    EXPECT(hyena_layer_step_bf16(&ls0, P, 2048, P, 1e-6f, (float *)P, P, 2048, nullptr), HM_OK);  // empty: no launch
    EXPECT(hyena_pack_in_proj_bf16(0, 64, P, 64, P, nullptr), HM_OK);  // empty: no launch
    EXPECT(hyena_pack_in_proj_bf16(24, 64, P, 64, P, nullptr), HM_ERR_UNSUPPORTED);
    EXPECT(hyena_pack_in_proj_bf16(16, 64, P, 32, P, nullptr), HM_ERR_INVALID_ARG);
    EXPECT(hyena_pack_in_proj_bf16(16, 64, nullptr, 64, P, nullptr), HM_ERR_INVALID_ARG);

    std::printf(failures ? "abi: %d failures\n" : "abi ok\n", failures);
    return failures ? 1 : 0;
}
