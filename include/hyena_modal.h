/*
 * hyena_modal.h -- C ABI of the MI355X (gfx950) modal-SSM Hyena library.
 *
 * The operator is the order-2 Hyena operator y = q * (h conv (k * v)): a causal
 * long convolution between two element-wise gates (StripedHyena article,
 * sections "Hyena塊" and "Hyena層次結構", which also give its matrix form
 * diag(q) T_h diag(k) v with T_h causal Toeplitz).  Each head's long filter,
 * shared by the head's channels (weight tying, Laughing Hyena Distillery review,
 * ABSTRACT and "提出的方法"), is a distilled low-dimensional linear SSM
 * (same review, ABSTRACT), taken here in diagonal (modal) form:
 *
 *     h[0] = D_h,   h[t] = Re( sum_n R_n * lambda_n^(t-1) )   for t >= 1,
 *
 * with d complex poles lambda_n, residues R_n and a real skip D_h per head.
 * Generation then costs O(d) memory and O(d) time per token (same review,
 * "主要发现"):  u = k v;  y = q (D_h u + Re(sum_n R_n x_n));  x_n <- lambda_n x_n + u.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All data pointers are DEVICE pointers (memory of the current HIP device),
 *    owned by the caller.  The library never allocates or frees memory, keeps no
 *    pointer after returning, and never synchronises: work is enqueued on
 *    `stream` (a hipStream_t; NULL = the default stream) and completes
 *    asynchronously.  The library holds no mutable global state, with one
 *    exception: the per-GPU scratch array of hyena_modal_prefill_noalloc
 *    (HM_NOALLOC_SCRATCH_BYTES on each device, for the life of the process).
 *  - Channel c (0 <= c < D) belongs to head g = c / (D / H).
 *  - Activations (q, k, v, y) are row-major: element (b, t, c) of a
 *    [B][T][width] tensor sits at element offset (b*T + t)*ld + c, where ld >= D
 *    is the row stride in elements.  Their type is hm_desc.act_dtype (float32 or
 *    bfloat16); arithmetic is float32 and y is rounded to the activation type
 *    (round to nearest even).
 *  - Modal state: float32 complex, interleaved (re, im), laid out
 *    [B][H][d][D/H]: the value of mode n of channel c = g*(D/H) + p in batch row b
 *    is at float2 index ((b*H + g)*d + n)*(D/H) + p.
 *  - Tables: poles and residues are [H][d] float32 complex interleaved (re, im);
 *    skip is [H] float32.  Precondition (not checked): |lambda| < 1, all inputs
 *    finite.
 *  - Errors are returned as hm_status, never thrown.  Arguments are validated on
 *    the host before any HIP call; on a validation error nothing is enqueued.
 *    HM_ERR_HIP reports a failed kernel launch (hipGetLastError after launch).
 *  - Alignment: every pointer must be aligned to its element (2 bytes for
 *    bfloat16, 4 for float32, 8 for the complex state); otherwise
 *    HM_ERR_UNSUPPORTED.  Wider vector paths are chosen automatically when
 *    pointers are 16-byte aligned and strides even.
 */
#ifndef HYENA_MODAL_H
#define HYENA_MODAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HM_ABI_VERSION 1
#define HM_MAX_MODES 64 /* largest supported d */

typedef enum hm_status {
    HM_OK = 0,
    HM_ERR_INVALID_ARG = 1, /* null pointer, negative size, D % H != 0, ld < D, bad version */
    HM_ERR_UNSUPPORTED = 2, /* d > HM_MAX_MODES, unknown dtype, misaligned pointer/stride */
    HM_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the queried size */
    HM_ERR_HIP = 4          /* a kernel launch failed */
} hm_status;

typedef enum hm_dtype { HM_F32 = 0, HM_BF16 = 1 } hm_dtype;

/* Operator descriptor.  Sizes: batch B >= 0, channels D >= 1, heads H >= 1 with
 * D % H == 0, modes 1 <= d <= HM_MAX_MODES.  Table pointers are device pointers
 * (see conventions above). */
typedef struct hm_desc {
    int32_t abi_version; /* must be HM_ABI_VERSION */
    int32_t act_dtype;   /* hm_dtype of q, k, v, y */
    int64_t batch;       /* B */
    int64_t channels;    /* D */
    int64_t heads;       /* H */
    int64_t modes;       /* d */
    const float *poles;    /* [H][d][2] */
    const float *residues; /* [H][d][2] */
    const float *skip;     /* [H] */
} hm_desc;

/* ABI version compiled into the library (HM_ABI_VERSION). */
int hm_abi_version(void);

/* Static, human-readable name of a status code. */
const char *hm_status_string(hm_status status);

/*
 * Workspace bytes hyena_modal_prefill needs for this descriptor and prompt
 * length L >= 0.  Writes the size to *bytes (0 is possible).  Pure host
 * computation.
 */
hm_status hyena_modal_prefill_workspace(const hm_desc *desc, int64_t L, size_t *bytes);

/*
 * Prefill: the causal long convolution over a prompt of L tokens plus the
 * end-of-prompt modal state (the Vandermonde contraction
 * x_n = lambda_n^L x0_n + sum_t lambda_n^(L-1-t) u_t).
 *   q, k, v   [B][L][ld_in] activations (may alias one fused [B][L][3D] buffer
 *             with k = q + D, v = q + 2D and ld_in = 3D).
 *   y         [B][L][ld_y] output activations.
 *   state_in  initial state x0 in the state layout, or NULL for zero (a fresh
 *             prompt).  A non-NULL state_in continues a previous prompt.
 *   state_out end-of-prompt state (may equal state_in).
 *   workspace device scratch of at least hyena_modal_prefill_workspace() bytes;
 *             its contents on entry do not matter.
 * Neither path materialises T_h (StripedHyena article, "Hyena層次結構").  On the
 * matrix cores the prompt runs in 64-step sub-blocks: a causal Toeplitz product
 * inside each, the modal state carried between them.  A prompt cut into
 * chunks (too few batch rows x channel tiles to fill the GPU) first gets each
 * chunk's end state from a state-only pass of the same sub-blocks, then a
 * carry scan over chunks.  The vector-ALU path (any shape) does a chunk-local
 * Vandermonde contraction, the carry scan, and an in-chunk modal scan.
 */
hm_status hyena_modal_prefill(const hm_desc *desc, int64_t L,
                              const void *q, const void *k, const void *v, int64_t ld_in,
                              void *y, int64_t ld_y,
                              const float *state_in, float *state_out,
                              void *workspace, size_t ws_bytes, void *stream);

/* Prefill options.  Zero-initialised options (or a NULL pointer) mean automatic. */
typedef enum hm_prefill_algo {
    HM_PREFILL_AUTO = 0, /* matrix-core sub-blocks when eligible, else the vector scan */
    HM_PREFILL_SCAN = 1, /* per-lane modal scan on the vector ALUs, any shape */
    HM_PREFILL_MFMA = 2  /* 64-step sub-blocks on the matrix cores: d in {8,16,32},
                            D/H a multiple of 64, 16-byte aligned activation rows;
                            otherwise HM_ERR_UNSUPPORTED */
} hm_prefill_algo;

typedef struct hm_prefill_opts {
    int64_t chunk; /* prompt chunk length: a positive multiple of 64, or 0 = automatic */
    int32_t algo;  /* hm_prefill_algo */
    int32_t reserved;
} hm_prefill_opts;

/*
 * The same prefill with options: the chunk length (how the prompt is split
 * across the GPU) and the in-chunk algorithm.  Neither changes the result
 * beyond float32 rounding.  Workspace size: hyena_modal_prefill_workspace_ex
 * with the same options.
 *
 * In-chunk algorithms.  HM_PREFILL_SCAN runs the recurrence lane by lane.
 * HM_PREFILL_MFMA cuts each chunk into 64-step sub-blocks; inside one, the
 * convolution is a 64x64 causal Toeplitz product with the filter taps, the
 * history enters through the modal state (readout rows Re(R lambda^i)), and the
 * state moves on with a 64-column Vandermonde product -- all three per-head
 * matrices shared by the head's channels (weight tying, Laughing Hyena
 * Distillery review, "提出的方法"), so they run on the matrix cores.  With the
 * prompt cut into chunks, the state each chunk hands on comes from a pass of
 * the same sub-blocks that reads only k and v and keeps only the state.
 */
hm_status hyena_modal_prefill_ex(const hm_desc *desc, int64_t L,
                                 const void *q, const void *k, const void *v, int64_t ld_in,
                                 void *y, int64_t ld_y,
                                 const float *state_in, float *state_out,
                                 void *workspace, size_t ws_bytes,
                                 const hm_prefill_opts *opts, void *stream);

hm_status hyena_modal_prefill_workspace_ex(const hm_desc *desc, int64_t L,
                                           const hm_prefill_opts *opts, size_t *bytes);

/*
 * What a prefill with these options would run, computed on the host only (no
 * GPU call): the in-chunk algorithm (HM_PREFILL_SCAN or HM_PREFILL_MFMA, never
 * AUTO), the chunk length, the number of chunks the prompt is cut into, and the
 * workspace size.  The answer assumes 16-byte aligned activation rows; with
 * unaligned rows an AUTO prefill runs the scan inside the chunks instead (a
 * chunked matrix-core plan still takes its chunk states from the state-only
 * sub-block pass, with element loads; same workspace).  opts may be NULL
 * (defaults).  HM_ERR_UNSUPPORTED when HM_PREFILL_MFMA is asked for a shape it
 * does not cover; other errors as for the workspace query.
 */
typedef struct hm_prefill_info {
    int32_t algo;           /* hm_prefill_algo that runs */
    int32_t channel_tile;   /* channels per matrix-core workgroup (64 or 128); 0 for the lane scan */
    int64_t chunk;          /* chunk length in steps (L when the prompt is one chunk; 0 when L = 0) */
    int64_t n_chunks;       /* number of chunks (0 when L = 0) */
    size_t workspace_bytes; /* as hyena_modal_prefill_workspace_ex */
} hm_prefill_info;

hm_status hyena_modal_prefill_plan(const hm_desc *desc, int64_t L, const hm_prefill_opts *opts,
                                   hm_prefill_info *info);

/*
 * The prefill of hyena_modal_prefill_ex without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that forbid hipMalloc).  The workspace comes from a scratch
 * array inside the library, HM_NOALLOC_SCRATCH_BYTES on each GPU, held from
 * library load until the process ends; its address on a device is looked up
 * on the first call made with that device current.  The call allocates and
 * frees nothing.
 *   Arguments as hyena_modal_prefill_ex (opts may be NULL: automatic).
 *   A plan whose workspace (hyena_modal_prefill_workspace_ex) exceeds
 *   HM_NOALLOC_SCRATCH_BYTES -> HM_ERR_WORKSPACE, before any HIP call; other
 *   errors as hyena_modal_prefill_ex.  A failed device lookup -> HM_ERR_HIP.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (two streams, two threads) race and give wrong results; calls on
 * one stream are ordered and safe.  The scratch needs no clearing: every byte
 * a call reads was written earlier in the same call.
 */
#define HM_NOALLOC_SCRATCH_BYTES (16 << 20) /* 16 MiB per GPU */

hm_status hyena_modal_prefill_noalloc(const hm_desc *desc, int64_t L,
                                      const void *q, const void *k, const void *v, int64_t ld_in,
                                      void *y, int64_t ld_y,
                                      const float *state_in, float *state_out,
                                      const hm_prefill_opts *opts, void *stream);

/*
 * One generation step for every batch row: reads the state before updating it,
 *   y = q (D_h u + Re(sum_n R_n x_n)),  x_n <- lambda_n x_n + u,  u = k v,
 * which is the convolution with h continued past the prompt (Laughing Hyena
 * Distillery review, "主要发现": O(d) memory and time per token).
 *   q, k, v  [B][ld_in] one token per batch row;  y [B][ld_y];
 *   state    [B][H][d][D/H] complex, updated in place.
 */
hm_status hyena_modal_decode_step(const hm_desc *desc,
                                  const void *q, const void *k, const void *v, int64_t ld_in,
                                  void *y, int64_t ld_y, float *state, void *stream);

/*
 * The first L taps of every head's filter, h_out [H][L] float32:
 *   h[g][0] = D_g,  h[g][t] = Re(sum_n R_gn lambda_gn^(t-1)).
 * Powers are formed in float64 and each tap is rounded once to float32.
 * HM_ERR_UNSUPPORTED when H * L / 128 exceeds 2^31 - 1 (launch grid limit).
 * (The distillation objective compares filters, Laughing Hyena Distillery
 * review, "提出的方法"; this exports them.)
 */
hm_status hyena_filter_materialize(const hm_desc *desc, int64_t L, float *h_out, void *stream);

/* ------------------------------------------------------------------------
 * Projections of a projected Hyena stack (a model built from the operator:
 * per-token input normalisation, in_proj D -> 3D, the operator, out_proj D -> D;
 * the 1.3B generation comparisons of the Laughing Hyena Distillery review,
 * "主要发现", are measured on such a model).
 * ------------------------------------------------------------------------ */

/*
 * inv_rms[m] = 1 / sqrt(mean_k x[m][k]^2 + eps) for every row m < M of a bf16
 * matrix x [M][ld] (D columns used), computed in float32.  Writes M floats.
 * Errors: M < 0, D < 1, ld < D or eps < 0 -> HM_ERR_INVALID_ARG.
 */
hm_status hyena_row_rms(const void *x, int64_t M, int64_t D, int64_t ld, float eps, float *inv_rms,
                        void *stream);

/*
 * C[m][n] = bf16( row_scale[m] * sum_k A[m][k] * W[n][k] ),  m < M, n < N, k < K.
 *   A [M][lda] bf16 (activations), W [N][ldw] bf16 (weights, output-major, as a
 *   torch Linear stores them), C [M][ldc] bf16, row_scale [M] float32 or NULL
 *   (= 1).  Products accumulate in float32 on the matrix cores; C is rounded
 *   once (nearest even).  C must not overlap A or W.
 * Requirements: K a positive multiple of 64; lda, ldw multiples of 8; A and W
 * 16-byte aligned (else HM_ERR_UNSUPPORTED).  M <= 64 takes a weight-streaming
 * path (the generation step), larger M an LDS-tiled path (M and N multiples of
 * 256 with K = 2048, ldc a multiple of 8 and C 16-byte aligned: K staged by
 * direct global-to-LDS loads and C written as whole row segments, the prompt
 * projections of the 1.3B-width stack).
 */
hm_status hyena_dense_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                           const void *W, int64_t ldw, const float *row_scale, void *C,
                           int64_t ldc, void *stream);

/*
 * The in_proj of a projected layer with its input normalisation fused:
 *   C[m][n] = bf16( sum_k A[m][k] W[n][k] / sqrt(mean_k A[m][k]^2 + eps) ),
 * the mean over the K columns of row m, in float32.  Same layouts and
 * requirements as hyena_dense_bf16; eps < 0 -> HM_ERR_INVALID_ARG.
 */
hm_status hyena_dense_rms_bf16(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                               const void *W, int64_t ldw, float eps, void *C, int64_t ldc,
                               void *stream);

/*
 * The same two products with a caller-owned workspace that enables the
 * split-K path for small M (M <= 64, N <= 4096, K in {512, 1024, 4096}; K =
 * 2048 and wider outputs take weight-streaming kernels that are faster
 * without it).  There, a workgroup owns 64 output columns and one 256-wide
 * K slice and writes a float32 partial to the workspace; a second pass sums
 * each column tile's partials and writes C.  Results equal the workspace-less
 * calls up to float32 summation order.
 *
 * hyena_dense_workspace: bytes needed for (M, N, K); 0 when the shape does not
 * take the split-K path (then workspace is ignored and may be NULL).
 * Workspace contract: 256-byte aligned, contents irrelevant (scratch), reusable
 * by any later call on the same stream if large enough; calls that share a
 * workspace must not run concurrently.  Too small -> HM_ERR_WORKSPACE;
 * misaligned -> HM_ERR_UNSUPPORTED; other errors as above.
 */
hm_status hyena_dense_workspace(int64_t M, int64_t N, int64_t K, size_t *bytes);

hm_status hyena_dense_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                              const void *W, int64_t ldw, const float *row_scale, void *C,
                              int64_t ldc, void *workspace, size_t ws_bytes, void *stream);

hm_status hyena_dense_rms_bf16_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                                  const void *W, int64_t ldw, float eps, void *C, int64_t ldc,
                                  void *workspace, size_t ws_bytes, void *stream);

/*
 * One generated token through a projected layer's in_proj and modal operator,
 * in one launch (the generation step whose throughput the Laughing Hyena
 * Distillery review compares at 1.3B width, 主要发现; the recurrence is the
 * O(d)-per-token decode of the same section).  Per batch row b < B:
 *   [q|k|v] = bf16( x[b] W_in^T / sqrt(mean_k x[b][k]^2 + eps) )   (as hyena_dense_rms_bf16)
 *   then hyena_modal_decode_step on those q, k, v: y[b] and the state updated.
 * The result equals those two calls bit for bit; q, k, v are never stored.
 *   desc         operator descriptor; act_dtype HM_BF16, batch = B rows
 *   x            bf16 [B][ldx], the layer input (D columns used)
 *   w_packed     bf16 [3D][D], W_in [3D][D] packed by hyena_pack_in_proj_bf16
 *   state        [B][H][d][P] complex float32, read and updated in place
 *   y            bf16 [B][ld_y], the operator output (D columns written)
 * Supported: B <= 64, D = 2048, d in {8, 16}, P a multiple of 16, ldx a
 * multiple of 8, ld_y even, x / w_packed / state 16-byte and y 4-byte aligned
 * (else HM_ERR_UNSUPPORTED: use the two separate calls).  Null pointers,
 * ldx or ld_y < D, eps < 0 -> HM_ERR_INVALID_ARG.  y must not overlap x.
 */
hm_status hyena_layer_step_bf16(const hm_desc *desc, const void *x, int64_t ldx, const void *w_packed,
                                float eps, float *state, void *y, int64_t ld_y, void *stream);

/*
 * Packs in_proj weights for hyena_layer_step_bf16: w_packed row 48 G + 16 j + i
 * = w_in row j D + 16 G + i (j = 0, 1, 2 for q, k, v; G = 16-channel group),
 * so one group's q, k and v rows are adjacent.
 *   w_in     bf16 [3D][ldw] (K columns used), w_packed bf16 [3D][K] (caller-owned)
 * D % 16, K % 8, ldw % 8 != 0 or misaligned (16 bytes) -> HM_ERR_UNSUPPORTED;
 * D < 0, K < 1, ldw < K, null pointers -> HM_ERR_INVALID_ARG.
 */
hm_status hyena_pack_in_proj_bf16(int64_t D, int64_t K, const void *w_in, int64_t ldw, void *w_packed,
                                  void *stream);

/* ------------------------------------------------------------------------
 * A generated token through a projected layer with the state kept one input
 * behind (the stack's generation step: this gate, then out_proj).
 *
 * The decode recurrence (Laughing Hyena Distillery review, 主要发现)
 *     y = q (D u + Re sum_n R_n x_n),   x_n <- lambda_n x_n + u
 * is evaluated with the addition of u deferred by one token: the stored
 * "deferred state" is s = x - u_prev, where u_prev is the layer's previous
 * input u (u is real, so it enters the real part of every mode).  Then
 *     prepare:  x = s + u_prev;  rho = Re sum_n R_n x_n;  s <- lambda x
 * needs nothing from the coming token, and the gate of that token is
 *     y = q (D u + rho),  u_prev <- u.
 * The two agree with hyena_modal_decode_step up to float32 rounding.  A
 * state from a prefill (or any state x) starts as s = x, u_prev = 0.  Between
 * tokens the state in the usual sense is s + u_prev (u_prev added to the real
 * parts) for a layer whose prepare has not yet run for the coming token.
 * Layouts: s as the modal state [B][H][d][D/H] complex, 16-byte aligned;
 * u_prev and rho float32 [B][D] (row stride D), 8-byte aligned; D/H even.
 * ------------------------------------------------------------------------ */

/*
 * prepare for every batch row and channel of desc (d in {8, 16, 32}, else
 * HM_ERR_UNSUPPORTED): reads s and u_prev, writes rho and the new s in place.
 */
hm_status hyena_decode_prepare(const hm_desc *desc, float *state, const float *u_prev, float *rho, void *stream);

/*
 * The gate of one generated token for every batch row, on packed in_proj
 * weights (hyena_pack_in_proj_bf16):
 *   [q|k|v] = bf16( x W_in^T / sqrt(mean_k x[b][k]^2 + eps) )   (as hyena_dense_rms_bf16)
 *   u = k v;  y = bf16( q (D_h u + rho) );  u_prev <- u
 * with rho from the prepare of this token.  In the same launch, four extra
 * waves per workgroup run hyena_decode_prepare of `next` (another operator:
 * the next layer, whose prepare needs nothing from this one) unless next is
 * NULL, so its state stream shares the launch with this weight stream.
 *   x       bf16 [B][ldx], the layer input (D columns)
 *   w_packed bf16 [3D][D] packed in_proj;  rho float32 [B][D] in;
 *   u_prev  float32 [B][D] out;  y bf16 [B][ld_y]
 *   next_state, next_u_prev, next_rho: as in hyena_decode_prepare for `next`
 * Supported: act_dtype HM_BF16, B <= 64, D = 2048, D/H a multiple of 16,
 * ldx a multiple of 8, ld_y even, x / w_packed 16-byte and y 4-byte aligned
 * (else HM_ERR_UNSUPPORTED).  Null pointers, ldx or ld_y < D, eps < 0 ->
 * HM_ERR_INVALID_ARG.  y must not overlap x.
 */
hm_status hyena_layer_gate_bf16(const hm_desc *desc, const void *x, int64_t ldx, const void *w_packed, float eps,
                                const float *rho, float *u_prev, void *y, int64_t ld_y, const hm_desc *next,
                                float *next_state, const float *next_u_prev, float *next_rho, void *stream);

/*
 * Non-distilled baseline: the Hyena operator's decode step through its
 * explicit long filter (StripedHyena article, Hyena層次結構) instead of the
 * modal recurrence -- the O(t)-per-token cost that distillation removes
 * (Laughing Hyena Distillery review, 研究动机与目标).  Per batch row b and
 * channel c in head g, at position t:
 *     u_t = k v  (appended to the cache, rounded to the activation dtype)
 *     y_t = q * sum_{j=0}^{min(t, W-1)} h[g][j] u_{t-j}
 * with W = window (0: every past step; > 0: the filter truncated to W taps).
 *
 *   u_cache  [B][cache_len][D] activation dtype, rows 0 .. t-1 filled by
 *            earlier steps or by hyena_fir_cache_fill; row t is written here.
 *   h        [H][h_len] float32 taps (e.g. from hyena_filter_materialize),
 *            h_len >= min(t + 1, W) (else HM_ERR_INVALID_ARG).
 *   q, k, v  [B][ld_in], y [B][ld_y], one token per batch row.
 *   workspace  float32 partial sums, hyena_fir_workspace bytes (256-byte
 *            aligned; scratch).
 * Requirements: D and D/H multiples of 8, u_cache 16-byte aligned (else
 * HM_ERR_UNSUPPORTED); 0 <= t < cache_len.  The modal state is not used.
 */
hm_status hyena_fir_workspace(const hm_desc *desc, size_t *bytes);

hm_status hyena_fir_decode_step(const hm_desc *desc, const float *h, int64_t h_len, int64_t window,
                                int64_t t, const void *q, const void *k, const void *v, int64_t ld_in,
                                void *y, int64_t ld_y, void *u_cache, int64_t cache_len,
                                void *workspace, size_t ws_bytes, void *stream);

/*
 * The same step with the cache's load policy chosen by the caller (for tests
 * of both kernel forms at any size, and for callers who know whether the
 * window stays cached between steps):
 *   loads = HM_FIR_LOADS_AUTO (0): non-temporal loads when the window is larger
 *           than 256 MB (the Infinity Cache), plain loads otherwise, as
 *           hyena_fir_decode_step;
 *           HM_FIR_LOADS_PLAIN (1): plain loads;
 *           HM_FIR_LOADS_NONTEMPORAL (2): non-temporal loads.
 * Results do not depend on the policy.  Other values -> HM_ERR_INVALID_ARG;
 * non-temporal float32 loads need D a multiple of 512 (else
 * HM_ERR_UNSUPPORTED).  Everything else as hyena_fir_decode_step.
 */
#define HM_FIR_LOADS_AUTO 0
#define HM_FIR_LOADS_PLAIN 1
#define HM_FIR_LOADS_NONTEMPORAL 2
hm_status hyena_fir_decode_step_ex(const hm_desc *desc, const float *h, int64_t h_len, int64_t window,
                                   int64_t t, const void *q, const void *k, const void *v, int64_t ld_in,
                                   void *y, int64_t ld_y, void *u_cache, int64_t cache_len, void *workspace,
                                   size_t ws_bytes, int32_t loads, void *stream);

/*
 * u_cache[b][t][c] = k[b][t][c] v[b][t][c] (rounded to the activation dtype)
 * for t < L: the prompt's rows of the cache.  k, v [B][L][ld_in].
 */
hm_status hyena_fir_cache_fill(const hm_desc *desc, int64_t L, const void *k, const void *v,
                               int64_t ld_in, void *u_cache, int64_t cache_len, void *stream);

/*
 * Prefill through the FFT, Hyena's own evaluation of its long convolution
 * (StripedHyena article, Hyena層次結構), for comparison with the modal prefill:
 *     y[b][t][c] = q * sum_{s<=t} h_g[t-s] u[s],   u = k v,   t < L,
 * with the filter taps materialised in float32 and the convolution computed
 * as IFFT(FFT(u) FFT(h)) over N = the power of two >= 2L, float32 throughout.
 * Same activation layouts as hyena_modal_prefill; no modal state in or out.
 * Up to N = 8192 (L <= 4096) each transform runs inside one workgroup's LDS;
 * beyond that, in three passes over HBM through a work buffer of B x N x D/2
 * complex float32 in the workspace (4.3 GB per batch row of D = 4096 at
 * L = 65536).
 * Requirements: 1 <= L <= 131072 (else HM_ERR_UNSUPPORTED; L = 0 or B = 0
 * does nothing), D/H even.  Workspace (taps, twiddles, filter spectra, the
 * work buffer): hyena_fft_prefill_workspace bytes, 256-byte aligned, scratch.
 */
hm_status hyena_fft_prefill_workspace(const hm_desc *desc, int64_t L, size_t *bytes);

hm_status hyena_fft_prefill(const hm_desc *desc, int64_t L, const void *q, const void *k, const void *v,
                            int64_t ld_in, void *y, int64_t ld_y, void *workspace, size_t ws_bytes,
                            void *stream);

/*
 * Distillation objective (Laughing Hyena Distillery review, 提出的方法: each
 * filter is fitted by a modal filter under a filter-discrepancy objective).
 * For the modal filter in desc (poles, residues, skip: the current fit) and
 * target taps h_target [H][L] float32:
 *     loss[g]   = sum_{t<L} (hhat_g[t] - h_g[t])^2,
 *     hhat_g[0] = D_g,  hhat_g[t] = Re sum_n R_gn lambda_gn^(t-1),
 * and its gradient: g_poles, g_res [H][d][2] (d/dRe, d/dIm of lambda and R),
 * g_skip [H].  Float64 inside, float32 out.  L >= 1.  Workspace:
 * hyena_distill_workspace bytes, 256-byte aligned, scratch.  batch is unused.
 */
hm_status hyena_distill_workspace(const hm_desc *desc, int64_t L, size_t *bytes);

hm_status hyena_distill_grad(const hm_desc *desc, int64_t L, const float *h_target, float *loss,
                             float *g_poles, float *g_res, float *g_skip, void *workspace,
                             size_t ws_bytes, void *stream);

/*
 * One Adam step on the modal parameters in place (poles, residues [H][d][2],
 * skip [H]) from the gradients above; m, v [H*d*4 + H] are the optimiser's
 * moments (zero before step 1; layout per mode: Re/Im lambda, Re/Im R, then
 * the H skips).  step >= 1 is the 1-based step count.  After the step every
 * pole with |lambda| > r_max is scaled back to radius r_max (0 < r_max < 1),
 * so the fitted recurrence stays stable.  Invalid hyper-parameters ->
 * HM_ERR_INVALID_ARG.
 */
hm_status hyena_distill_adam_step(int64_t H, int64_t d, float *poles, float *residues, float *skip,
                                  const float *g_poles, const float *g_res, const float *g_skip,
                                  float *m, float *v, int64_t step, float lr, float beta1, float beta2,
                                  float eps, float r_max, void *stream);

/* ------------------------------------------------------------------------
 * Set-up of a distillation on the host (Laughing Hyena Distillery review,
 * 提出的方法: the state dimension follows the spectrum of each filter's Hankel
 * operator, and the filter is reduced by modal truncation with a Prony-like
 * parametrisation).  These three run on the CPU: every pointer is a HOST
 * pointer, float64 inside, and no GPU call is made.  Threads: one per head,
 * up to the host's hardware threads.
 * ------------------------------------------------------------------------ */

/*
 * Singular values, in decreasing order, of the n x n Hankel matrix
 * Hk[i][j] = h[1 + i + j] of one filter h [L] (the taps after the skip).
 * Requires L >= 2n (else HM_ERR_INVALID_ARG); n <= 4096 (else
 * HM_ERR_UNSUPPORTED).  sv: n doubles.
 */
hm_status hyena_hankel_singular_values(const float *h, int64_t L, int64_t n, double *sv);

/*
 * Order of each head's filter, h [H][L]: the number of Hankel singular values
 * (n x n, as above) above rel_tol times the largest.  A filter of d complex
 * modes has order at most 2d (one per real dimension of its minimal
 * realisation), so ceil(order / 2) modes suffice up to that tolerance.
 * order: H int64.  0 < rel_tol < 1.
 */
hm_status hyena_modal_order(const float *h, int64_t H, int64_t L, int64_t n, double rel_tol, int64_t *order);

/*
 * Initial modal fit of each head's filter h [H][L] (h[g][0] is the skip):
 * poles from the matrix pencil of the first taps with 2d exponentials (real
 * taps give conjugate pairs; each pair is one mode, its upper half-plane
 * member), each pole scaled back to radius r_max if it lies outside; then the
 * residues that minimise sum_{1 <= t < L} (Re sum_n R_n lambda_n^(t-1) - h[t])^2
 * for those poles; skip = h[g][0].  Modes beyond the filter's own order get
 * zero residues.  A filter of at most d distinct modes is recovered up to
 * rounding.  Outputs (host): poles, residues [H][d][2], skip [H], float32.
 * 0 < r_max < 1; d <= HM_MAX_MODES; L must hold the pencil (about 6d taps;
 * else HM_ERR_INVALID_ARG).
 */
hm_status hyena_modal_fit_init(const float *h, int64_t H, int64_t L, int64_t d, float r_max, float *poles,
                               float *residues, float *skip);

#ifdef __cplusplus
}
#endif

#endif /* HYENA_MODAL_H */
