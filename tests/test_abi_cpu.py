"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

from distilled_modal_ssm_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hyena_modal.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hb.LIB_PATH):
        from distilled_modal_ssm_amd import build
        build.build()
    return hb.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(hm_\w+|hyena_\w+)\s*\(", src))


def test_header_and_binding_agree():
    assert _declared() == set(hb.EXPORTS)
    m = re.search(r"#define HM_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == hb.HM_NOALLOC_SCRATCH_BYTES


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_strings(lib):
    assert hb.hm_abi_version() == hb.HM_ABI_VERSION
    for s in range(5):
        assert lib.hm_status_string(s).decode().startswith("HM_")


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _desc(**kw):
    base = dict(batch=2, channels=64, heads=4, modes=8, act_dtype=hb.HM_F32, poles=FAKE,
                residues=FAKE, skip=FAKE)
    base.update(kw)
    d = hb.make_desc(base["batch"], base["channels"], base["heads"], base["modes"], base["act_dtype"],
                     base["poles"], base["residues"], base["skip"])
    if "abi_version" in kw:
        d.abi_version = kw["abi_version"]
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(abi_version=99), hb.HM_ERR_INVALID_ARG),
    (dict(act_dtype=7), hb.HM_ERR_UNSUPPORTED),
    (dict(channels=60, heads=8), hb.HM_ERR_INVALID_ARG),     # D % H != 0
    (dict(modes=0), hb.HM_ERR_INVALID_ARG),
    (dict(modes=65), hb.HM_ERR_UNSUPPORTED),
    (dict(batch=-1), hb.HM_ERR_INVALID_ARG),
    (dict(heads=0), hb.HM_ERR_INVALID_ARG),
    (dict(poles=0), hb.HM_ERR_INVALID_ARG),
    (dict(skip=0x10002), hb.HM_ERR_UNSUPPORTED),            # misaligned table
])
def test_descriptor_validation(lib, kw, status):
    d = _desc(**kw)
    with pytest.raises(hb.HMError) as e:
        hb.hyena_filter_materialize(d, 16, FAKE, stream=0)
    assert e.value.status == status
    with pytest.raises(hb.HMError) as e:
        hb.hyena_modal_decode_step(d, FAKE, FAKE, FAKE, 64, FAKE, 64, FAKE, stream=0)
    assert e.value.status == status
    with pytest.raises(hb.HMError) as e:
        hb.hyena_modal_prefill_workspace(d, 128)
    assert e.value.status == status


def test_prefill_argument_errors(lib):
    d = _desc()
    ws = hb.hyena_modal_prefill_workspace(d, 4096)
    assert ws > 0
    ok = dict(q=FAKE, k=FAKE, v=FAKE, ld_in=64, y=FAKE, ld_y=64, state_in=None, state_out=FAKE,
              workspace=FAKE, ws_bytes=ws)

    def call(L=4096, chunk=0, algo="auto", **kw):
        a = dict(ok)
        a.update(kw)
        hb.hyena_modal_prefill(d, L, a["q"], a["k"], a["v"], a["ld_in"], a["y"], a["ld_y"],
                               a["state_in"], a["state_out"], a["workspace"], a["ws_bytes"], stream=0,
                               chunk=chunk, algo=algo)

    cases = [
        (dict(L=-1), hb.HM_ERR_INVALID_ARG),
        (dict(q=None), hb.HM_ERR_INVALID_ARG),
        (dict(y=None), hb.HM_ERR_INVALID_ARG),
        (dict(state_out=None), hb.HM_ERR_INVALID_ARG),
        (dict(ld_in=63), hb.HM_ERR_INVALID_ARG),
        (dict(ld_y=10), hb.HM_ERR_INVALID_ARG),
        (dict(k=FAKE + 2), hb.HM_ERR_UNSUPPORTED),            # misaligned f32 pointer
        (dict(workspace=None), hb.HM_ERR_WORKSPACE),
        (dict(ws_bytes=ws - 1), hb.HM_ERR_WORKSPACE),
        (dict(workspace=FAKE + 16), hb.HM_ERR_UNSUPPORTED),    # workspace must be 256-B aligned
        (dict(chunk=100), hb.HM_ERR_UNSUPPORTED),              # chunk not a multiple of 64
        (dict(chunk=-64), hb.HM_ERR_INVALID_ARG),
        (dict(algo=7), hb.HM_ERR_INVALID_ARG),                 # unknown algorithm
        (dict(algo="mfma"), hb.HM_ERR_UNSUPPORTED),            # head dim 16: no matrix-core path
    ]
    for kw, status in cases:
        with pytest.raises(hb.HMError) as e:
            call(**kw)
        assert e.value.status == status, kw


def test_no_work_calls_succeed_without_gpu(lib):
    """B = 0 and empty filters enqueue nothing, so they return OK even here."""
    d = _desc(batch=0)
    hb.hyena_modal_prefill(d, 128, None, None, None, 64, None, 64, None, None, None, 0, stream=0)
    hb.hyena_modal_decode_step(d, None, None, None, 64, None, 64, None, stream=0)
    assert hb.hyena_modal_prefill_workspace(d, 128) == 0
    hb.hyena_filter_materialize(_desc(), 0, None, stream=0)


def test_workspace_sizes_follow_the_chunk_plan(lib):
    d = _desc(batch=4, channels=4096, heads=32, modes=32)
    # a single chunk needs no workspace on the vector scan, only tables on the matrix cores
    assert hb.hyena_modal_prefill_workspace(d, 4096, chunk=4096, algo="scan") == 0
    tab = hb.hyena_modal_prefill_workspace(d, 4096, chunk=4096, algo="mfma")
    assert 0 < tab < 4 << 20
    big = hb.hyena_modal_prefill_workspace(d, 65536, chunk=2048, algo="scan")
    # 32 chunk-state slots of B*D*d complex64 dominate
    assert big >= 32 * 4 * 4096 * 32 * 8
    assert hb.hyena_modal_prefill_workspace(d, 65536, chunk=4096, algo="scan") < big
    # the matrix-core plan takes its chunk states from its own 64-step tables: no
    # Vandermonde matrix that grows with the chunk length
    one = _desc(batch=1, channels=4096, heads=32, modes=32)
    slots = 4 * 1 * 4096 * 32 * 8
    mf = hb.hyena_modal_prefill_workspace(one, 65536, chunk=16384, algo="mfma")
    sc = hb.hyena_modal_prefill_workspace(one, 65536, chunk=16384, algo="scan")
    assert slots <= mf < slots + (3 << 20) < sc
    assert hb.hyena_modal_prefill_workspace(one, 65536, chunk=32768, algo="mfma") < mf


def test_prefill_plan_choices(lib):
    """The host-side plan: matrix cores for d in {8,16,32} with 64-channel heads,
    one chunk when batch x heads x tiles cover the CUs, the scan otherwise."""
    w2 = _desc(batch=16, channels=2048, heads=16, modes=16, act_dtype=hb.HM_BF16)
    p = hb.hyena_modal_prefill_plan(w2, 2048)
    assert p["algo"] == "mfma" and p["n_chunks"] == 1 and p["chunk"] == 2048
    assert p["workspace_bytes"] == hb.hyena_modal_prefill_workspace(w2, 2048)
    # 128-channel workgroups when batch x heads still gives 256 of them, else 64
    assert p["channel_tile"] == 128
    w4 = _desc(batch=4, channels=4096, heads=32, modes=32)
    p = hb.hyena_modal_prefill_plan(w4, 65536)
    assert p["channel_tile"] == 64 and p["n_chunks"] == 1
    p = hb.hyena_modal_prefill_plan(_desc(batch=1, channels=4096, heads=32, modes=32), 65536)
    assert p["channel_tile"] == 64 and p["n_chunks"] == 4
    assert hb.hyena_modal_prefill_plan(w2, 2048, algo="scan")["channel_tile"] == 0
    # float32 keeps three bfloat16 parts of every operand: at d = 32 a 128-channel
    # tile no longer fits the LDS, and its tables take 3/2 of the bfloat16 bytes
    f32_32 = _desc(batch=16, channels=2048, heads=16, modes=32, act_dtype=hb.HM_F32)
    assert hb.hyena_modal_prefill_plan(f32_32, 2048)["channel_tile"] == 64
    assert hb.hyena_modal_prefill_plan(_desc(batch=16, channels=2048, heads=16, modes=16, act_dtype=hb.HM_F32),
                                       2048)["channel_tile"] == 128
    bf_32 = _desc(batch=16, channels=2048, heads=16, modes=32, act_dtype=hb.HM_BF16)
    assert hb.hyena_modal_prefill_plan(bf_32, 2048)["channel_tile"] == 128
    t_bf = hb.hyena_modal_prefill_workspace(bf_32, 2048)
    t_f32 = hb.hyena_modal_prefill_workspace(f32_32, 2048)
    assert t_f32 - 16 * 32 * 8 == (t_bf - 16 * 32 * 8) * 3 // 2  # tables grow by half; lambda^64 does not
    # a single batch row over 4 heads: the prompt is cut into 64-step multiples
    few = _desc(batch=1, channels=256, heads=4, modes=8)
    p = hb.hyena_modal_prefill_plan(few, 4096)
    assert p["algo"] == "mfma" and p["n_chunks"] > 1 and p["chunk"] % 64 == 0
    assert p["chunk"] * (p["n_chunks"] - 1) < 4096 <= p["chunk"] * p["n_chunks"]
    # shapes outside the matrix-core path run the scan; asking for mfma is refused
    for kw in (dict(modes=12), dict(modes=64), dict(channels=96, heads=4)):
        d = _desc(**kw)
        assert hb.hyena_modal_prefill_plan(d, 512)["algo"] == "scan"
        with pytest.raises(hb.HMError) as e:
            hb.hyena_modal_prefill_plan(d, 512, algo="mfma")
        assert e.value.status == hb.HM_ERR_UNSUPPORTED
    assert hb.hyena_modal_prefill_plan(w2, 2048, algo="scan")["algo"] == "scan"
    p = hb.hyena_modal_prefill_plan(w2, 2048, chunk=256)
    assert p["chunk"] == 256 and p["n_chunks"] == 8
    p = hb.hyena_modal_prefill_plan(w2, 0)
    assert p["chunk"] == 0 and p["n_chunks"] == 0
    with pytest.raises(hb.HMError):
        hb.hyena_modal_prefill_plan(w2, -1)
    with pytest.raises(hb.HMError):
        hb.hyena_modal_prefill_plan(w2, 2048, chunk=100)


def test_filter_validation(lib):
    d = _desc()
    for L, h, status in [(-1, FAKE, hb.HM_ERR_INVALID_ARG), (16, None, hb.HM_ERR_INVALID_ARG),
                         (16, FAKE + 2, hb.HM_ERR_UNSUPPORTED),
                         (1 << 40, FAKE, hb.HM_ERR_UNSUPPORTED)]:  # beyond the launch grid
        with pytest.raises(hb.HMError) as e:
            hb.hyena_filter_materialize(d, L, h, stream=0)
        assert e.value.status == status, (L, h)


def test_decode_state_validation(lib):
    d = _desc()
    with pytest.raises(hb.HMError) as e:
        hb.hyena_modal_decode_step(d, FAKE, FAKE, FAKE, 64, FAKE, 64, None, stream=0)
    assert e.value.status == hb.HM_ERR_INVALID_ARG
    with pytest.raises(hb.HMError) as e:
        hb.hyena_modal_decode_step(d, FAKE, FAKE, FAKE, 64, FAKE, 64, FAKE + 4, stream=0)
    assert e.value.status == hb.HM_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    saved = hb._lib
    hb._lib = None
    try:
        with pytest.raises(hb.LibraryMissing):
            hb.load(str(tmp_path / "nope.so"))
    finally:
        hb._lib = saved


def test_dense_and_rms_validation(lib):
    def dense(**kw):
        a = dict(M=64, N=128, K=256, A=FAKE, lda=256, W=FAKE, ldw=256, S=None, C=FAKE, ldc=128)
        a.update(kw)
        hb.hyena_dense_bf16(a["M"], a["N"], a["K"], a["A"], a["lda"], a["W"], a["ldw"], a["S"], a["C"],
                            a["ldc"], stream=0)

    cases = [
        (dict(K=0), hb.HM_ERR_INVALID_ARG),
        (dict(M=-1), hb.HM_ERR_INVALID_ARG),
        (dict(lda=100), hb.HM_ERR_INVALID_ARG),
        (dict(ldc=64), hb.HM_ERR_INVALID_ARG),
        (dict(A=None), hb.HM_ERR_INVALID_ARG),
        (dict(K=96, lda=96, ldw=96), hb.HM_ERR_UNSUPPORTED),   # K not a multiple of 64
        (dict(lda=260), hb.HM_ERR_UNSUPPORTED),                # row stride not a multiple of 8
        (dict(W=FAKE + 8), hb.HM_ERR_UNSUPPORTED),             # W not 16-byte aligned
        (dict(S=FAKE + 2), hb.HM_ERR_UNSUPPORTED),             # misaligned row scale
    ]
    for kw, status in cases:
        with pytest.raises(hb.HMError) as e:
            dense(**kw)
        assert e.value.status == status, kw
    dense(M=0)  # empty: no launch
    with pytest.raises(hb.HMError) as e:
        hb.hyena_dense_rms_bf16(64, 128, 256, FAKE, 256, FAKE, 256, -1.0, FAKE, 128, stream=0)
    assert e.value.status == hb.HM_ERR_INVALID_ARG
    with pytest.raises(hb.HMError) as e:
        hb.hyena_dense_rms_bf16(64, 128, 96, FAKE, 96, FAKE, 96, 1e-6, FAKE, 128, stream=0)
    assert e.value.status == hb.HM_ERR_UNSUPPORTED
    for kw, status in [(dict(D=0), hb.HM_ERR_INVALID_ARG), (dict(ld=10), hb.HM_ERR_INVALID_ARG),
                       (dict(eps=-1.0), hb.HM_ERR_INVALID_ARG), (dict(x=FAKE + 1), hb.HM_ERR_UNSUPPORTED)]:
        a = dict(x=FAKE, M=4, D=64, ld=64, eps=1e-6, out=FAKE)
        a.update(kw)
        with pytest.raises(hb.HMError) as e:
            hb.hyena_row_rms(a["x"], a["M"], a["D"], a["ld"], a["eps"], a["out"], stream=0)
        assert e.value.status == status, kw


def test_split_k_workspace_contract(lib):
    """Workspace sizes of the small-M split-K path and its validation."""
    need = hb.hyena_dense_workspace(64, 2048, 1024)
    tiles, slices = 2048 // 64, 1024 // 256
    assert need == tiles * slices * (4096 + 64) * 4
    assert hb.hyena_dense_workspace(64, 4096, 4096) == (4096 // 64) * 16 * (4096 + 64) * 4
    # K = 2048 takes the streaming kernel at any width; wider than 4096: no split-K
    assert hb.hyena_dense_workspace(64, 2048, 2048) == 0
    assert hb.hyena_dense_workspace(64, 6144, 2048) == 0
    assert hb.hyena_dense_workspace(64, 6144, 1024) == 0
    assert hb.hyena_dense_workspace(37, 96, 1024) == 2 * 4 * (4096 + 64) * 4
    # shapes outside the path need none: M > 64, K not a multiple of 256, a single slice
    assert hb.hyena_dense_workspace(65, 6144, 2048) == 0
    assert hb.hyena_dense_workspace(64, 2048, 320) == 0
    assert hb.hyena_dense_workspace(64, 2048, 256) == 0
    assert hb.hyena_dense_workspace(64, 2048, 1536) == 0  # 6 slices: not a supported slice count
    with pytest.raises(hb.HMError) as e:
        hb.hyena_dense_workspace(-1, 8, 256)
    assert e.value.status == hb.HM_ERR_INVALID_ARG

    def call(ws, nbytes, M=64):
        hb.hyena_dense_bf16(M, 2048, 1024, FAKE, 1024, FAKE, 1024, None, FAKE, 2048, stream=0,
                            workspace=ws, ws_bytes=nbytes)

    for ws, nbytes, status in [(FAKE, need - 1, hb.HM_ERR_WORKSPACE), (FAKE + 16, need, hb.HM_ERR_UNSUPPORTED)]:
        with pytest.raises(hb.HMError) as e:
            call(ws, nbytes)
        assert e.value.status == status
    with pytest.raises(hb.HMError) as e:
        hb.hyena_dense_rms_bf16(64, 2048, 1024, FAKE, 1024, FAKE, 1024, 1e-6, FAKE, 2048, stream=0,
                                workspace=FAKE, ws_bytes=16)
    assert e.value.status == hb.HM_ERR_WORKSPACE


def test_fir_validation(lib):
    d = _desc(batch=2, channels=64, heads=4)
    need = hb.hyena_fir_workspace(d)
    assert need > 0 and need % (2 * 64 * 4) == 0

    def step(**kw):
        a = dict(h=FAKE, h_len=100, window=0, t=50, q=FAKE, k=FAKE, v=FAKE, ld_in=64, y=FAKE, ld_y=64,
                 cache=FAKE, cache_len=200, ws=FAKE, ws_bytes=need, desc=d)
        a.update(kw)
        st = lib.hyena_fir_decode_step(ctypes.byref(a["desc"]), a["h"], a["h_len"], a["window"], a["t"],
                                       a["q"], a["k"], a["v"], a["ld_in"], a["y"], a["ld_y"], a["cache"],
                                       a["cache_len"], a["ws"], a["ws_bytes"], None)
        return st

    cases = [
        (dict(t=200), hb.HM_ERR_INVALID_ARG),                 # t beyond the cache
        (dict(t=-1), hb.HM_ERR_INVALID_ARG),
        (dict(window=-2), hb.HM_ERR_INVALID_ARG),
        (dict(h_len=50), hb.HM_ERR_INVALID_ARG),              # full window needs t + 1 taps
        (dict(h=None), hb.HM_ERR_INVALID_ARG),
        (dict(ld_in=32), hb.HM_ERR_INVALID_ARG),
        (dict(cache=FAKE + 8), hb.HM_ERR_UNSUPPORTED),        # cache rows must be 16-byte aligned
        (dict(ws=None), hb.HM_ERR_WORKSPACE),
        (dict(ws_bytes=need - 4), hb.HM_ERR_WORKSPACE),
        (dict(ws=FAKE + 64), hb.HM_ERR_UNSUPPORTED),
        (dict(desc=_desc(batch=2, channels=60, heads=4)), hb.HM_ERR_UNSUPPORTED),  # D not a multiple of 8
        (dict(desc=_desc(batch=2, channels=48, heads=4)), hb.HM_ERR_UNSUPPORTED),  # head dim 12
    ]
    for kw, status in cases:
        assert step(**kw) == status, kw
    # a truncated window needs only W taps: validation passes up to the launch,
    # which needs a GPU, so only the zero-batch call is made here
    assert step(desc=_desc(batch=0, channels=64, heads=4), h_len=8, window=8) == hb.HM_OK
    assert lib.hyena_fir_cache_fill(ctypes.byref(d), 201, FAKE, FAKE, 64, FAKE, 200, None) == hb.HM_ERR_INVALID_ARG
    assert lib.hyena_fir_cache_fill(ctypes.byref(d), 0, FAKE, FAKE, 64, FAKE, 200, None) == hb.HM_OK


def test_fir_load_policy_validation(lib):
    """hyena_fir_decode_step_ex: the policy is checked on the host; float32
    non-temporal loads need D a multiple of 512."""
    def step(desc, loads):
        need = hb.hyena_fir_workspace(desc)
        D = desc.channels
        return lib.hyena_fir_decode_step_ex(ctypes.byref(desc), FAKE, 100, 0, 50, FAKE, FAKE, FAKE, D, FAKE, D,
                                            FAKE, 200, FAKE, need, loads, None)

    f32, bf16 = hb.HM_F32, hb.HM_BF16
    assert step(_desc(batch=2, channels=64, heads=4), 3) == hb.HM_ERR_INVALID_ARG
    assert step(_desc(batch=2, channels=64, heads=4), -1) == hb.HM_ERR_INVALID_ARG
    assert step(_desc(batch=2, channels=64, heads=4, act_dtype=f32), hb.HM_FIR_LOADS_NONTEMPORAL) == \
        hb.HM_ERR_UNSUPPORTED
    # accepted up to the launch (zero batch: nothing is launched)
    for act, D in ((bf16, 64), (f32, 512), (f32, 64)):
        for loads in (hb.HM_FIR_LOADS_AUTO, hb.HM_FIR_LOADS_PLAIN) + \
                ((hb.HM_FIR_LOADS_NONTEMPORAL,) if act == bf16 or D % 512 == 0 else ()):
            assert step(_desc(batch=0, channels=D, heads=4, act_dtype=act), loads) == hb.HM_OK, (act, D, loads)


def test_fft_prefill_validation(lib):
    d = _desc(batch=2, channels=64, heads=4)
    n = hb.hyena_fft_prefill_workspace(d, 2048)
    # taps [4][2048] fp32, twiddles [2048] complex, spectra [4][4096] complex
    assert n == 4 * 2048 * 4 + 2048 * 8 + 4 * 4096 * 8
    assert hb.hyena_fft_prefill_workspace(d, 0) == 0
    # past N = 8192 the three-pass transform adds its work buffer [B][N][D/2] complex
    al = lambda x: (x + 255) // 256 * 256
    n_long = hb.hyena_fft_prefill_workspace(d, 4097)
    off_z = al(al(4 * 4097 * 4) + 8192 * 8) + 4 * 16384 * 8
    assert n_long == al(off_z) + 2 * 16384 * 32 * 8
    assert hb.hyena_fft_prefill_workspace(d, 131072) > 2 * 262144 * 32 * 8
    with pytest.raises(hb.HMError) as e:
        hb.hyena_fft_prefill_workspace(d, 131073)
    assert e.value.status == hb.HM_ERR_UNSUPPORTED

    def call(L=2048, ws=FAKE, nbytes=n, desc=d, ld=64):
        st = lib.hyena_fft_prefill(ctypes.byref(desc), L, FAKE, FAKE, FAKE, ld, FAKE, ld, ws, nbytes, None)
        return st

    assert call(L=131073) == hb.HM_ERR_UNSUPPORTED
    assert call(L=4097) == hb.HM_ERR_WORKSPACE  # the 2048-step workspace lacks the work buffer
    assert call(L=-1) == hb.HM_ERR_INVALID_ARG
    assert call(ws=None) == hb.HM_ERR_WORKSPACE
    assert call(nbytes=n - 8) == hb.HM_ERR_WORKSPACE
    assert call(ws=FAKE + 16) == hb.HM_ERR_UNSUPPORTED
    assert call(ld=32) == hb.HM_ERR_INVALID_ARG
    assert call(desc=_desc(batch=2, channels=12, heads=4)) == hb.HM_ERR_UNSUPPORTED  # head dim 3 is odd
    assert call(L=0) == hb.HM_OK


def test_distill_validation(lib):
    d = _desc(batch=0, channels=4, heads=4, modes=8)
    n = hb.hyena_distill_workspace(d, 1000)
    # residual [4][1000] f64 | loss partials [4][tiles] | gradient partials [4*8][1][4] f64
    assert n >= 4 * 1000 * 8 + 4 * 8 * 4 * 8
    with pytest.raises(hb.HMError) as e:
        hb.hyena_distill_workspace(d, 0)
    assert e.value.status == hb.HM_ERR_INVALID_ARG
    st = lib.hyena_distill_grad(ctypes.byref(d), 1000, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, n - 8, None)
    assert st == hb.HM_ERR_WORKSPACE
    st = lib.hyena_distill_grad(ctypes.byref(d), 1000, None, FAKE, FAKE, FAKE, FAKE, FAKE, n, None)
    assert st == hb.HM_ERR_INVALID_ARG

    def adam(**kw):
        a = dict(H=4, d=8, step=1, lr=1e-2, b1=0.9, b2=0.999, eps=1e-8, r_max=0.9999)
        a.update(kw)
        return lib.hyena_distill_adam_step(a["H"], a["d"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           a["step"], a["lr"], a["b1"], a["b2"], a["eps"], a["r_max"], None)
    for kw in (dict(step=0), dict(lr=0.0), dict(b1=1.0), dict(b2=-0.1), dict(eps=0.0), dict(r_max=1.0),
               dict(r_max=0.0), dict(d=65), dict(H=0)):
        assert adam(**kw) == hb.HM_ERR_INVALID_ARG, kw


def test_layer_step_and_pack_validation(lib):
    """The fused generation step reports shapes it does not cover as a status
    (the caller then makes the two separate calls); argument errors raise."""
    base = dict(batch=64, channels=2048, heads=16, modes=16, act_dtype=hb.HM_BF16)

    def step(desc_kw=None, **kw):
        dk = dict(base)
        dk.update(desc_kw or {})
        a = dict(x=FAKE, ldx=2048, w=FAKE, eps=1e-6, state=FAKE, y=FAKE, ld_y=2048)
        a.update(kw)
        return hb.hyena_layer_step_bf16(_desc(**dk), a["x"], a["ldx"], a["w"], a["eps"], a["state"], a["y"],
                                        a["ld_y"], stream=0)

    for dk in [dict(channels=1024, heads=8), dict(modes=32), dict(batch=65), dict(act_dtype=hb.HM_F32),
               dict(heads=256)]:  # heads=256: 8 channels per head
        assert step(dk) == hb.HM_ERR_UNSUPPORTED, dk
    for kw in [dict(ldx=2052), dict(ld_y=2049), dict(state=FAKE + 8), dict(y=FAKE + 2), dict(w=FAKE + 8)]:
        assert step(**kw) == hb.HM_ERR_UNSUPPORTED, kw
    for kw in [dict(x=None), dict(w=None), dict(state=None), dict(y=None), dict(eps=-1.0), dict(ldx=100),
               dict(ld_y=100)]:
        with pytest.raises(hb.HMError) as e:
            step(**kw)
        assert e.value.status == hb.HM_ERR_INVALID_ARG, kw
    assert step(dict(batch=0)) == hb.HM_OK  # empty: no launch

    for args, status in [((-1, 64, FAKE, 64, FAKE), hb.HM_ERR_INVALID_ARG),
                         ((16, 64, None, 64, FAKE), hb.HM_ERR_INVALID_ARG),
                         ((16, 64, FAKE, 32, FAKE), hb.HM_ERR_INVALID_ARG),    # ldw < K
                         ((24, 64, FAKE, 64, FAKE), hb.HM_ERR_UNSUPPORTED),    # D not a multiple of 16
                         ((16, 64, FAKE + 8, 64, FAKE), hb.HM_ERR_UNSUPPORTED)]:
        with pytest.raises(hb.HMError) as e:
            hb.hyena_pack_in_proj_bf16(*args, stream=0)
        assert e.value.status == status, args
    hb.hyena_pack_in_proj_bf16(0, 64, FAKE, 64, FAKE, stream=0)  # empty: no launch


def test_noalloc_prefill_validation(lib):
    """The allocation-free prefill validates like the workspace form, and a plan
    whose workspace exceeds the built-in scratch is refused on the host."""
    d = _desc(batch=2, channels=256, heads=2, modes=16)
    ok = dict(q=FAKE, k=FAKE, v=FAKE, ld_in=256, y=FAKE, ld_y=256, state_in=None, state_out=FAKE)

    def call(dd=d, L=700, chunk=64, algo="scan", **kw):
        a = dict(ok)
        a.update(kw)
        hb.hyena_modal_prefill_noalloc(dd, L, a["q"], a["k"], a["v"], a["ld_in"], a["y"], a["ld_y"],
                                       a["state_in"], a["state_out"], stream=0, chunk=chunk, algo=algo)

    for kw, status in [(dict(L=-1), hb.HM_ERR_INVALID_ARG), (dict(q=None), hb.HM_ERR_INVALID_ARG),
                       (dict(state_out=None), hb.HM_ERR_INVALID_ARG), (dict(ld_y=8), hb.HM_ERR_INVALID_ARG),
                       (dict(k=FAKE + 2), hb.HM_ERR_UNSUPPORTED), (dict(chunk=100), hb.HM_ERR_UNSUPPORTED),
                       (dict(algo=7), hb.HM_ERR_INVALID_ARG)]:
        with pytest.raises(hb.HMError) as e:
            call(**kw)
        assert e.value.status == status, kw
    # the lane-scan plan of a long prompt in many chunks needs more than the scratch holds
    big = _desc(batch=4, channels=4096, heads=32, modes=32)
    assert hb.hyena_modal_prefill_workspace(big, 65536, chunk=2048, algo="scan") > 16 << 20
    with pytest.raises(hb.HMError) as e:
        call(dd=big, L=65536, chunk=2048, algo="scan", ld_in=4096, ld_y=4096)
    assert e.value.status == hb.HM_ERR_WORKSPACE
    # B = 0 enqueues nothing and needs no device
    hb.hyena_modal_prefill_noalloc(_desc(batch=0), 128, None, None, None, 64, None, 64, None, None, stream=0)


def test_host_modal_fit_matches_oracle(lib):
    """The library's host-side distillation set-up against the oracle: Hankel
    singular values, the order they give, and the matrix-pencil fit (float32
    taps in, float32 tables out) of d-mode and 2d-mode filters."""
    import numpy as np

    import oracle
    from workloads.generate import ModalParams
    rng = np.random.default_rng(51)
    H, d, L = 4, 16, 2048
    r = rng.uniform(0.8, 0.999, (H, d))
    lam = r * np.exp(1j * rng.uniform(0.05, np.pi - 0.05, (H, d)))
    R = (rng.standard_normal((H, d)) + 1j * rng.standard_normal((H, d))) / np.sqrt(2 * d)
    p = ModalParams(np.stack([lam.real, lam.imag], -1).astype(np.float32),
                    np.stack([R.real, R.imag], -1).astype(np.float32), rng.standard_normal(H).astype(np.float32))
    h = oracle.filter_taps(p, L)
    h32 = h.astype(np.float32)
    sv_lib = hb.hyena_hankel_singular_values(h32[0], 80)
    sv_or = oracle.hankel_singular_values(h32[0].astype(np.float64), 80)
    assert np.max(np.abs(sv_lib - sv_or)) <= 1e-9 * sv_or[0]
    # the order counts the singular values above the threshold: at most 2d (the real
    # dimension of d complex modes), the same count as the oracle's spectrum gives
    order = hb.hyena_modal_order(h32, 80, 1e-7)
    for g in range(H):
        sv = oracle.hankel_singular_values(h32[g].astype(np.float64), 80)
        assert order[g] == np.sum(sv > 1e-7 * sv[0]) and 2 * d - 4 <= order[g] <= 2 * d
    # fit: the d-mode filter is reproduced from its float32 taps
    P, Rf, S = hb.hyena_modal_fit_init(h32, d)
    h_fit = oracle.filter_taps(ModalParams(P, Rf, S), L)
    assert np.max(np.abs(h_fit - h)) <= 1e-6 * np.max(np.abs(h))
    Po, Ro, So = oracle.modal_fit_init(h32.astype(np.float64), d)
    h_or = oracle.filter_taps(ModalParams(Po, Ro, So), L)
    assert np.max(np.abs(h_or - h)) <= 1e-6 * np.max(np.abs(h))
    # (clustered poles near the unit circle are ill-determined by float32 taps, so the
    # filters are compared, not the poles; well-separated poles are compared below)
    th = np.linspace(0.2, 2.9, 6)
    lam_s = np.array([0.9, 0.8, 0.95, 0.7, 0.85, 0.6]) * np.exp(1j * th)
    R_s = np.array([1.0, -0.5j, 0.3 + 0.2j, 0.7, -0.4, 0.25j])
    ps = ModalParams(np.stack([lam_s.real, lam_s.imag], -1)[None].astype(np.float32),
                     np.stack([R_s.real, R_s.imag], -1)[None].astype(np.float32), np.array([0.5], np.float32))
    hs = oracle.filter_taps(ps, 300).astype(np.float32)
    a = hb.hyena_modal_fit_init(hs, 6)[0][0]
    b = oracle.modal_fit_init(hs.astype(np.float64), 6)[0][0]
    a, b = a[:, 0] + 1j * a[:, 1], b[:, 0] + 1j * b[:, 1]
    assert max(np.min(np.abs(a - z)) for z in b) <= 1e-5
    assert max(np.min(np.abs(a - z)) for z in lam_s.astype(np.complex64)) <= 1e-5
    # a 2d-mode filter truncated to d modes: the library's fit is as good as the oracle's
    lam2 = np.concatenate([lam, lam[:, ::-1] * 0.98], 1)
    R2 = np.concatenate([R, 0.5 * R], 1)
    p2 = ModalParams(np.stack([lam2.real, lam2.imag], -1), np.stack([R2.real, R2.imag], -1), p.skip)
    h2 = oracle.filter_taps(p2, L).astype(np.float32)
    e_lib = np.sum((oracle.filter_taps(ModalParams(*hb.hyena_modal_fit_init(h2, d)), L) - h2) ** 2, 1)
    e_or = np.sum((oracle.filter_taps(ModalParams(*oracle.modal_fit_init(h2.astype(np.float64), d)), L) - h2) ** 2, 1)
    assert np.all(e_lib <= 1.01 * e_or + 1e-9)


def test_host_modal_fit_validation(lib):
    import numpy as np
    h = np.ones((2, 100), np.float32)
    for args in [(h, 0), (h, 65), (np.ones((2, 20), np.float32), 8)]:
        with pytest.raises(hb.HMError):
            hb.hyena_modal_fit_init(*args)
    with pytest.raises(hb.HMError) as e:
        hb.hyena_hankel_singular_values(h[0], 51)       # needs L >= 2n
    assert e.value.status == hb.HM_ERR_INVALID_ARG
    with pytest.raises(hb.HMError):
        hb.hyena_modal_order(h, 10, 1.5)


def test_deferred_generation_validation(lib):
    """The prepare and the gate of the deferred state reject bad arguments on
    the host, before any HIP call."""
    d = _desc(batch=4, channels=2048, heads=16, modes=16, act_dtype=hb.HM_BF16)
    with pytest.raises(hb.HMError) as e:
        hb.hyena_decode_prepare(d, None, FAKE, FAKE, stream=0)
    assert e.value.status == hb.HM_ERR_INVALID_ARG
    with pytest.raises(hb.HMError) as e:
        hb.hyena_decode_prepare(_desc(batch=4, channels=2048, heads=16, modes=12), FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == hb.HM_ERR_UNSUPPORTED          # d = 12 has no prepare kernel
    with pytest.raises(hb.HMError) as e:
        hb.hyena_decode_prepare(d, FAKE + 8, FAKE, FAKE, stream=0)
    assert e.value.status == hb.HM_ERR_UNSUPPORTED          # state not 16-byte aligned
    hb.hyena_decode_prepare(_desc(batch=0), None, None, None, stream=0)   # nothing to do
    ok = dict(x=FAKE, ldx=2048, w=FAKE, eps=1e-6, rho=FAKE, u=FAKE, y=FAKE, ld_y=2048)

    def gate(dd=d, **kw):
        a = dict(ok)
        a.update(kw)
        return hb.hyena_layer_gate_bf16(dd, a["x"], a["ldx"], a["w"], a["eps"], a["rho"], a["u"], a["y"], a["ld_y"],
                                        stream=0)
    for kw, status in [(dict(x=None), hb.HM_ERR_INVALID_ARG), (dict(ldx=100), hb.HM_ERR_INVALID_ARG),
                       (dict(eps=-1.0), hb.HM_ERR_INVALID_ARG), (dict(rho=None), hb.HM_ERR_INVALID_ARG)]:
        with pytest.raises(hb.HMError) as e:
            gate(**kw)
        assert e.value.status == status, kw
    # shapes outside the launch report HM_ERR_UNSUPPORTED (the stack then takes another path)
    assert gate(dd=_desc(batch=65, channels=2048, heads=16, modes=16, act_dtype=hb.HM_BF16)) == hb.HM_ERR_UNSUPPORTED
    assert gate(dd=_desc(batch=4, channels=1024, heads=16, modes=16, act_dtype=hb.HM_BF16)) == hb.HM_ERR_UNSUPPORTED
    assert gate(dd=_desc(batch=4, channels=2048, heads=16, modes=16)) == hb.HM_ERR_UNSUPPORTED  # float32
    assert gate(x=FAKE + 2) == hb.HM_ERR_UNSUPPORTED
