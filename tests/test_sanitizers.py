"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The float64 oracle and the library's host side (descriptor and argument
validation, the prefill plan, the workspace queries) are rebuilt with the
sanitizers and driven by small programs under tests/sanitize/; any report
aborts the program.  Only host code is instrumented: on the hipcc line every
sanitizer flag is passed to the host compilation alone, and the library's
device code is built as usual (the drivers make no GPU call)."""

from __future__ import annotations

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "distilled_modal_ssm_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
from distilled_modal_ssm_amd.build import SOURCES as LIB_SOURCES  # every source the library links
# host-only instrumentation for hipcc
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _clean(r):
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-3000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-fopenmp", os.path.join(ROOT, "oracle", "modal_oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="4"), timeout=120)
    _clean(r)
    assert "oracle ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_library_host_side_under_sanitizers(tmp_path):
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC] + HOST_SAN.split()
    objs = [str(tmp_path / (s + ".o")) for s in LIB_SOURCES]

    def compile_one(i):
        _run([HIPCC] + flags + ["-x", "hip", "-c", os.path.join(CSRC, LIB_SOURCES[i]), "-o", objs[i]])

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, range(len(LIB_SOURCES))))
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC] + flags + ["-c", os.path.join(HERE, "abi_driver.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC] + HOST_SAN.split() + [drv] + objs + ["-o", exe])
    # the HIP runtime's own allocations are not instrumented: leak reports off
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"), timeout=120)
    _clean(r)
    assert "abi ok" in r.stdout
