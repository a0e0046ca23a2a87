"""Host code under sanitizers (CPU only).

Three drivers in tests/sanitize/ are built with AddressSanitizer +
UndefinedBehaviorSanitizer, and the threaded ones also with
ThreadSanitizer:
  - oracle_driver.c: every oracle function, including the threaded shard
    step (results must not depend on the thread count);
  - offload_driver.cpp: zs_cpu_step, the ZeRO-Offload host update of the
    product library, with one and several worker threads, and the piecewise
    update behind zs_offload_step with host-side hooks;
  - abi_driver.c: the host-only logic of libzeroshard (partition, scaler,
    device-scaler image, argument rejection), linked against a build of the
    library whose host code is sanitized (the device code is not: GPU
    sanitizers are not used here).
A memory error, undefined behaviour or data race aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "sharded_mixed_precision_zs_amd", "csrc")
ASAN_UBSAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
TSAN = ["-fsanitize=thread"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...: rc={r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.parametrize("san", ["asan_ubsan", "tsan"])
def test_oracle_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / f"oracle_{san}")
    flags = ASAN_UBSAN if san == "asan_ubsan" else TSAN
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", *flags,
          "-I", ORACLE, os.path.join(SAN, "oracle_driver.c"), os.path.join(ORACLE, "zs_oracle.c"),
          "-o", exe, "-pthread", "-lm"])
    assert "oracle driver ok" in _run([exe])


@pytest.mark.parametrize("san", ["asan_ubsan", "tsan"])
def test_offload_update_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / f"offload_{san}")
    flags = ASAN_UBSAN if san == "asan_ubsan" else TSAN
    _run(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math", "-mf16c",
          "-pthread", *flags, "-I", INCLUDE, "-I", CSRC, os.path.join(SAN, "offload_driver.cpp"),
          os.path.join(CSRC, "offload_cpu.cpp"), "-o", exe])
    assert "offload driver ok" in _run([exe])


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs hipcc and ROCm's clang")
def test_library_host_code_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libzs_hostsan.so")
    # the sanitizer flags apply to the host compilation only
    host_san = []
    for f in ASAN_UBSAN:
        host_san += ["-Xarch_host", f]
    _run([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fPIC", "-shared",
          *host_san, "-I", INCLUDE, os.path.join(CSRC, "zeroshard.hip"), "-o", lib])
    exe = str(tmp_path / "abi_asan")
    _run([CLANG, "-std=c11", "-O1", "-g", *ASAN_UBSAN, "-I", INCLUDE,
          os.path.join(SAN, "abi_driver.c"), "-o", exe, "-L", str(tmp_path), "-lzs_hostsan",
          f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib"])
    assert "abi driver ok" in _run([exe])


def test_tools_present():
    assert shutil.which("gcc") and shutil.which("g++")
