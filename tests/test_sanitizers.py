"""The oracle's C code and the library's host code (validation, sizing,
workspace carving of include/kvc.h's entry points) built for the CPU with
AddressSanitizer and UndefinedBehaviorSanitizer and driven by the C programs
in tests/sanitize/: every oracle entry point on small odd and even lengths
and degenerate rows, every prefill entry point on problems that are refused
before any launch.  No GPU: the sanitizers instrument host code only (the
GPU kernels in the linked objects are never launched)."""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(map(str, cmd)), r.stdout[-2000:], r.stderr[-4000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_c_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_drv"
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-o", exe, SAN / "oracle_driver.c", ROOT / "oracle" / "kvc_oracle.c", "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    assert "oracle driver ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="needs the ROCm toolchain")
def test_host_code_under_asan_and_ubsan(tmp_path):
    from audio_kv_cache_amd import build
    objs = sorted((build.BUILD).glob("*.o"))
    if len(objs) < len(build.SOURCES):
        build.build()
        objs = sorted((build.BUILD).glob("*.o"))
    others = [o for o in objs if o.name != "kvc_host.o"]
    host_o = tmp_path / "kvc_host_san.o"
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", ROOT / "include",
          "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-c", ROOT / "audio_kv_cache_amd" / "csrc" / "kvc_host.hip", "-o", host_o])
    drv_o = tmp_path / "host_driver.o"
    _run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I", ROOT / "include", "-c", SAN / "host_driver.c",
          "-o", drv_o])
    exe = tmp_path / "host_drv"
    _run([HIPCC, "--offload-arch=gfx950",
          "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined",
          "-o", exe, drv_o, host_o, *others])
    r = _run([exe], env=ENV)
    assert "host driver ok" in r.stdout
