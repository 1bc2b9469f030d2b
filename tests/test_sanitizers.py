"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/ are built with both sanitizers and run as child processes:
  oracle_driver.c  every oracle function on small inputs in exactly sized heap buffers, through
                   its edge paths (invalid pages, holes, repeats, empty sets, skipped tokens)
  abi_driver.c     every libdsa.so entry point with host arguments it must reject before any
                   launch, and the workspace-size queries at extreme sizes; the library's host
                   code (dsa_abi.hip) is instrumented (host pass only), the kernels are linked as
                   built
A sanitizer report aborts the driver, so a nonzero exit status fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)} failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"), "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "dsa_oracle.c"), "-lm"], tmp_path)
    assert "oracle driver: ok" in _run([exe], tmp_path)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_code_under_sanitizers(tmp_path):
    from sparse_attention_06_amd import build as lib_build

    objs = [os.path.join(lib_build.OBJ, s.replace(".hip", ".o")) for s in lib_build.SOURCES if s != "dsa_abi.hip"]
    if not all(os.path.exists(o) for o in objs):
        lib_build.build()
    abi = str(tmp_path / "abi_san.o")
    # instrument the host pass only: each sanitizer flag follows -Xarch_host
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={lib_build.ARCH}", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", lib_build.CSRC,
          "-c", os.path.join(lib_build.CSRC, "dsa_abi.hip"), "-o", abi], tmp_path)
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "-fsanitize=address,undefined", "-fno-gpu-sanitize", f"--offload-arch={lib_build.ARCH}",
          "-I", os.path.join(ROOT, "include"), "-x", "c", os.path.join(SAN, "abi_driver.c"), "-x", "none", abi,
          *objs, "-o", exe], tmp_path)
    assert "abi driver: ok" in _run([exe], tmp_path)
