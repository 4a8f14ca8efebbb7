"""Host-code sanitizer runs (CPU, no GPU needed).

* The oracle (oracle/ssm_oracle.c) built with AddressSanitizer +
  UndefinedBehaviorSanitizer, and separately with ThreadSanitizer (its rows
  go to worker threads), runs tests/sanitize/oracle_driver.c: every oracle
  routine on small inputs with several threads, and its invalid-argument
  paths.
* The C ABI's argument checking (api.cpp) built with AddressSanitizer +
  UndefinedBehaviorSanitizer on the host side, linked with the library's
  other objects, runs tests/sanitize/abi_driver.c: every entry point with a
  null handle or invalid arguments (all of which return before any HIP
  call), with leak detection on.
The sanitizers abort the driver on the first finding; a clean run exits 0.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE_C = os.path.join(ROOT, "oracle", "ssm_oracle.c")
CSRC = os.path.join(ROOT, "mamba_selective_scan_ssm_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ROCM_CLANG = "/opt/rocm/lib/llvm/bin/clang"


def run(cmd, env=None, timeout=300):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("san", ["address,undefined", "thread"])
def test_oracle_under_sanitizer(tmp_path, san):
    exe = str(tmp_path / "oracle_driver")
    flags = ["-fsanitize=" + san, "-fno-omit-frame-pointer", "-g", "-O1"]
    if san != "thread":
        flags.append("-fno-sanitize-recover=all")
    run(["gcc", "-std=c11", "-ffp-contract=off"] + flags +
        ["-o", exe, os.path.join(SAN, "oracle_driver.c"), ORACLE_C, "-lm", "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", TSAN_OPTIONS="halt_on_error=1")
    r = run([exe], env=env)
    assert "all calls as expected" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(ROCM_CLANG)),
                    reason="ROCm compilers not available")
def test_abi_argument_checks_under_asan_ubsan(tmp_path):
    from mamba_selective_scan_ssm_amd import build as pkg_build
    objs = [os.path.join(pkg_build.BUILD, f + ".o") for f in pkg_build.SOURCES if f != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        pkg_build.build_library()
    api_o, drv_o, exe = (str(tmp_path / n) for n in ("api.o", "drv.o", "abi_driver"))
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950"] + host_san +
        ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o])
    run([ROCM_CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-I", INCLUDE, "-c", os.path.join(SAN, "abi_driver.c"),
         "-o", drv_o])
    run([HIPCC, "--offload-arch=gfx950", "-fsanitize=address,undefined", "-fno-gpu-sanitize",
         "-o", exe, drv_o, api_o] + objs)
    r = run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "all calls as expected" in r.stdout
