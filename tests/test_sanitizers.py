"""Host-side AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only):

- the fp64 oracle (plain C), built with gcc's sanitizers, driven through every
  entry point on small shapes and edge cases (tests/sanitize/oracle_driver.c);
- the C-ABI validation of libmamba_scan: the library is built with the
  sanitizers on its host code only (device code is unchanged), and a driver
  calls every entry point with arguments validation must refuse, including
  extreme dims whose products overflow 32 bits, and with valid arguments
  only when no GPU is visible (tests/sanitize/abi_driver.cpp).

Any sanitizer report makes the driver exit non-zero. Leak checking is off:
the HIP runtime keeps allocations for the life of the process.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, **kw)


def _check(res, what):
    out = res.stdout + res.stderr
    assert res.returncode == 0, "%s failed (%d):\n%s" % (what, res.returncode, out[-4000:])
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


@pytest.fixture(scope="module")
def outdir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("sanitize"))


def test_oracle_under_asan_ubsan(outdir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = os.path.join(outdir, "oracle_driver")
    res = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-fopenmp", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
                os.path.join(ROOT, "oracle", "mamba_oracle.c"), os.path.join(ROOT, "oracle", "mamba2_oracle.c"),
                "-lm"])
    _check(res, "oracle driver build")
    _check(_run([exe], env=ENV), "oracle driver")


def test_c_abi_validation_under_asan_ubsan(outdir):
    from selective_state_space_07_amd import build
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        pytest.skip("ROCm clang++ not available")
    lib = os.path.join(outdir, "libmamba_scan_sanitized.so")
    # sanitizers on the host half only: each -fsanitize= behind -Xarch_host
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host += ["-Xarch_host", f]
    flags = [f for f in build.HIPCC_FLAGS if f != "-O3"]
    res = _run([build.hipcc(), *flags, "-O1", "-g", *host, "-I", os.path.join(ROOT, "include"), "-o", lib,
                *(os.path.join(build.CSRC, s) for s in build.SOURCES)])
    _check(res, "sanitized library build")
    exe = os.path.join(outdir, "abi_driver")
    res = _run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I",
                os.path.join(ROOT, "include"), "-o", exe, os.path.join(HERE, "abi_driver.cpp"), lib,
                "-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + outdir,
                "-Wl,-rpath," + os.path.join(rocm, "lib")])
    _check(res, "abi driver build")
    _check(_run([exe], env=ENV, timeout=300), "abi driver")
