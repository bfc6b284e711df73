"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:

* the oracle (oracle/gs_oracle.c), driven by tests/sanitize_oracle.c through
  every entry point on small generated scenes and degenerate inputs;
* the C ABI's host code (gaussian_splatting_tile_amd/csrc/*.hip, host side
  only: the device code is not instrumented and no device is touched),
  driven by tests/sanitize_abi.c through the argument checks and size
  queries of every call in include/gs.h.

Each driver is built into a temporary directory with the sanitizers, must
exit 0 and must print no sanitizer report."""

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gaussian_splatting_tile_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(exe, env):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert "LeakSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.slow
def test_oracle_under_address_and_undefined_sanitizers():
    cc = shutil.which("gcc")
    assert cc, "gcc is needed"
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_san")
        subprocess.run([cc, "-std=c11", "-ffp-contract=off", "-fopenmp", *SAN, "-I", os.path.join(ROOT, "oracle"),
                        os.path.join(ROOT, "oracle", "gs_oracle.c"), os.path.join(ROOT, "tests", "sanitize_oracle.c"),
                        "-lm", "-o", exe], check=True, capture_output=True)
        out = _run(exe, ENV)
    assert out.count("scene n=") == 5


@pytest.mark.slow
def test_abi_host_code_under_address_and_undefined_sanitizers():
    hip = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    clangxx = "/opt/rocm/llvm/bin/clang++"
    clang = "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hip) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    from gaussian_splatting_tile_amd import build as gbuild
    host_san = []
    for f in SAN:
        host_san += ["-Xarch_host", f]
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in gbuild.SOURCES:
            obj = os.path.join(d, os.path.splitext(src)[0] + ".o")
            subprocess.run([hip, "-std=c++17", "-O3", "-fPIC", f"--offload-arch={gbuild.ARCH}", "-I",
                            os.path.join(ROOT, "include"), "-I", CSRC, "-Xclang", "-target-feature", "-Xclang",
                            "-packed-fp32-ops", *host_san, "-c", os.path.join(CSRC, src), "-o", obj],
                           check=True, capture_output=True)
            objs.append(obj)
        drv = os.path.join(d, "sanitize_abi.o")
        subprocess.run([clang, "-std=c11", *SAN, "-I", os.path.join(ROOT, "include"), "-c",
                        os.path.join(ROOT, "tests", "sanitize_abi.c"), "-o", drv], check=True, capture_output=True)
        exe = os.path.join(d, "abi_san")
        subprocess.run([clangxx, *SAN, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
                        "-o", exe], check=True, capture_output=True)
        # the HIP runtime's own allocations are not this library's: leaks are
        # not checked for this driver
        out = _run(exe, dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert "0 failures" in out, out[-2000:]
