"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Every libwhiflash source is compiled for the host only with both sanitizers, and
linked with tests/host_sanitize/abi_driver.cpp, which stands in for the HIP runtime
calls the host code makes and records each kernel launch without running it.  The
driver calls every entry point with good and bad arguments and checks statuses,
workspace sizes, sweep plans and every recorded launch shape.  Any sanitizer report
aborts the driver, and the test fails."""

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "drafter_routing_verification_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp")
ROCM = "/opt/rocm"
HIPCC = os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _sources():
    from drafter_routing_verification_amd.build import SOURCES
    return [os.path.join(CSRC, s) for s in SOURCES]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-3000:] + r.stderr[-3000:]
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17",
              "-fPIC", "-c", *SANITIZE_HOST, "-I", INCLUDE, "-I", CSRC, src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        objs = list(pool.map(compile_one, _sources()))
    # The host objects refer to the device code objects of their sources by name; the
    # driver's registration stand-in never reads them, so empty arrays take their place.
    nm = shutil.which("nm") or os.path.join(ROCM, "llvm", "bin", "llvm-nm")
    undefined = _run([nm, "-u", *objs]).stdout
    blobs = sorted(set(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", undefined)))
    stub = tmp_path / "fatbin_stubs.c"
    stub.write_text("".join(f"char {b}[16] __attribute__((aligned(16)));\n" for b in blobs))
    drv = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", CSRC,
          "-I", os.path.join(ROCM, "include"), *SANITIZE, "-c", DRIVER, "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, *SANITIZE, "-x", "c", str(stub), "-x", "none", drv, *objs, "-o", exe,
          "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "all checks passed" in r.stdout
