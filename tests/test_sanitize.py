"""The host code of libsmcsd.so (argument validation, launch plans and workspace layouts of
every entry point, api.cpp) and the CPU oracle (oracle/smcsd_oracle.c), built for the host
with AddressSanitizer and UndefinedBehaviorSanitizer and run without a GPU: the kernels'
launchers are stubs that count calls and fail (tests/sanitize/stubs.cpp), so a valid call
ends at its first launch. tests/sanitize/driver.cpp holds the checks."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
INC = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
       "-I" + os.path.join(ROOT, "smc_particle_resampling_amd", "csrc")]


def _build() -> str:
    os.makedirs(OUT, exist_ok=True)
    cxx, cc = os.path.join(LLVM, "clang++"), os.path.join(LLVM, "clang")
    objs = []
    for src in (os.path.join(ROOT, "smc_particle_resampling_amd", "csrc", "api.cpp"),
                os.path.join(SRC, "stubs.cpp"), os.path.join(SRC, "driver.cpp")):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        subprocess.run([cxx, "-x", "c++", "-std=c++17", *SAN, *INC, "-c", src, "-o", obj],
                       check=True, capture_output=True, text=True)
        objs.append(obj)
    obj = os.path.join(OUT, "smcsd_oracle.o")
    subprocess.run([cc, "-std=c11", *SAN, "-ffp-contract=off", "-c",
                    os.path.join(ROOT, "oracle", "smcsd_oracle.c"), "-o", obj],
                   check=True, capture_output=True, text=True)
    objs.append(obj)
    exe = os.path.join(OUT, "driver")
    subprocess.run([cxx, *SAN, *objs, "-lm", "-o", exe], check=True, capture_output=True, text=True)
    return exe


@pytest.mark.skipif(not os.path.exists(os.path.join(LLVM, "clang++")), reason="no ROCm clang")
def test_host_code_and_oracle_under_asan_ubsan():
    try:
        exe = _build()
    except subprocess.CalledProcessError as e:
        raise AssertionError("sanitizer build failed:\n%s" % e.stderr)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "sanitized host checks passed" in p.stdout
    assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr, p.stderr
