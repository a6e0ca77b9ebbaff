"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
sekv_api.cpp is rebuilt with both sanitizers on its host side (its device code
as usual), linked with the library's other objects and tests/abi_sanitize.cpp
into one executable that drives every host-side argument check, and run on a
machine without a GPU.  Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

from compressed_kv_attention_sekv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize.cpp")
OUT_DIR = os.path.join(B.BUILD_DIR, "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
# each sanitizer flag applies to the host side of the HIP compile only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def _device_objects():
    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o")
            for s in B.SOURCES if s != "sekv_api.cpp"]
    return objs if all(os.path.exists(o) for o in objs) else None


@pytest.fixture(scope="module")
def sanitized_driver():
    if not (os.path.exists(B.HIPCC) and os.path.exists(CLANG)):
        pytest.skip("hipcc / clang++ not available")
    objs = _device_objects()
    if objs is None:
        pytest.skip("library objects not built")
    os.makedirs(OUT_DIR, exist_ok=True)
    api_o = os.path.join(OUT_DIR, "sekv_api_san.o")
    drv_o = os.path.join(OUT_DIR, "abi_sanitize.o")
    exe = os.path.join(OUT_DIR, "abi_sanitize")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([B.HIPCC, *flags, *HOST_SAN, "-x", "hip", "-c",
                    os.path.join(B.CSRC, "sekv_api.cpp"), "-o", api_o], check=True)
    subprocess.run([CLANG, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    *LINK_SAN, "-c", DRIVER, "-o", drv_o], check=True)
    subprocess.run([CLANG, *LINK_SAN, drv_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe], check=True)
    yield exe
    shutil.rmtree(OUT_DIR, ignore_errors=True)


def test_host_checks_clean_under_asan_and_ubsan(sanitized_driver):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    r = subprocess.run([sanitized_driver], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "all passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in report
    assert "runtime error" not in report
