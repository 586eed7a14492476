"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every .hip source is compiled with the sanitizers on its host side only
(device code is built as usual, without them), linked with the driver
`host_sanitize/abi_driver.cpp`, and run. The driver calls every entry point
with arguments that fail validation, and plans workspaces over the whole
supported shape set up to the largest sizes the ABI accepts, so no HIP call
is reached: the test needs no GPU and is skipped on a machine that has one
(the sanitizers' runtime and a live GPU runtime are not meant to meet here).
A sanitizer report (out-of-bounds access, signed overflow, invalid shift,
misaligned access ...) ends the run with a non-zero status.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_long_context_page_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "abi_driver.cpp")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
ROCM = "/opt/rocm"
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")

# sanitizers on the host side of every hipcc line (device code is untouched)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src):
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-fPIC", *HOST_SAN,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return obj


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host-only check; a GPU is present")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                    reason="ROCm compilers not installed")
def test_abi_host_code_is_clean_under_asan_and_ubsan():
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    drv = os.path.join(OUT, "abi_driver.o")
    exe = os.path.join(OUT, "abi_driver")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer"]
    r = subprocess.run([CLANG, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *san,
                        f"-I{INCLUDE}", f"-I{ROCM}/include", "-c", DRIVER, "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([CLANG, *san, drv, *objs, f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib",
                        "-lamdhip64", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "abi driver ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
