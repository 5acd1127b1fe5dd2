"""The library's host code (argument checks, workspace planning, the causal
recursion driver up to its first launch, the host projection matrix) built
with AddressSanitizer and UndefinedBehaviorSanitizer and run by a C++
driver of the C ABI (tests/sanitize/abi_driver.cpp).  Needs no GPU: every
call returns before a kernel is enqueued (HYPERATTN_FAIL_AT stops whole
calls at their first launcher)."""

import glob
import os
import shutil
import subprocess

import pytest

from approximate_long_context_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(B.BUILD, "san")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
# host-side sanitizer flags for the hipcc compile of the driver source (the
# device code is left alone)
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SAN = ["-fsanitize=address,undefined", "-shared-libasan"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


@pytest.fixture(scope="module")
def driver():
    if not os.path.exists(CLANG) or not glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        pytest.skip("ROCm clang with the sanitizer runtimes is not installed")
    rt = os.path.dirname(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")[0])
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in B.SOURCES:
        if src == "ha_api.cpp":
            continue
        o = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        if not os.path.exists(o):
            os.makedirs(B.BUILD, exist_ok=True)
            B._compile(src)
        objs.append(o)
    api_o = os.path.join(SAN_DIR, "ha_api.o")
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([B.hipcc()] + flags + HOST_SAN + ["-c", os.path.join(B.CSRC, "ha_api.cpp"), "-o", api_o])
    lib = os.path.join(SAN_DIR, "libhyperattn_san.so")
    _run([CLANG, "-shared", "-fPIC"] + LINK_SAN + ["-o", lib, api_o] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    exe = os.path.join(SAN_DIR, "abi_driver")
    _run([CLANG, "-O1", "-g", "-fno-sanitize-recover=undefined"] + LINK_SAN +
         ["-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
          "-o", exe, f"-L{SAN_DIR}", "-lhyperattn_san", f"-Wl,-rpath,{SAN_DIR}", f"-Wl,-rpath,{rt}",
          "-Wl,-rpath,/opt/rocm/lib"])
    return lib, exe


def test_sanitized_library_is_instrumented(driver):
    lib, _ = driver
    nm = shutil.which("nm") or "/opt/rocm/lib/llvm/bin/llvm-nm"
    syms = _run([nm, "-D", "--undefined-only", lib]).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms


def test_host_code_under_asan_and_ubsan(driver):
    _, exe = driver
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    env.pop("HYPERATTN_FAIL_AT", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, f"rc {res.returncode}\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "all expectations held" in res.stdout
