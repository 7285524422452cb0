"""The C ABI's host code under the address and undefined-behaviour sanitizers.

abi.cpp (argument validation, overlap checks, size arithmetic, dispatch) is
compiled with the sanitizers on its host side only and linked with the
library's other objects into tests/abi_host_check.cpp, which drives every
entry point through its error paths, empty batches and - when no GPU is
visible - valid calls whose launches the HIP runtime refuses (LA_ERR_HIP).
CPU only: nothing here runs a kernel.
"""

import os
import shutil
import subprocess

import pytest

from gated_delta_rule_causal_amd import build as b

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    objs = [os.path.join(b.BUILD, s + ".o") for s in b.SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        b.build(verbose=False)
    out = tmp_path_factory.mktemp("asan")
    abi_o = str(out / "abi_asan.o")
    exe = str(out / "abi_host_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in b.compile_flags() if f != "-O3"] + ["-O1", "-g"]
    subprocess.run([hipcc] + flags + san + ["-x", "hip", "-c", os.path.join(b.CSRC, "abi.cpp"), "-o", abi_o],
                   check=True, capture_output=True, text=True)
    # the driver is plain host C++: ROCm's clang++ (the compiler behind hipcc)
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = shutil.which("clang++") or pytest.skip("clang++ not available")
    rocm_inc = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "include")
    drv_o = str(out / "driver.o")
    subprocess.run([clangxx, "-std=c++17", "-O1", "-g", "-I", b.INCLUDE, "-I", rocm_inc, "-D__HIP_PLATFORM_AMD__",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                    "-c", os.path.join(HERE, "abi_host_check.cpp"), "-o", drv_o],
                   check=True, capture_output=True, text=True)
    link = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", "-fsanitize=address,undefined", "-fno-gpu-sanitize",
                           "-o", exe, drv_o, abi_o] + objs, capture_output=True, text=True)
    if link.returncode != 0:
        pytest.fail("link failed:\n" + link.stderr[-3000:])
    return exe


def test_abi_validation_under_sanitizers(checker):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([checker], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
    assert " 0 failed" in r.stdout
