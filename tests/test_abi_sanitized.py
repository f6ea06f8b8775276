"""The host code of the C ABI (argument validation, workspace layout, the
attention plan) under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: abi.cpp is compiled again with both sanitizers on its host side
only (the device code of a HIP source cannot take them), linked with the
kernel objects of the normal build, and the host-side tests of
test_abi_host.py run against that library in a process with the ASan
runtime preloaded.  Every call there fails validation before anything is
enqueued, so no GPU is needed; any out-of-bounds access, use of freed
memory or undefined behaviour on those paths aborts the run."""

import glob
import os
import subprocess
import sys

import pytest

from vision_transformer_encoder_amd import build as B

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    runtimes = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not runtimes:
        pytest.skip("no ASan runtime next to hipcc")
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "abi.cpp"]
    if not all(os.path.exists(o) for o in objs):
        B.build(verbose=False)
    abi_o = str(tmp_path / "abi.o")
    lib = str(tmp_path / "libvit_sanitized.so")
    r = subprocess.run([B.HIPCC, *B.FLAGS, "-O1", "-g", *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, "abi.cpp"),
                        "-o", abi_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan", *SAN, "-o", lib,
                        *objs, abi_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the library is instrumented: it calls into both runtimes
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, VIT_LIBRARY=lib, LD_PRELOAD=runtimes[-1], HIP_VISIBLE_DEVICES="",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(os.path.dirname(os.path.abspath(__file__)), "test_abi_host.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "failed" not in r.stdout
