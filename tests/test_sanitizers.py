"""Host sanitizers over the C code, on the CPU: the float64 oracle (test
infrastructure) and the C ABI layer (argument checks, size, workspace and
layout arithmetic, with the kernel dispatchers replaced by host stand-ins)
are built with AddressSanitizer and UndefinedBehaviorSanitizer, every
finding fatal, and run over small and extreme sizes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _have(tool):
    return shutil.which(tool) is not None


def _build(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    if r.returncode != 0 and "sanitize" in r.stderr and "cannot find" in r.stderr:
        pytest.skip("the host compiler has no sanitizer runtime")
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe, expect):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0 and expect in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])


@pytest.mark.skipif(not _have("gcc"), reason="no host C compiler")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-std=c11", *FLAGS, os.path.join(SAN, "oracle_driver.c"),
            os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], str(tmp_path))
    _run(exe, "oracle ok")


@pytest.mark.skipif(not _have("g++") or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="no host C++ compiler or HIP headers")
def test_abi_layer_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "scan_selective_fwd_amd", "csrc")
    _build(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
            f"-I{ROOT}/include", f"-I{csrc}", os.path.join(SAN, "abi_driver.cpp"),
            os.path.join(SAN, "dispatch_stubs.cpp"), os.path.join(csrc, "api.cpp"),
            f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", exe], str(tmp_path))
    _run(exe, "abi ok")
