"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer.

* The oracle (oracle/hqq_oracle.c) with a driver that runs every entry point
  over every format, ragged shapes and edge values (tests/sanitize/oracle_check.c).
* The library's host-side code (hqq_abi.cpp: argument checks, the shrink
  certificate, the planning of batched launches; hqq_stream.cpp: the chunking
  of streamed weights) with its kernel launchers and HIP calls replaced by
  recording stubs (tests/sanitize/abi_host_check.cpp).

Both are built with gcc / g++ (no GPU code) and must exit 0 with no sanitizer
report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
       "-fno-sanitize-recover=undefined"]
ROCM_INC = "/opt/rocm/include"


def _run(exe):
    # the environment is passed on as it is; a library preloaded ahead of the
    # ASan runtime is allowed (verify_asan_link_order=0)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    subprocess.check_call(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                           os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"),
                           os.path.join(ROOT, "oracle", "hqq_oracle.c"), "-o", exe, "-lm"])
    assert "oracle checks passed" in _run(exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INC),
                    reason="g++ or the HIP headers not available")
def test_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_check")
    csrc = os.path.join(ROOT, "weight_quantization_group_amd", "csrc")
    # host-only build of the library's host code: the file-scope device array
    # of the static streamed entry point becomes a host array, and its
    # address lookup a recording stub
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-Wno-unused-result",
                           "-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=x",
                           "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(ROOT, "tests", "sanitize", "abi_host_check.cpp"),
                           os.path.join(csrc, "hqq_abi.cpp"), os.path.join(csrc, "hqq_stream.cpp"),
                           "-o", exe])
    assert "abi host checks passed" in _run(exe)
