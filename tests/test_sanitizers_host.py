"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host-side code (CPU only).

* The fp64 oracle (oracle/ja_oracle.c), built with gcc, driven by
  tests/sanitize/oracle_check.c over ragged batches, every activation and mask,
  backward, tile lists with exactly-sized buffers and the MXFP8 path; leaks are
  reported too.
* The C-ABI layer (csrc/ja_api.cpp: argument checks, workspace plans, launch
  set-up), built with g++ against the HIP runtime's host API, with the kernel
  launchers replaced by stubs that check every workspace region a launch receives
  lies inside the caller's workspace without overlapping another
  (tests/sanitize/host_abi_check.cpp), over a sweep of sizes and every entry point.
Any sanitizer report aborts the program, which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, env_extra):
    env = dict(os.environ, **env_extra)
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc is required for the sanitizer build")
    exe = str(tmp_path / "oracle_check")
    b = subprocess.run([gcc, "-std=gnu99", *SAN, "-pthread", "-I", os.path.join(ROOT, "oracle"),
                        os.path.join(ROOT, "oracle", "ja_oracle.c"),
                        os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-lm", "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr
    r = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_host_abi_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.fail("g++ and the HIP runtime headers are required for the sanitizer build")
    exe = str(tmp_path / "abi_check")
    csrc = os.path.join(ROOT, "jagged_attention_recsys_amd", "csrc")
    b = subprocess.run([gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                        "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "ja_api.cpp"),
                        os.path.join(ROOT, "tests", "sanitize", "host_abi_check.cpp"),
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
                        "-o", exe], capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr
    # The HIP runtime keeps its own allocations until exit: leak reports off, every
    # other ASan / UBSan finding still aborts.
    r = _run([exe], {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
