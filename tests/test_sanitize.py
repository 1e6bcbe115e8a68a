"""CPU sanitizer builds (no GPU): the C ABI layer of libtwq and the C oracle under
AddressSanitizer and UndefinedBehaviorSanitizer.

* libtwq's argument validation, workspace layouts and launch planning (twq_api.cpp,
  plan.cpp) are built with g++ against host stand-ins for the kernel launchers
  (tests/sanitize/stub_launch.cpp), which touch every byte the kernels would; the
  driver (tests/sanitize/abi_driver.cpp) calls every entry point on buffers of exactly
  the documented sizes and with invalid arguments.
* The oracle (oracle/twq_oracle.c) is built the same way and its pinned tests
  (tests/test_oracle.py) run against that build in a child process.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} is not installed")


def test_abi_layer_under_asan_ubsan(tmp_path):
    _need("g++")
    exe = tmp_path / "abi_driver"
    csrc = os.path.join(ROOT, "w4a4_rank_gemm_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
           os.path.join(csrc, "twq_api.cpp"), os.path.join(csrc, "plan.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "stub_launch.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stderr[-4000:]
    assert "all calls returned the expected status" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    _need("gcc")
    import oracle
    lib = tmp_path / "libtwq_oracle_san.so"
    flags = [f for f in oracle.CFLAGS if not f.startswith("-O")] + ["-O1"] + SAN
    subprocess.run(["gcc", *flags, os.path.join(ROOT, "oracle", "twq_oracle.c"), "-o", str(lib), "-lm"],
                   check=True, capture_output=True, text=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("libasan is not installed")
    env = {**os.environ, "TWQ_ORACLE_LIB": str(lib), "LD_PRELOAD": asan,
           "ASAN_OPTIONS": "detect_leaks=0", "OMP_NUM_THREADS": "4"}
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       capture_output=True, text=True, env=env, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
