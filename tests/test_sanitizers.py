"""AddressSanitizer and UndefinedBehaviorSanitizer builds, CPU only.

* The oracle (plain C, gcc) runs small caches of every supported shape with buffers
  allocated to their exact layout sizes (tests/sanitize/oracle_driver.c).
* The host side of the C ABI (argument checks, buffer sizing, split choice, error
  returns) runs with its kernel launchers stubbed out (tests/sanitize/abi_driver.cpp);
  the sanitizers instrument host code only, the device code is built as usual.

A sanitizer report aborts the driver (-fno-sanitize-recover), so exit status 0 means
clean.  Builds go to a temporary directory.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, env=None, timeout=300):
    p = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout, env=env)
    return p.returncode, p.stdout + p.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_driver")
    rc, log = _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    assert rc == 0, log
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    rc, log = _run([exe], env=env)
    assert rc == 0 and "runtime error" not in log and "AddressSanitizer" not in log, log
    assert log.count(": ok") == 11, log


def test_abi_host_paths_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "quantized_decode_attn_amd", "csrc")
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        san += ["-Xarch_host", flag]                    # host code only
    rc, log = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "kvq_api.hip"), os.path.join(HERE, "abi_driver.cpp"), "-o", exe],
                   timeout=600)
    assert rc == 0, log
    # the HIP runtime keeps its own allocations until exit: leak checking is off here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    rc, log = _run([exe], env=env)
    assert rc == 0 and "runtime error" not in log and "AddressSanitizer" not in log, log
    assert "ok (0 failures)" in log, log
