"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

- The C ABI's host-side validation and dispatch (sk_api.cpp), built host-only
  with the sanitizers and driven by tests/abi_validation_driver.cpp, whose
  stub launchers count the calls that reach a launch.
- The oracle (oracle/sketchssm_oracle.c), built with the sanitizers and run
  through its pin tests in a child process with the sanitizer runtime
  preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def test_abi_validation_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_san")
    flags = []
    for f in SAN:                       # host code only: each sanitizer flag after -Xarch_host
        flags += ["-Xarch_host", f]
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950"] + flags + \
          ["-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "ssm_decode_amd", "csrc", "sk_api.cpp"),
           os.path.join(ROOT, "tests", "abi_validation_driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env={**os.environ, **ENV_SAN}, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "all checks passed" in out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-3000:]


def test_oracle_pins_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    import oracle
    lib = oracle.build(force=True, out=str(tmp_path / "liboracle_san.so"), extra=SAN + ["-g"])
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = {**os.environ, **ENV_SAN, "SKSSM_ORACLE_LIB": lib, "LD_PRELOAD": asan, "OMP_NUM_THREADS": "2"}
    tests = ["tests/test_oracle_pins.py", "tests/test_wy_pullback.py", "tests/test_coef_map.py",
             "tests/test_dense_fallback.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] + tests,
                       cwd=ROOT, capture_output=True, text=True, env=env, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
