"""Host sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) on the CPU:

  * the oracle (oracle/oracle.c) built with them and run through the pin suite
    (tests/test_oracle_*.py), the sanitizer runtimes preloaded into Python;
  * the C ABI's host code (padding_free_expert_amd/csrc/api.cpp: validation,
    error reporting, dispatch) built with them beside no-op launchers
    (tests/sanitize/launch_stubs.cpp) and driven through every entry point
    (tests/sanitize/api_driver.cpp), then with random arguments from the edges
    of every parameter's range (tests/sanitize/api_fuzz.cpp).

Only host code is built here, with gcc/g++; no device code is compiled with a
sanitizer.  Skipped when the compilers or the sanitizer runtimes are missing.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime(name):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"{name} not found")
    return p


@pytest.mark.slow
def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    lib = ob.build(out=str(tmp_path / "liboracle_san.so"), extra=SAN)
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               XMOE_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    pins = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f != "test_oracle_mutants.py")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + pins,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def _build_abi(tmp_path, driver):
    _runtime("libasan.so")
    if not shutil.which("g++") or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("g++ or the HIP headers not found")
    exe = str(tmp_path / ("api_san_" + driver))
    src = [os.path.join(ROOT, "padding_free_expert_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", driver + ".cpp")]
    cmd = ["g++", "-std=c++17", "-O1"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"] + src + \
          ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-3000:]
    return exe


def _run(exe):
    return subprocess.run([exe], capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES=""))


@pytest.mark.slow
def test_abi_host_code_under_sanitizers(tmp_path):
    r = _run(_build_abi(tmp_path, "api_driver"))
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, (r.stdout + r.stderr)[-3000:]


@pytest.mark.slow
def test_abi_validation_fuzz_under_sanitizers(tmp_path):
    """Random sizes (0, 1, tile edges, 2^31, 2^62, INT64_MAX, negatives),
    dtypes, flags and NULL / misaligned pointers for every entry point: each
    call returns a documented status with a message and the sanitizers stay
    silent (the size checks form no product that could overflow)."""
    r = _run(_build_abi(tmp_path, "api_fuzz"))
    assert r.returncode == 0 and "fuzz: 0 failures" in r.stdout, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
