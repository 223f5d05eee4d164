"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. tests/sanitize/pack_fuzz.cpp: the library's host packing code
   (sampler_abi.cpp, with no-op kernel launchers) and the oracle's C source,
   built with g++/gcc -fsanitize=address,undefined, run over thousands of
   random batches (CSR histories and biases, duplicate ids, every invalid
   value the ABI rejects, exact-size and undersized buffers) and random
   oracle rows.  Any sanitizer report aborts the driver.
2. The oracle pins and the host-ABI tests against the sanitized oracle build,
   in a subprocess that preloads the ASan runtime.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    if not out or not os.path.exists(out):
        pytest.skip("libasan.so not found")
    return out


def test_pack_and_oracle_fuzz_under_sanitizers(tmp_path):
    _need("g++")
    _need("gcc")
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers not available")
    obj = tmp_path / "cd_oracle.o"
    subprocess.check_call(["gcc", "-std=gnu11", *SAN, "-ffp-contract=off", "-fPIC", "-c",
                           os.path.join(ROOT, "oracle", "cd_oracle.c"), "-o", str(obj)])
    exe = tmp_path / "pack_fuzz"
    subprocess.check_call([
        "g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
        "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(ROOT, "constrained_decoding_amd", "csrc"),
        os.path.join(ROOT, "tests", "sanitize", "pack_fuzz.cpp"),
        os.path.join(ROOT, "constrained_decoding_amd", "csrc", "sampler_abi.cpp"), str(obj),
        "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-lm", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe), "3000"], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "batches packed" in r.stdout


def test_oracle_pins_under_sanitized_oracle():
    _need("gcc")
    sys.path.insert(0, ROOT)
    import oracle.build as ob
    ob.build(force=True, sanitize=True)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), CDS_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py"),
         os.path.join(ROOT, "tests", "test_oracle_draws.py"), "-m", "not slow"],
        capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
