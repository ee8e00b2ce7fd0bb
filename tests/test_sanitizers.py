"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code, on
the CPU: the fp64 oracle (oracle/tg_oracle.c) driven through every entry
point single- and multi-threaded, and the C ABI's argument checks
(csrc/tg_api.cpp) with launcher stand-ins.  Any sanitizer report aborts the
driver (no recovery), so a clean exit means none was found."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, tmp, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{r.stderr}"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"{exe} exited {r.returncode}:\n{r.stdout}\n{r.stderr}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-D_GNU_SOURCE", *SAN, "-ffp-contract=off", os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "tg_oracle.c"), "-o", exe, "-lm", "-lpthread"], tmp_path, exe)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "learned_token_pruning_mlp_amd", "csrc")
    _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
          os.path.join(HERE, "abi_driver.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
          os.path.join(csrc, "tg_api.cpp"), "-o", exe], tmp_path, exe)
