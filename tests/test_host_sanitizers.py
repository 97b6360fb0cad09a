"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source is compiled again with the sanitizers on its host code only
(the device code is unchanged), linked with tests/abi_fuzz.c into one
executable, and run: fixed argument cases with known statuses, then a seeded
fuzz over edge values of every entry point (see abi_fuzz.c).  On a machine
without a GPU the calls that pass validation run the host dispatch up to the
kernel launch, which fails; the driver makes only validation-failure calls
when a GPU is visible.  Takes about a minute (the compile)."""

import os
import shutil
import subprocess

import pytest

from int8_int4_dequant_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
# host-side sanitizer options: on hipcc lines each one right after -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


@pytest.mark.timeout(600)
def test_abi_under_host_sanitizers(tmp_path):
    if not (os.path.exists(build.HIPCC) and os.path.exists(os.path.join(LLVM, "clang"))):
        pytest.skip("hipcc / clang not installed")
    objs = build.compile_objects(str(tmp_path / "obj"), HOST_SAN)
    drv = str(tmp_path / "abi_fuzz.o")
    san = "-fsanitize=address,undefined"
    subprocess.run([os.path.join(LLVM, "clang"), "-O1", "-g", san,
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                    "-c", os.path.join(ROOT, "tests", "abi_fuzz.c"), "-o", drv],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_fuzz")
    subprocess.run([os.path.join(LLVM, "clang++"), san, drv, *objs, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "abi_fuzz:" in out and " 0 failures" in out, out[-4000:]
