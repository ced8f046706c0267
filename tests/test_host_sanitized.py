"""The host side of the library (ledger, argument validation, layout) built
for the CPU with AddressSanitizer and UndefinedBehaviorSanitizer, and run
through the same C-ABI checks as tests/test_abi_cpu.py: the ledger against
the oracle's bookkeeping over random operations and 100,000 steps, positions
near 2^63, errors that must change nothing, invalid configurations rejected
before any device work.  The device launchers are replaced by stand-ins
(tests/sanitize/launch_stubs.cpp) that no path reached here calls.  Any
sanitizer report aborts the child process and fails the test."""

import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rolling_kv_cache_ring_amd", "csrc")


def test_host_code_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    assert gxx, "g++ is needed for the sanitizer build"
    lib = str(tmp_path / "liba8r_host_sanitized.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared", "-Wl,--no-undefined",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "a8r_host.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    runtime = [subprocess.run([gxx, f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
               for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, LD_PRELOAD=":".join(runtime),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    driver = ("import sys; sys.path.insert(0, {root!r}); import rolling_kv_cache_ring_amd as a8r; "
              "a8r.LIB_PATH = {lib!r}; import pytest; "
              "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', '-m', 'not gpu', {tests!r}]))").format(
        root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    run = subprocess.run([sys.executable, "-c", driver], capture_output=True, text=True, env=env, cwd=ROOT,
                         timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "passed" in run.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
