"""The C ABI used from C alone: tests/c/closed_form.c allocates with hipMalloc,
drives a cache on its own HIP stream through include/a8r.h, and checks closed
forms of the attention (a one-key window returns that key's value row bit for
bit; a zero query returns the window's mean value row) and the ring state."""

import os
import shutil
import subprocess

import pytest

import rolling_kv_cache_ring_amd as a8r
from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_closed_forms(tmp_path):
    say("c_program_closed_forms")
    gcc = shutil.which("gcc")
    assert gcc, "gcc not found"
    assert os.path.exists(a8r.LIB_PATH), a8r.LIB_PATH
    libdir = os.path.dirname(a8r.LIB_PATH)
    exe = tmp_path / "closed_form"
    r = subprocess.run([gcc, "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                        os.path.join(ROOT, "tests", "c", "closed_form.c"), "-o", str(exe),
                        os.path.abspath(a8r.LIB_PATH), f"-L{ROCM}/lib", "-lamdhip64", "-lm",
                        f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{ROCM}/lib"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip())
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "closed forms hold" in r.stdout
