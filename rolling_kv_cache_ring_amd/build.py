"""Build the HIP library in-tree: rolling_kv_cache_ring_amd/liba8r.so (gfx950).

    python -m rolling_kv_cache_ring_amd.build

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host
pass prints a harmless warning that it does not know that feature.

``-mllvm -amdgpu-mfma-vgpr-form=1`` makes the backend give MFMA results and
accumulators VGPRs.  Without it the decode kernel's PV accumulators (updated
by VALU in the online softmax) lived in VGPRs while each MFMA wrote an AGPR,
so every visit copied them across and back (about 200 extra instructions per
two visits); no kernel spills with it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liba8r.so")
ARCH = "gfx950"

SOURCES = ["a8r_host.cpp", "a8r_kernels.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def compile_device(out_dir: str) -> tuple[dict[str, dict[str, int]], str]:
    """Compiles the kernels' device code once more, to assembly under out_dir,
    with the backend's resource remarks.  Returns, per kernel symbol, its VGPRs,
    AGPRs, scratch bytes per lane, occupancy (waves per SIMD) and LDS bytes per
    block, and the assembly text."""
    import re
    asm = os.path.join(out_dir, "a8r_kernels_device.s")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-S", "--cuda-device-only",
           "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "a8r_kernels.hip"), "-o", asm]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy", "LDS Size [bytes/block]": "lds"}
    usage: dict[str, dict[str, int]] = {}
    cur = None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = usage.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(.+?): (\d+)", line)
        if cur is not None and m and m.group(1) in keys:
            cur[keys[m.group(1)]] = int(m.group(2))
    with open(asm) as f:
        return usage, f.read()


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
