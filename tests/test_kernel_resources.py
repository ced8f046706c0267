"""Register, scratch and LDS budgets and the memory waits of the device code,
from the compiler's resource remarks and the assembly it produces for the
kernels (no GPU needed).

A kernel that spills to scratch is slow here in a way that tests of results
never show: scratch reloads are counted with the vector-memory loads, so the
waits the compiler puts before them also wait for every direct global->LDS
load in flight, and the walk's pipelining is gone.  The same happens when the
compiler cannot tell which LDS object a read touches: it then waits for all
of those loads (vmcnt 0) right before the read.  The decode and chunk kernels
hold one block per CU with two waves per SIMD (at most 256 registers each)
and up to 160 KiB of LDS."""

import re

import pytest

from rolling_kv_cache_ring_amd import build

LDS_PER_CU = 160 * 1024


@pytest.fixture(scope="module")
def device(tmp_path_factory):
    return build.compile_device(str(tmp_path_factory.mktemp("dev")))


def functions(asm):
    """(symbol, instruction lines) of every kernel in the assembly."""
    for m in re.finditer(r"^(_ZN3a8r\w+):[^\n]*\n(.*?)^\.Lfunc_end\d+:", asm, re.M | re.S):
        lines = [ln.strip() for ln in m.group(2).split("\n")
                 if ln.startswith("\t") and ln.strip() and not ln.strip().startswith((".", ";"))]
        yield m.group(1), lines


def test_every_kernel_reported(device):
    usage, _ = device
    names = " ".join(usage)
    for k in ["decode_mfma", "chunk_pipe", "combine_kernel", "append_kernel", "rebuild_kernel", "attn_portable"]:
        assert k in names, k
    for name, u in usage.items():
        assert {"vgpr", "scratch", "lds", "occupancy"} <= set(u), (name, u)


def test_no_kernel_spills(device):
    usage, _ = device
    spills = {name: u["scratch"] for name, u in usage.items() if u["scratch"]}
    assert not spills, spills


def test_walk_kernels_fit_one_block_per_cu(device):
    usage, _ = device
    for name, u in usage.items():
        if "decode_mfma" in name or "chunk_pipe" in name:
            assert u["lds"] <= LDS_PER_CU, (name, u)
            assert u["vgpr"] + u.get("agpr", 0) <= 256, (name, u)
            assert u["occupancy"] >= 2, (name, u)


def test_no_load_drain_before_an_lds_read(device):
    """No `s_waitcnt vmcnt(0)` directly in front of an LDS read in the walk
    kernels: their reads of DMA-written LDS wait with explicit counts only."""
    _, asm = device
    found = {}
    n_fn = 0
    for name, lines in functions(asm):
        if "decode_mfma" not in name and "chunk_pipe" not in name:
            continue
        n_fn += 1
        bad = [i for i in range(len(lines) - 1)
               if lines[i] == "s_waitcnt vmcnt(0)" and lines[i + 1].startswith("ds_read")]
        if bad:
            found[name] = len(bad)
    assert n_fn >= 20, n_fn
    assert not found, found
