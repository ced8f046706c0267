"""Register, scratch and LDS budgets of the device code, from the compiler's
resource remarks (no GPU needed).

A kernel that spills to scratch is slow here in a way that tests of results
never show: scratch reloads are counted with the vector-memory loads, so the
waits the compiler puts before them also wait for every direct global->LDS
load in flight, and the walk's pipelining is gone.  The decode and chunk
kernels hold one block per CU with two waves per SIMD (at most 256 registers
each) and up to 160 KiB of LDS."""

import pytest

from rolling_kv_cache_ring_amd import build

LDS_PER_CU = 160 * 1024


@pytest.fixture(scope="module")
def usage(tmp_path_factory):
    return build.resource_usage(str(tmp_path_factory.mktemp("res")))


def test_every_kernel_reported(usage):
    names = " ".join(usage)
    for k in ["decode_mfma", "chunk_pipe", "combine_kernel", "append_kernel", "rebuild_kernel", "attn_portable"]:
        assert k in names, k
    for name, u in usage.items():
        assert {"vgpr", "scratch", "lds", "occupancy"} <= set(u), (name, u)


def test_no_kernel_spills(usage):
    spills = {name: u["scratch"] for name, u in usage.items() if u["scratch"]}
    assert not spills, spills


def test_walk_kernels_fit_one_block_per_cu(usage):
    for name, u in usage.items():
        if "decode_mfma" in name or "chunk_pipe" in name:
            assert u["lds"] <= LDS_PER_CU, (name, u)
            assert u["vgpr"] + u.get("agpr", 0) <= 256, (name, u)
            assert u["occupancy"] >= 2, (name, u)
