"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, validates arguments before touching a device, and its host
ledger matches the oracle's bookkeeping bit for bit."""

import ctypes
import os
import random
import re

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
from oracle.ledger import StreamLedger

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "a8r.h")



@pytest.fixture(scope="module", autouse=True)
def built_library():
    """These tests need the library, never skip for want of it: build it when
    it is missing (a failed build fails the tests)."""
    if not os.path.exists(a8r.LIB_PATH):
        from rolling_kv_cache_ring_amd import build
        build.build()
    assert os.path.exists(a8r.LIB_PATH), a8r.LIB_PATH


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(a8r_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ["a8r_cache_create", "a8r_append_kv", "a8r_decode_attn", "a8r_chunk_attn", "a8r_reset"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(a8r.LIB_PATH)
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(a8r.EXPORTED) == names


def test_config_struct_layout_matches_header():
    # 10 int32 + double + 2 float + 2 int32 = 40 + 8 + 8 + 8 = 64 bytes, double at offset 40
    assert ctypes.sizeof(a8r.Config) == 64
    assert a8r.Config.rope_theta.offset == 40
    assert a8r.Config.prefix_capacity.offset == 56


def test_version():
    assert "gfx950" in a8r.version()


@pytest.mark.parametrize("bad", [
    dict(n_layers=0), dict(n_streams=0), dict(n_q_heads=3, n_kv_heads=2), dict(head_dim=96),
    dict(window=0), dict(max_chunk=0), dict(max_chunk=65), dict(rope_theta=0.0),
    dict(rope_theta=float("nan")),
])
def test_invalid_config_rejected_before_device(bad):
    kw = dict(n_layers=2, n_streams=3, n_q_heads=16, n_kv_heads=2, head_dim=128, window=64, max_chunk=8)
    kw.update(bad)
    theta = kw.pop("rope_theta", 1.0e6)
    cfg = a8r.make_config(**kw, rope_theta=theta)
    assert a8r.workspace_bytes(cfg) == 0
    with pytest.raises(a8r.A8RError) as e:
        a8r.cache_create(cfg)
    assert e.value.status in (a8r.A8R_EINVAL, a8r.A8R_EUNSUPPORTED)


def test_workspace_bytes_3b_batched():
    cfg = a8r.make_config(36, 64, 16, 2, 128, 4096, 1)
    ring = 36 * 64 * 2 * 4096 * 128 * 2
    assert a8r.workspace_bytes(cfg) >= 2 * ring
    assert a8r.workspace_bytes(cfg) < 2 * ring + 64 * 2**20


def test_null_handles_rejected():
    L = a8r.lib()
    assert L.a8r_append_kv(None, 0, 0, 1, 1, None, None, None, None) == a8r.A8R_EINVAL
    assert L.a8r_decode_attn(None, 0, 0, 1, None, None) == a8r.A8R_EINVAL
    assert L.a8r_chunk_attn(None, 0, 0, 1, 1, None, None) == a8r.A8R_EINVAL
    assert L.a8r_reset(None, 0, 1, None, None) == a8r.A8R_EINVAL
    assert b"NULL" in L.a8r_last_error()
    L.a8r_cache_destroy(None)


# ---- host ledger against the oracle ledger ----------------------------------------

def test_ledger_matches_oracle_random_ops():
    rng = random.Random(42)
    for window in [1, 2, 5, 31, 32, 33, 100, 4096]:
        n_layers, n_streams = 3, 4
        led = a8r.Ledger(n_layers, n_streams, window)
        ref = {(l, b): StreamLedger(window) for l in range(n_layers) for b in range(n_streams)}
        for _ in range(600):
            if rng.random() < 0.03:
                b0 = rng.randrange(n_streams)
                nb = rng.randint(1, n_streams - b0)
                pos = [rng.randrange(0, 1 << 50) for _ in range(nb)]
                slot = None if rng.random() < 0.5 else [rng.randrange(window) for _ in range(nb)]
                led.reset(b0, pos, slot)
                for i in range(nb):
                    for l in range(n_layers):
                        ref[(l, b0 + i)].reset(pos[i], None if slot is None else slot[i])
                continue
            layer = rng.randrange(n_layers)
            b0 = rng.randrange(n_streams)
            nb = rng.randint(1, n_streams - b0)
            n_new = rng.randint(1, min(window, 9))
            slots, ev = led.append(layer, b0, nb, n_new)
            for i in range(nb):
                s, e = ref[(layer, b0 + i)].append(n_new)
                assert list(slots[i]) == s
                assert list(ev[i]) == e
        for (l, b), r in ref.items():
            assert led.get(l, b) == r.state()


def test_ledger_100k_steps_w4096():
    led = a8r.Ledger(1, 1, 4096)
    ref = StreamLedger(4096)
    for _ in range(100_000 // 50):
        slots, ev = led.append(0, 0, 1, 50)
        s, e = ref.append(50)
        assert list(slots[0]) == s and list(ev[0]) == e
    assert led.get(0, 0) == ref.state() == (100_000, 4096, 100_000 % 4096)


def test_ledger_errors_change_nothing():
    led = a8r.Ledger(2, 2, 8)
    led.append(0, 0, 2, 3)
    before = [led.get(l, b) for l in range(2) for b in range(2)]
    bad_calls = [
        lambda: led.append(2, 0, 1, 1),        # layer out of range
        lambda: led.append(0, 1, 2, 1),        # streams out of range
        lambda: led.append(0, 0, 1, 0),        # n_new < 1
        lambda: led.append(0, 0, 1, 9),        # n_new > W
        lambda: led.reset(0, [-1]),            # negative position
        lambda: led.reset(0, [5], [8]),        # slot out of range
        lambda: led.reset(1, [5, 6]),          # streams out of range
    ]
    for call in bad_calls:
        with pytest.raises(a8r.A8RError) as e:
            call()
        assert e.value.status == a8r.A8R_EINVAL
    assert [led.get(l, b) for l in range(2) for b in range(2)] == before


def test_ledger_position_overflow_rejected():
    led = a8r.Ledger(1, 1, 4)
    led.reset(0, [2**63 - 4])
    slots, ev = led.append(0, 0, 1, 3)
    assert list(slots[0]) == [(2**63 - 4 + j) % 4 for j in range(3)]
    with pytest.raises(a8r.A8RError):
        led.append(0, 0, 1, 1)
    assert led.get(0, 0) == (2**63 - 1, 3, (2**63 - 1) % 4)


def test_reset_applies_to_all_layers_and_default_slot():
    led = a8r.Ledger(4, 2, 10)
    for l in range(4):
        led.append(l, 0, 2, 7)
    led.reset(1, [123])
    for l in range(4):
        assert led.get(l, 1) == (123, 0, 3)
        assert led.get(l, 0) == (7, 7, 7)


def test_header_is_plain_c_and_links(tmp_path):
    """A C11 program (gcc, -pedantic -Werror) includes the header, takes the
    address of every declared function, links against the library and runs its
    host-only calls: the boundary is a C ABI, not a C++ one."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    assert gcc, "gcc not found"
    names = declared_functions()
    src = tmp_path / "use_a8r.c"
    src.write_text("\n".join([
        "#include <stddef.h>",
        "#include <stdio.h>",
        "#include <string.h>",
        '#include "a8r.h"',
        '_Static_assert(sizeof(a8r_config) == 64, "a8r_config is 64 bytes");',
        '_Static_assert(offsetof(a8r_config, rope_theta) == 40, "rope_theta at 40");',
        "typedef void (*any_fn)(void);",
        "static const any_fn every_call[] = {",
        *[f"    (any_fn){n}," for n in names],
        "};",
        "int main(void) {",
        "    a8r_config cfg;",
        "    memset(&cfg, 0, sizeof cfg);",
        "    cfg.n_layers = 36; cfg.n_streams = 64; cfg.n_q_heads = 16; cfg.n_kv_heads = 2;",
        "    cfg.head_dim = 128; cfg.window = 4096; cfg.max_chunk = 8; cfg.dtype = A8R_BF16;",
        "    cfg.rope_theta = 1.0e6;",
        "    size_t ws = a8r_workspace_bytes(&cfg);",
        "    if (ws < (size_t)2 * 36 * 64 * 2 * 4096 * 128 * 2) return 2;",
        "    cfg.n_layers = 0;",
        "    a8r_cache* c = NULL;",
        "    if (a8r_cache_create(&cfg, NULL, NULL, 0, &c) != A8R_EINVAL || c != NULL) return 3;",
        "    if (strlen(a8r_last_error()) == 0) return 4;",
        "    a8r_ledger* led = NULL;",
        "    if (a8r_ledger_create(1, 1, 3, &led) != A8R_OK) return 5;",
        "    int32_t slots[5]; int64_t ev[5]; int64_t p; int32_t l, s;",
        "    for (int i = 0; i < 5; ++i)",
        "        if (a8r_ledger_append(led, 0, 0, 1, 1, &slots[i], &ev[i]) != A8R_OK) return 6;",
        "    if (a8r_ledger_get(led, 0, 0, &p, &l, &s) != A8R_OK) return 7;",
        "    a8r_ledger_destroy(led);",
        "    /* five tokens into a ring of three: slots 0 1 2 0 1, positions 0 and 1 evicted */",
        "    if (slots[3] != 0 || slots[4] != 1 || ev[2] != -1 || ev[3] != 0 || ev[4] != 1) return 8;",
        "    if (p != 5 || l != 3 || s != 2) return 9;",
        '    printf("%s: %zu calls, workspace %zu bytes\\n", a8r_version(),',
        "           sizeof every_call / sizeof every_call[0], ws);",
        "    return 0;",
        "}",
    ]) + "\n")
    exe = tmp_path / "use_a8r"
    libdir = os.path.dirname(a8r.LIB_PATH)
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                        os.path.join(ROOT, "include"), str(src), "-o", str(exe), os.path.abspath(a8r.LIB_PATH),
                        f"-Wl,-rpath,{libdir}", "-Wl,--allow-shlib-undefined"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert f"{len(names)} calls" in r.stdout
