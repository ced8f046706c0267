"""Pins of the ring's key storage form (oracle/storage.py), CPU only.

Independent of the float32 emulation itself:
* offset 0 in a tile stores the input bits (R(0) is the identity);
* the stored bits depend on the slot only through its offset in a 32-slot tile
  (slots 32 apart store the same bits), and different offsets differ;
* undoing the rotation in float64 (oracle.rope, R(-t)) recovers the input
  within one rounding to the cache dtype;
* attention read from the stored keys, each rotated by R(r - t) in float64
  (r its re-based index, t its slot's tile offset), equals the re-based
  attention of the raw keys (oracle.attention) within the rounding bound, on a
  wrapped window whose ring size is not a multiple of 32.
Planted mistakes (the slot instead of its tile offset; the re-based index
instead of the slot) must fail.
"""

import math

import numpy as np
import pytest

import oracle.attention as att
import oracle.rebase as rb
import oracle.rope as rope
import oracle.storage as storage


def _keys(rng, n, hkv, d, bf16):
    x = rng.standard_normal((n, hkv, d)).astype(np.float32)
    return rb.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("bf16", [True, False])
def test_offset_zero_stores_input(bf16):
    rng = np.random.default_rng(1)
    k = _keys(rng, 3, 2, 128, bf16)
    got = storage.stored_keys(k, np.array([0, 32, 4064]), bf16)
    assert np.array_equal(got.view(np.uint32), k.view(np.uint32))


@pytest.mark.parametrize("bf16", [True, False])
def test_depends_on_tile_offset_only(bf16):
    rng = np.random.default_rng(2)
    k = _keys(rng, 1, 2, 64, bf16)
    for t in (1, 7, 31):
        a = storage.stored_keys(k, t, bf16)
        for m in (1, 5, 127):
            assert np.array_equal(a.view(np.uint32), storage.stored_keys(k, t + 32 * m, bf16).view(np.uint32))
    assert not np.array_equal(storage.stored_keys(k, 3, bf16), storage.stored_keys(k, 4, bf16))


@pytest.mark.parametrize("bf16,rel", [(True, 2.0 ** -8), (False, 2.0 ** -22)])
def test_inverse_recovers_input_within_one_rounding(bf16, rel):
    rng = np.random.default_rng(3)
    n, hkv, d = 64, 2, 128
    k = _keys(rng, n, hkv, d, bf16)
    slots = rng.integers(0, 5000, n)
    st = storage.stored_keys(k, slots[:, None], bf16).astype(np.float64)
    back = rope.rotate(st, -(slots % 32)[:, None])
    # per pair (i, i + D/2): the error of one rounding of the rotated pair
    h = d // 2
    pair_norm = np.sqrt(k[..., :h].astype(np.float64) ** 2 + k[..., h:].astype(np.float64) ** 2)
    err = np.sqrt((back[..., :h] - k[..., :h]) ** 2 + (back[..., h:] - k[..., h:]) ** 2)
    assert np.all(err <= rel * pair_norm + 1e-7)


def _read_from_stored(q, stored, v, slots, c):
    """Attention of the C newest queries over a window read from stored keys:
    key j (re-based index j, slot slots[j]) rotated by R(j - slots[j] mod 32)."""
    n = stored.shape[0]
    idx = np.arange(n)
    k_eff = rope.rotate(stored.astype(np.float64), (idx - slots % 32)[:, None])
    r_q = n - c + np.arange(c)
    qr = rope.rotate(q, r_q[:, None])
    vis = idx[None, :] <= r_q[:, None]
    return att.attend(qr, k_eff, v, att.default_scale(q.shape[-1]), vis)


@pytest.mark.parametrize("bf16,tol", [(True, 5e-3), (False, 1e-6)])
def test_attention_from_stored_equals_rebased(bf16, tol):
    rng = np.random.default_rng(4)
    w, hkv, hq, d, c = 100, 2, 8, 64, 4
    oldest = 77                                   # the window wraps past slot W - 1
    slots = (oldest + np.arange(w)) % w
    k = _keys(rng, w, hkv, d, bf16)
    v = _keys(rng, w, hkv, d, bf16).astype(np.float64)
    q = _keys(rng, c, hq, d, bf16).astype(np.float64)
    st = storage.stored_keys(k, slots[:, None], bf16)
    got = _read_from_stored(q, st, v, slots, c)
    exp = att.chunk_rebased(q, k.astype(np.float64), v)
    assert float(np.max(np.abs(got - exp))) <= tol


def test_planted_storage_mistakes_fail(monkeypatch):
    rng = np.random.default_rng(5)
    # the slot itself instead of its offset in the tile
    monkeypatch.setattr(storage, "TILE", 1 << 30)
    k = _keys(rng, 1, 2, 64, True)
    assert not np.array_equal(storage.stored_keys(k, 3, True), storage.stored_keys(k, 35, True))
    monkeypatch.undo()
    # the re-based index instead of the slot: the read no longer matches
    w, hkv, hq, d, c = 100, 2, 8, 64, 4
    slots = (77 + np.arange(w)) % w
    k = _keys(rng, w, hkv, d, True)
    v = _keys(rng, w, hkv, d, True).astype(np.float64)
    q = _keys(rng, c, hq, d, True).astype(np.float64)
    bad = storage.stored_keys(k, np.arange(w)[:, None], True)
    got = _read_from_stored(q, bad, v, slots, c)
    exp = att.chunk_rebased(q, k.astype(np.float64), v)
    assert float(np.max(np.abs(got - exp))) > 5e-2
