"""CPU pins of the window re-prefill oracle (oracle/prefill.py and
OracleCache.rebuild): a hand-derived fixture, identity weights, linearity, the
head layout of the output features, and a rebuilt window attending exactly as
the same tokens appended one by one; planted mistakes must fail."""

import json
import os

import numpy as np
import pytest

import oracle.prefill as prefill
from oracle.model import OracleCache

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "prefill_hand.json")


def fixture():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_hand():
    g = fixture()
    k, v = prefill.rebuild_kv(np.array(g["hidden"]), np.array(g["w_k"]), np.array(g["w_v"]), 1, 2)
    assert np.array_equal(k[:, 0], np.array(g["k"]))
    assert np.array_equal(v[:, 0], np.array(g["v"]))


def test_output_feature_is_head_major():
    g = fixture()
    k, _ = prefill.rebuild_kv(np.array(g["hidden"]), np.array(g["w_k"]), np.array(g["w_v"]), 2, 1)
    # feature kh * D + d with D = 1: head 0 is feature 0, head 1 feature 1
    assert np.array_equal(k[:, 0, 0], np.array(g["k"])[:, 0])
    assert np.array_equal(k[:, 1, 0], np.array(g["k"])[:, 1])


def test_identity_weights_return_the_hidden_states():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 8))
    k, v = prefill.rebuild_kv(h, np.eye(8), 2 * np.eye(8), 2, 4)
    assert np.array_equal(k.reshape(5, 8), h)
    assert np.array_equal(v.reshape(5, 8), 2 * h)


def test_linear_in_the_hidden_states():
    rng = np.random.default_rng(2)
    h1, h2 = rng.standard_normal((7, 16)), rng.standard_normal((7, 16))
    w = rng.standard_normal((6, 16))
    lhs = prefill.project(3 * h1 - 0.5 * h2, w)
    rhs = 3 * prefill.project(h1, w) - 0.5 * prefill.project(h2, w)
    assert np.max(np.abs(lhs - rhs)) < 1e-12


@pytest.mark.parametrize("w,n,p0", [(16, 16, 100), (16, 9, 40), (33, 20, 2**24 + 5)])
def test_rebuilt_window_attends_like_appended_tokens(w, n, p0):
    """A window rebuilt from hidden states equals, for attention, the same
    projected tokens appended one by one at the same positions: the re-based
    attention sees only the window's contents and their order."""
    rng = np.random.default_rng(w + n)
    hq, hkv, d, hid = 4, 2, 8, 24
    h = rng.standard_normal((n, hid))
    wk, wv = rng.standard_normal((hkv * d, hid)), rng.standard_normal((hkv * d, hid))
    k, v = prefill.rebuild_kv(h, wk, wv, hkv, d)
    a = OracleCache(1, 1, hq, hkv, d, w)
    a.reset(0, [p0 - w - 3], [5])
    for _ in range(w + 3):                             # a full, wrapped window of other tokens
        a.append(0, 0, rng.standard_normal((1, 1, hkv, d)), rng.standard_normal((1, 1, hkv, d)))
    a.rebuild(0, 0, k[None], v[None])
    led = a.ledger(0, 0)
    assert (led.next_pos, led.length, led.next_slot) == (p0, n, n % w)
    b = OracleCache(1, 1, hq, hkv, d, w)
    b.reset(0, [p0 - n])
    b.append(0, 0, k[None], v[None])
    q = rng.standard_normal((1, 3, hq, d))
    assert np.max(np.abs(a.chunk(0, 0, q) - b.chunk(0, 0, q))) < 1e-12
    # the next append continues the rebuilt window at slot n mod W
    kn, vn = rng.standard_normal((1, 1, hkv, d)), rng.standard_normal((1, 1, hkv, d))
    slots, _ = a.append(0, 0, kn, vn)
    assert slots[0][0] == n % w
    b.append(0, 0, kn, vn)
    assert np.max(np.abs(a.decode(0, 0, q[:, 0]) - b.decode(0, 0, q[:, 0]))) < 1e-12


def test_planted_transposed_weight_fails(monkeypatch):
    g = fixture()
    monkeypatch.setattr(prefill, "project",
                        lambda hidden, weight: np.asarray(hidden, np.float64) @ np.asarray(weight, np.float64))
    k, _ = prefill.rebuild_kv(np.array(g["hidden"]), np.array(g["w_k"]), np.array(g["w_v"]), 1, 2)
    assert not np.array_equal(k[:, 0], np.array(g["k"]))


def test_planted_window_in_wrong_order_fails():
    """Oldest first matters: the same tokens rebuilt newest first attend
    differently."""
    rng = np.random.default_rng(3)
    hq, hkv, d, w, n = 4, 1, 8, 16, 12
    k, v = rng.standard_normal((1, n, hkv, d)), rng.standard_normal((1, n, hkv, d))
    a, b = OracleCache(1, 1, hq, hkv, d, w), OracleCache(1, 1, hq, hkv, d, w)
    for c in (a, b):
        c.reset(0, [50])
        c.append(0, 0, rng.standard_normal((1, n, hkv, d)), rng.standard_normal((1, n, hkv, d)))
    a.rebuild(0, 0, k, v)
    b.rebuild(0, 0, k[:, ::-1], v[:, ::-1])
    q = rng.standard_normal((1, hq, d))
    assert np.max(np.abs(a.decode(0, 0, q) - b.decode(0, 0, q))) > 1e-3
