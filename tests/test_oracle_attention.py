"""Pins of the oracle's re-based window attention (CPU only).

Independent of the oracle's own formulas:
* a hand-worked W=2 example with an eviction (tests/golden/window_d2_hand.json);
* special cases with closed forms: one live token returns its value; a zero
  query returns the window mean; a "needle" key built (through the complex form
  of RoPE) to align with the query dominates at any absolute position;
* torch's scaled_dot_product_attention in float64 on operands rotated with the
  complex form (a library routine for the window-fits-history case);
* brute-force attention at absolute positions over the full history equals the
  ring + re-basing result, including across many wraparounds and at positions
  beyond 2**24 (within the float64 angle-error bound derived in pinlib).
Planted mistakes in the oracle (query origin off by one, a query that cannot see
itself, oldest-kept eviction, naive float32 absolute angles, wrong scale, wrong
GQA head map) must each fail at least one of these pins.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.attention as att
import oracle.model as model_mod
import oracle.rope as rope_mod
from oracle.ledger import StreamLedger
from oracle.model import OracleCache
from pinlib import complex_form, pin_brute_force, pin_sdpa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_window_hand():
    with open(os.path.join(GOLDEN, "window_d2_hand.json")) as f:
        fx = json.load(f)
    expected = [1.0 / (1.0 + math.exp((1.0 - math.cos(1.0)) / math.sqrt(2.0)))]
    expected.append(1.0 - expected[0])
    assert expected == pytest.approx(fx["expected"], abs=1e-15)
    c = OracleCache(1, 1, 1, 1, 2, fx["window"])
    ev = None
    for i, _ in enumerate(fx["positions"]):
        k = np.array(fx["k"][i], dtype=np.float64).reshape(1, 1, 1, 2)
        v = np.array(fx["v"][i], dtype=np.float64).reshape(1, 1, 1, 2)
        _, ev = c.append(0, 0, k, v)
    assert ev == [[fx["evicted_on_last_append"]]]
    out = c.decode(0, 0, np.array(fx["q_last"]).reshape(1, 1, 2))
    assert out[0, 0] == pytest.approx(expected, abs=1e-15)


def test_single_live_token_returns_value():
    rng = np.random.default_rng(0)
    for hq, hkv in [(8, 8), (16, 2)]:
        q = rng.standard_normal((hq, 128))
        k = rng.standard_normal((1, hkv, 128))
        v = rng.standard_normal((1, hkv, 128))
        out = att.decode_rebased(q, k, v)
        g = hq // hkv
        for h in range(hq):
            assert np.allclose(out[h], v[0, h // g], rtol=0, atol=1e-15)


def test_zero_query_gives_window_mean():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((37, 2, 64))
    v = rng.standard_normal((37, 2, 64))
    out = att.decode_rebased(np.zeros((16, 64)), k, v)
    for h in range(16):
        assert np.allclose(out[h], v[:, h // 8].mean(axis=0), rtol=0, atol=1e-14)


@pytest.mark.parametrize("p0", [0, 1_000_000, 2**24 - 3])
def test_needle(p0):
    """Key j is set to R(p_q - p_j) (alpha q) for head 0 (built with the complex
    form), so its score is alpha |q|^2 / sqrt(D) wherever the window sits."""
    rng = np.random.default_rng(p0 % 97)
    d, w, alpha = 128, 64, 400.0
    c = OracleCache(1, 1, 8, 1, d, w)
    c.reset(0, [p0])
    n_tok = w + 19                      # wraps once; the window is the last 64
    ks = rng.standard_normal((n_tok, 1, d)) * 0.1
    vs = rng.standard_normal((n_tok, 1, d))
    q = rng.standard_normal((8, d))
    q[0] /= np.linalg.norm(q[0])
    p_q = p0 + n_tok - 1
    j = n_tok - 30                      # a live token, neither oldest nor newest
    ks[j, 0] = complex_form(alpha * q[0], p_q - (p0 + j), 1.0e6)
    for t in range(n_tok):
        c.append(0, 0, ks[t][None, None], vs[t][None, None])
    out = c.decode(0, 0, q[None])[0]
    assert np.max(np.abs(out[0] - vs[j, 0])) < 1e-3
    hist = np.arange(p0, p0 + n_tok)
    bf = att.brute_force(q[None], [p_q], hist, ks, vs, p0 + n_tok, w)
    assert np.max(np.abs(bf[0, 0] - vs[j, 0])) < 1e-3


def test_sdpa_reference():
    pin_sdpa()


@pytest.mark.parametrize("cfg", [
    dict(window=8, hq=8, hkv=8, d=64, p0=0, chunk=1, steps=60),
    dict(window=8, hq=16, hkv=2, d=128, p0=1_000_000, s0=3, chunk=1, steps=40),
    dict(window=16, hq=16, hkv=2, d=128, p0=2**24 - 20, chunk=4, steps=20),
    dict(window=7, hq=4, hkv=2, d=64, p0=12345, s0=6, chunk=3, steps=25),
    dict(window=64, hq=8, hkv=8, d=64, p0=0, chunk=1, steps=256, check_every=16),
])
def test_brute_force_equals_rebased(cfg):
    pin_brute_force(**cfg)


def test_brute_force_error_small_at_2p24():
    worst = pin_brute_force(window=32, hq=16, hkv=2, d=128, p0=2**24 - 40, chunk=8, steps=12)
    assert worst < 1e-9


# ---- planted mistakes: each must fail a pin ------------------------------------

def query_off_by_one(q, k_win, v_win, theta=1.0e6, scale=None):
    q = np.asarray(q, dtype=np.float64)
    c, _, d = q.shape
    n = k_win.shape[0]
    scale = att.default_scale(d) if scale is None else scale
    r_k = np.arange(n)
    r_q = n - c + np.arange(c)
    qr = att.rotate(q, (r_q + 1)[:, None], theta)        # query origin shifted by one
    kr = att.rotate(np.asarray(k_win, np.float64), r_k[:, None], theta)
    return att.attend(qr, kr, np.asarray(v_win, np.float64), scale, r_k[None] <= r_q[:, None])


def exclude_self(q, k_win, v_win, theta=1.0e6, scale=None):
    q = np.asarray(q, dtype=np.float64)
    c, _, d = q.shape
    n = k_win.shape[0]
    scale = att.default_scale(d) if scale is None else scale
    r_k = np.arange(n)
    r_q = n - c + np.arange(c)
    qr = att.rotate(q, r_q[:, None], theta)
    kr = att.rotate(np.asarray(k_win, np.float64), r_k[:, None], theta)
    vis = r_k[None] < r_q[:, None]
    vis[:, 0] = True                                     # keep rows non-empty
    return att.attend(qr, kr, np.asarray(v_win, np.float64), scale, vis)


def wrong_scale(q, k_win, v_win, theta=1.0e6, scale=None):
    return att.chunk_rebased(q, k_win, v_win, theta, 1.0 / q.shape[-1])


def wrong_gqa_map(q, k_win, v_win, theta=1.0e6, scale=None):
    q = np.asarray(q, dtype=np.float64)
    hkv = k_win.shape[1]
    hq = q.shape[1]
    perm = [(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)]   # h -> h % Hkv
    out = att.chunk_rebased(q[:, perm], k_win, v_win, theta, scale)
    inv = np.argsort(perm)
    return out[:, inv]


class EvictNewestLedger(StreamLedger):
    """Keeps the oldest tokens and overwrites the newest slot once full."""

    def append(self, n_new):
        slots, evicted = [], []
        for j in range(n_new):
            if self.length == self.window:
                last = (self.next_slot - 1) % self.window
                slots.append(last)
                evicted.append(self.next_pos + j - 1)
            else:
                slots.append(self.next_slot)
                evicted.append(-1)
                self.next_slot = (self.next_slot + 1) % self.window
                self.length += 1
        self.next_pos += n_new
        return slots, evicted


class NaiveFp32Absolute(OracleCache):
    """Attention at absolute positions with float32 angles fl(p) * fl(f)."""

    def chunk(self, layer, b0, q):
        q = np.asarray(q, dtype=np.float64)
        out = np.empty_like(q)
        for i in range(q.shape[0]):
            kw, vw, origin = self.window_kv(layer, b0 + i)
            n, c, d = kw.shape[0], q.shape[1], q.shape[-1]
            f32 = rope_mod.inv_freq(d, self.theta).astype(np.float32)

            def rot(x, pos):
                a = (pos.astype(np.float32)[:, None] * f32[None, :]).astype(np.float64)
                a = a[:, None, :]
                x1, x2 = x[..., :d // 2], x[..., d // 2:]
                return np.concatenate([x1 * np.cos(a) - x2 * np.sin(a),
                                       x2 * np.cos(a) + x1 * np.sin(a)], axis=-1)
            kp = origin + np.arange(n)
            qp = origin + n - c + np.arange(c)
            vis = kp[None] <= qp[:, None]
            out[i] = att.attend(rot(q[i], qp), rot(kw, kp), vw, 1 / math.sqrt(d), vis)
        return out


@pytest.mark.parametrize("mutant", [query_off_by_one, exclude_self, wrong_scale, wrong_gqa_map])
def test_planted_attention_mistakes_fail_sdpa(mutant):
    with pytest.raises(AssertionError):
        pin_sdpa(mutant)


@pytest.mark.parametrize("mutant", [query_off_by_one, exclude_self])
def test_planted_attention_mistakes_fail_brute_force(monkeypatch, mutant):
    monkeypatch.setattr(model_mod, "chunk_rebased", mutant)
    with pytest.raises(AssertionError):
        pin_brute_force(window=8, hq=8, hkv=8, d=64, p0=100, chunk=1, steps=20)


def test_planted_evict_newest_fails(monkeypatch):
    monkeypatch.setattr(model_mod, "StreamLedger", EvictNewestLedger)
    with pytest.raises(AssertionError):
        pin_brute_force(window=8, hq=8, hkv=8, d=64, p0=0, chunk=1, steps=30)


def test_planted_naive_fp32_absolute_fails_at_2p24():
    with pytest.raises(AssertionError):
        pin_brute_force(NaiveFp32Absolute, window=32, hq=16, hkv=2, d=128, p0=2**24 - 40,
                        chunk=8, steps=12)
