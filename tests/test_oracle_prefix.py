"""Pins of the oracle's pinned prompt prefix (CPU only).

Independent of the oracle's own attention code:
* torch's scaled_dot_product_attention (float64) on [prefix; live window]
  rotated with the complex form of RoPE at consecutive indices 0 .. F + L - 1
  (queries at F + L - C + c), gathered from a plain history of appends, through
  fills, wraparounds, chunks and a reset;
* a "needle" key placed in the prefix and built to align with the query at the
  distance the reading gives it dominates the output after many wraparounds (the
  prefix is never evicted and its distance to the query stays fixed once the
  window is full);
* relative invariance: the same prefix + window attended from any absolute
  start position gives the same output (the prefix is re-based with the window).
Planted mistakes (the prefix evicted with the window, prefix indices restarting
at the window origin) must fail.
"""

import math

import numpy as np
import pytest

from oracle.model import OracleCache
from pinlib import complex_form, sdpa_reference

THETA = 1.0e6


def _run(w, hq, hkv, d, f, chunks, steps, seed, p0=0, reset_at=None):
    rng = np.random.default_rng(seed)
    ora = OracleCache(1, 1, hq, hkv, d, w)
    ora.reset(0, [p0], [p0 % w])
    pk, pv = rng.standard_normal((1, f, hkv, d)), rng.standard_normal((1, f, hkv, d))
    ora.append_prefix(0, 0, pk, pv)
    hist_k, hist_v = [], []
    worst = 0.0
    for t in range(steps):
        if reset_at is not None and t == reset_at:
            ora.reset(0, [12345], [7 % w])
            hist_k, hist_v = [], []
        n = chunks[t % len(chunks)]
        k, v = rng.standard_normal((1, n, hkv, d)), rng.standard_normal((1, n, hkv, d))
        ora.append(0, 0, k, v)
        hist_k += list(k[0])
        hist_v += list(v[0])
        c = min(n, len(hist_k), w)
        q = rng.standard_normal((1, c, hq, d))
        got = ora.chunk(0, 0, q)[0]
        live_k = np.array(hist_k[-w:])
        live_v = np.array(hist_v[-w:])
        seq_k = np.concatenate([pk[0], live_k])
        seq_v = np.concatenate([pv[0], live_v])
        exp = sdpa_reference(q[0], seq_k, seq_v, THETA, 1.0 / math.sqrt(d))
        worst = max(worst, float(np.max(np.abs(got - exp))))
    return worst


@pytest.mark.parametrize("w,hq,hkv,d,f,chunks,steps", [
    (8, 4, 2, 16, 3, [1], 30), (6, 2, 1, 8, 1, [2, 1, 3], 25), (16, 8, 2, 64, 40, [4], 20),
])
def test_prefix_equals_sdpa(w, hq, hkv, d, f, chunks, steps):
    assert _run(w, hq, hkv, d, f, chunks, steps, seed=w + f) <= 1e-12


def test_prefix_survives_reset():
    assert _run(8, 4, 2, 16, 5, [1, 2], 30, seed=3, reset_at=12) <= 1e-12


def test_prefix_needle_after_many_wraps():
    """A prefix key aligned with the query at its distance F + L - 1 - j takes
    almost all the weight, whatever the window has seen."""
    rng = np.random.default_rng(4)
    w, hq, hkv, d, f = 16, 2, 1, 32, 6
    ora = OracleCache(1, 1, hq, hkv, d, w)
    q = rng.standard_normal((hq, d))
    j = 2
    dist = f + w - 1 - j                       # query index minus the needle's, window full
    # complex_form(k, a) . complex_form(q, b) depends on b - a only: a key equal to
    # R(dist) q (in complex form) scores |q|^2
    needle = 6.0 * complex_form(q[0], dist, THETA)
    pk = rng.standard_normal((1, f, hkv, d)) * 0.1
    pk[0, j, 0] = needle
    pv = np.zeros((1, f, hkv, d))
    pv[0, j, 0, 0] = 1.0                     # one-hot value: out[0] is the needle weight
    ora.append_prefix(0, 0, pk, pv)
    for _ in range(10 * w):
        ora.append(0, 0, rng.standard_normal((1, 1, hkv, d)) * 0.1, rng.standard_normal((1, 1, hkv, d)) * 0.1)
    out = ora.decode(0, 0, q[None])[0, 0]
    assert out[0] > 0.99 and np.all(np.abs(out[1:]) < 0.05)


def test_prefix_relative_invariance():
    a = _run(8, 4, 2, 16, 4, [1, 3], 20, seed=5, p0=0)
    b = _run(8, 4, 2, 16, 4, [1, 3], 20, seed=5, p0=2**24 + 5)
    assert a <= 1e-12 and b <= 1e-12


@pytest.mark.parametrize("mutant", ["evicted", "restart_index"])
def test_planted_prefix_mistakes_fail(monkeypatch, mutant):
    import oracle.model as model_mod
    orig = model_mod.OracleCache.chunk

    def bad_chunk(self, layer, b0, q):
        if mutant == "evicted":                 # prefix dropped once the window is full
            led = self.ledger(layer, b0)
            if led.length == self.window:
                saved = dict(self._prefix)
                self._prefix.clear()
                try:
                    return orig(self, layer, b0, q)
                finally:
                    self._prefix.update(saved)
            return orig(self, layer, b0, q)
        # prefix indices restarting at the window origin: prefix and window both from 0
        q = np.asarray(q, dtype=np.float64)
        out = np.empty_like(q)
        kw, vw, _ = self.window_kv(layer, b0)
        pk, pv = self.prefix_kv(layer, b0)
        from oracle.attention import attend, default_scale
        from oracle.rope import rotate
        c = q.shape[1]
        n = kw.shape[0]
        r_q = n - c + np.arange(c)
        kr = np.concatenate([rotate(pk, np.arange(pk.shape[0])[:, None]), rotate(kw, np.arange(n)[:, None])])
        vis = np.concatenate([np.ones((c, pk.shape[0]), bool), np.arange(n)[None, :] <= r_q[:, None]], axis=1)
        out[0] = attend(rotate(q[0], r_q[:, None]), kr, np.concatenate([pv, vw]), default_scale(q.shape[-1]), vis)
        return out

    monkeypatch.setattr(model_mod.OracleCache, "chunk", bad_chunk)
    assert _run(8, 4, 2, 16, 3, [1], 30, seed=8) > 1e-6
