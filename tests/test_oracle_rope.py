"""Pins of the oracle's split-half rotary embedding (CPU only).

Independent checks:
* hand-worked D=2 values (tests/golden/rope_d2_hand.json), re-evaluated here
  with ``math.cos`` / ``math.sin``;
* the complex-number form of RoPE: pair i is z_i = x_i + j x_{i+D/2} and the
  rotation multiplies it by exp(j * index * theta**(-2i/D)), with the frequency
  formed as exp(-(2i/D) ln theta) - a different computation path from the oracle's;
* rotation identities: norm preservation, composition R(a)R(b) = R(a+b) and
  relative invariance <R(a)q, R(b)k> = <R(a+d)q, R(b+d)k> for large shifts d.
Planted mistakes (interleaved pairing, a sign flip, a wrong frequency law) must
fail the complex-form pin.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.rope as rope
from pinlib import complex_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TWO52 = 2.0 ** -52


def pin_complex_form(rotate_fn, theta=1.0e6):
    rng = np.random.default_rng(7)
    for d in (2, 8, 64, 128):
        x = rng.standard_normal((33, d))
        idx = rng.integers(0, 100_000, size=33)
        got = rotate_fn(x, idx, theta)
        exp = complex_form(x, idx, theta)
        # |angle error| <= index * 2**-52 in either path, plus a few ulps
        tol = 8 * (100_000 * TWO52 + TWO52) * np.max(np.abs(x)) * 2
        assert np.max(np.abs(got - exp)) <= tol, (d, np.max(np.abs(got - exp)), tol)


def test_golden_d2_hand_values():
    with open(os.path.join(GOLDEN, "rope_d2_hand.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        r = case["index"]
        closed = [math.cos(r), math.sin(r)]
        assert closed == pytest.approx(case["expected"], abs=1e-16)
        got = rope.rotate(np.array(fx["x"]), r, fx["theta"])
        assert got == pytest.approx(closed, abs=2e-16)


def test_identity_at_zero():
    x = np.random.default_rng(1).standard_normal((5, 128))
    assert np.array_equal(rope.rotate(x, 0), x)


def test_complex_form():
    pin_complex_form(rope.rotate)


def test_inv_freq_values():
    f = rope.inv_freq(128, 1.0e6)
    assert f[0] == 1.0
    # last pair: theta ** (-126/128)
    assert f[-1] == pytest.approx(math.exp(-(126 / 128) * math.log(1.0e6)), rel=1e-15)
    assert np.all(np.diff(f) < 0)


@pytest.mark.parametrize("d", [2, 64, 128])
def test_norm_preserved_per_pair(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((50, d))
    idx = rng.integers(0, 2**24 + 8192, size=50)
    y = rope.rotate(x, idx)
    h = d // 2
    n_in = x[:, :h] ** 2 + x[:, h:] ** 2
    n_out = y[:, :h] ** 2 + y[:, h:] ** 2
    assert np.max(np.abs(n_in - n_out)) <= 16 * TWO52 * np.max(n_in)


def test_composition():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 128))
    for a, b in [(1, 2), (4095, 1), (1_000_000, 4096), (2**24, 8191)]:
        lhs = rope.rotate(rope.rotate(x, a), b)
        rhs = rope.rotate(x, a + b)
        tol = 8 * (a + b + 1) * TWO52 * np.max(np.abs(x)) * 2
        assert np.max(np.abs(lhs - rhs)) <= tol


@pytest.mark.parametrize("delta", [1, 4096, 1_000_000, 2**24])
def test_relative_invariance(delta):
    rng = np.random.default_rng(delta % 1000)
    q = rng.standard_normal(128)
    k = rng.standard_normal((64, 128))
    a = 4095
    b = rng.integers(0, 4096, size=64)
    s0 = rope.rotate(k, b) @ rope.rotate(q, a)
    s1 = rope.rotate(k, b + delta) @ rope.rotate(q, a + delta)
    tol = 8 * (a + delta + 1) * TWO52 * np.linalg.norm(q) * np.max(np.linalg.norm(k, axis=1)) * 4
    assert np.max(np.abs(s0 - s1)) <= tol


# ---- planted mistakes: each must fail the complex-form pin ----------------------

def interleaved(x, index, theta=1.0e6):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(index, dtype=np.float64)[..., None] * rope.inv_freq(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xo * c + xe * s
    return y


def sign_flipped(x, index, theta=1.0e6):
    return rope.rotate(x, -np.asarray(index), theta)


def wrong_freq_law(x, index, theta=1.0e6):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    f = np.power(theta, -np.arange(h) / d)          # theta**(-i/D): exponent halved
    ang = np.asarray(index, dtype=np.float64)[..., None] * f
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


@pytest.mark.parametrize("mutant", [interleaved, sign_flipped, wrong_freq_law])
def test_planted_rope_mistakes_fail(mutant):
    with pytest.raises(AssertionError):
        pin_complex_form(mutant)
