"""Checks that pin the oracle to things other than itself (CPU only).

Used by the oracle tests; each function raises AssertionError when the oracle
(or a planted mutant of it) disagrees with the independent computation.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle.attention as att
from oracle.model import OracleCache

TWO52 = 2.0 ** -52


def complex_form(x, index, theta):
    """RoPE as complex multiplication: pair i is x_i + j x_{i+D/2}, rotated by
    exp(j * index * exp(-(2i/D) ln theta))."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    i = np.arange(h, dtype=np.float64)
    f = np.exp(-(2.0 * i / d) * math.log(theta))
    z = x[..., :h] + 1j * x[..., h:]
    idx = np.asarray(index, dtype=np.float64)[..., None]
    w = z * np.exp(1j * idx * f)
    return np.concatenate([w.real, w.imag], axis=-1)


def sdpa_reference(q, k_win, v_win, theta, scale):
    """torch's scaled_dot_product_attention (float64, CPU) on operands rotated
    with ``complex_form`` at indices 0..L-1 (keys) and L-C..L-1 (queries), with a
    causal band mask and grouped-query head sharing.  q [C, Hq, D]."""
    q = np.asarray(q, dtype=np.float64)
    c, hq, d = q.shape
    n, hkv, _ = k_win.shape
    r_q = np.arange(n - c, n)
    qr = complex_form(q, r_q[:, None], theta)
    kr = complex_form(k_win, np.arange(n)[:, None], theta)
    mask = np.arange(n)[None, :] <= r_q[:, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qr).permute(1, 0, 2)[None],
        torch.from_numpy(kr).permute(1, 0, 2)[None],
        torch.from_numpy(np.asarray(v_win, dtype=np.float64)).permute(1, 0, 2)[None],
        attn_mask=torch.from_numpy(mask), scale=scale, enable_gqa=(hq != hkv))
    return out[0].permute(1, 0, 2).numpy()


def pin_sdpa(chunk_fn=None, theta=1.0e6):
    """chunk_rebased (or a mutant) equals torch SDPA on pre-rotated operands."""
    chunk_fn = chunk_fn or att.chunk_rebased
    rng = np.random.default_rng(11)
    for (hq, hkv, d, n, c) in [(8, 8, 64, 40, 1), (16, 2, 128, 33, 1), (16, 2, 128, 50, 8),
                               (4, 1, 64, 9, 9), (6, 3, 32, 17, 4)]:
        q = rng.standard_normal((c, hq, d))
        k = rng.standard_normal((n, hkv, d))
        v = rng.standard_normal((n, hkv, d))
        scale = 1.0 / math.sqrt(d)
        got = chunk_fn(q, k, v, theta, None)
        exp = sdpa_reference(q, k, v, theta, scale)
        err = np.max(np.abs(got - exp))
        assert err <= 1e-12, (hq, hkv, d, n, c, err)


def brute_force_tolerance(max_pos, q, k, v, scale):
    """Bound on |re-based - absolute| from the float64 angle error alone.

    An angle index*f is formed with relative error <= 2**-53, i.e. absolute error
    <= index * 2**-53 (f <= 1); cos/sin add ~2**-53.  A score moves by at most
    scale * 2 * max_angle_err * |q| |k|, a softmax weight by that much relative,
    and the output by sum_j |dp_j| |v_j| <= 2 * dscore * max|v|.
    """
    ang = (2 * max_pos + 4) * TWO52
    ds = scale * 2 * ang * np.max(np.linalg.norm(q, axis=-1)) * np.max(np.linalg.norm(k, axis=-1))
    return 4 * ds * np.max(np.abs(v)) + 64 * TWO52 * np.max(np.abs(v))


def pin_brute_force(cache_cls=OracleCache, *, window=8, hq=16, hkv=2, d=64, p0=0, s0=None,
                    chunk=1, steps=40, theta=1.0e6, seed=5, check_every=1):
    """Run one stream through the cache model; after each append compare its
    re-based attention with brute force at absolute positions over the full
    history since the reset."""
    rng = np.random.default_rng(seed)
    cache = cache_cls(1, 1, hq, hkv, d, window, theta)
    cache.reset(0, [p0], None if s0 is None else [s0])
    hist_pos, hist_k, hist_v = [], [], []
    pos = p0
    worst = 0.0
    for step in range(steps):
        k = rng.standard_normal((1, chunk, hkv, d))
        v = rng.standard_normal((1, chunk, hkv, d))
        q = rng.standard_normal((1, chunk, hq, d))
        cache.append(0, 0, k, v)
        for j in range(chunk):
            hist_pos.append(pos + j)
            hist_k.append(k[0, j])
            hist_v.append(v[0, j])
        pos += chunk
        if step % check_every:
            continue
        got = cache.chunk(0, 0, q)[0]
        q_pos = np.arange(pos - chunk, pos)
        exp = att.brute_force(q[0], q_pos, hist_pos, hist_k, hist_v, pos, window, theta)
        tol = brute_force_tolerance(pos, q, np.array(hist_k), np.array(hist_v), 1 / math.sqrt(d))
        err = float(np.max(np.abs(got - exp)))
        worst = max(worst, err)
        assert err <= tol, (step, pos, err, tol)
    return worst
