"""Split-half rotary position embedding at an arbitrary integer index, float64.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Sources:
* "Audio8-ASR-0.1B in audio.cpp", section "Architecture": the decoder's RoPE
  base is theta = 1e6.
* "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift": these
  checkpoints were trained with the split-half (rotate_half) pairing; the
  interleaved pairing runs but produces nonsense.

Reading (the pages give theta and the pairing, not the frequency law): the usual
RoPE frequencies inv_freq_i = theta ** (-2 i / D) for i in [0, D/2), and the
pair rotated by angle idx * inv_freq_i is (x_i, x_{i + D/2}):

    y_i       = x_i       cos(a_i) - x_{i+D/2} sin(a_i)
    y_{i+D/2} = x_{i+D/2} cos(a_i) + x_i       sin(a_i)

Angles are formed in float64 from the exact integer index, so the oracle stays
exact (to ~1e-16 relative) for any index the tests use, including absolute
positions beyond 2**24 where float32 can no longer count.

Pinned by ``tests/test_oracle_rope.py``: identity at 0, a hand-computed D=2
value, a complex-exponential formulation, norm preservation, composition and
relative invariance under an origin shift.
"""

from __future__ import annotations

import numpy as np

DEFAULT_THETA = 1.0e6


def inv_freq(head_dim: int, theta: float = DEFAULT_THETA) -> np.ndarray:
    """theta ** (-2 i / D), i = 0 .. D/2 - 1, float64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rotate(x: np.ndarray, index, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Rotate the last axis of x (length D) by integer index/indices.

    ``index`` broadcasts against ``x.shape[:-1]`` (one index per row vector).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    idx = np.asarray(index, dtype=np.int64).astype(np.float64)  # exact below 2**53
    ang = idx[..., None] * inv_freq(d, theta)                     # [..., D/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
