"""Storage form of keys in the ring (tile-phase K): the bits a slot must hold.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

The pages fix what attention computes, not how the ring stores a key; this is
the library's storage reading, stated so that ring contents can be checked bit
for bit.  Source of the method it serves: "Audio8 ASR Infinite: What It
Actually Takes to Listen Forever", section "Inside the Rolling KV Cache and
Exact RoPE Re-Basing" (keys are re-based on read; a stored key is never
re-rotated as the origin moves).

A key k written to ring slot s is stored as R(s mod 32) k: the split-half
rotation by the slot's offset in its 32-slot tile, a quantity that does not
depend on the window's origin and never changes while the token is live.  The
arithmetic is that of ``rebase.rotate_f32`` (float32 multiplies and adds, no
fused multiply-add) with coefficients (cos, sin)(t * theta^(-2i/D)) computed in
float64 and rounded once to float32 (``rebase.coef_f32``), then one rounding to
the cache dtype (bf16: nearest, ties to even).  Values are stored as appended.
Pinned prefix token j of a stream is stored the same way at offset j mod 32.

Attention is unaffected in exact arithmetic: a key at re-based index
r = rho + t (t = s mod 32) enters as R(rho) R(t) k = R(r) k.

Pinned by ``tests/test_oracle_storage.py``: offset 0 stores the input bits;
slots 32 apart store identical bits; undoing the rotation in float64 recovers
the input within one rounding; attention over the stored keys rotated by
R(r - t) in float64 equals the re-based attention of the raw keys within the
rounding bound; planted mistakes (the slot instead of its tile offset, the
re-based index instead of the slot) must fail.
"""

from __future__ import annotations

import numpy as np

from .rebase import coef_f32, rotate_f32, to_storage
from .rope import DEFAULT_THETA

TILE = 32


def stored_keys(k: np.ndarray, slots, bf16: bool, theta: float = DEFAULT_THETA) -> np.ndarray:
    """Stored form of keys k [..., D] (storage-precision values) written to
    ring slots ``slots``: an int, or an integer array over k's leading axes
    (e.g. [n] for k [n, Hkv, D]); returns float32 arrays holding the stored
    values."""
    k = np.asarray(k, dtype=np.float32)
    t = np.asarray(slots, dtype=np.int64) % TILE
    t = np.broadcast_to(t.reshape(t.shape + (1,) * (k.ndim - 1 - t.ndim)), k.shape[:-1])
    c, s = coef_f32(t, k.shape[-1], theta)
    return to_storage(rotate_f32(k, c, s), bf16)
