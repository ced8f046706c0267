"""Rebase-on-evict comparison variant: keys stored rotated, re-rotated at every eviction.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Sources:
* "Audio8 ASR Infinite: What It Actually Takes to Listen Forever", section
  "Inside the Rolling KV Cache and Exact RoPE Re-Basing" (the paragraph on why
  re-basing is harder than it sounds: a rounding artifact in recomputing the
  rotation of a token that has been re-based many times is never reported and
  accumulates) and section "Failure Modes That Only Appear on Day Three of a
  Session" (re-basing executed in low precision at every cache boundary lets a
  small error enter the rotation and never leave).
* "Audio8-ASR-Infinite-Compressed", the Linux CPU notes: that build re-bases a
  BF16 cache.

The pages name the hazard, not an algorithm.  The reading modelled here (and
run by the library under ``A8R_REBASE_ON_EVICT``): K is stored already rotated
to its re-based index, in the storage precision; when an append of n tokens to
a window of L0 evicts e = L0 + n - min(L0 + n, W) tokens, the origin moves by e
and every surviving key is re-rotated by R(-e); each new token is rotated by
R(r) at its own index r.  Every re-rotation is rounded back to storage, so the
stored key of a token that has lived through k evictions carries k roundings.

Arithmetic (this is what the comparison is about, so it is fixed exactly):
coefficients (cos, sin)(r * theta^(-2i/D)) computed in float64 and rounded once
to float32; per pair

    y1 = fl32(fl32(x1 * c) - fl32(x2 * s))
    y2 = fl32(fl32(x2 * c) + fl32(x1 * s))

(float32 multiplies and adds, no fused multiply-add), then rounded to the
storage type (bf16: round to nearest, ties to even).  numpy float32 operations
are IEEE single precision, so this emulation is bit for bit.

Attention in this variant uses the stored keys as they are and rotates the
query by its re-based index (float64 here).

Pinned by ``tests/test_oracle_rebase.py``: with float64 storage and arithmetic
the variant equals the method's re-based attention (and the brute force) to
1e-12, which fixes the bookkeeping, the rotation directions and the shift
amounts; a shift by e equals e shifts by 1 in exact arithmetic; the bf16
rounding matches a direct definition; and without any eviction every stored key
is the once-rounded rotation of its input.
"""

from __future__ import annotations

import numpy as np

from .attention import attend, default_scale
from .ledger import StreamLedger
from .rope import DEFAULT_THETA, inv_freq, rotate


def coef_f32(index, head_dim: int, theta: float = DEFAULT_THETA) -> tuple[np.ndarray, np.ndarray]:
    """(cos, sin) of index * theta^(-2i/D) in float64, rounded once to float32.

    ``index`` is an int or integer array; the result has shape index.shape + (D/2,).
    """
    idx = np.asarray(index, dtype=np.int64).astype(np.float64)
    ang = idx[..., None] * inv_freq(head_dim, theta)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    bf16 keeps the top 16 bits of the float32 encoding; rounding adds half of
    the dropped range (0x7FFF) plus the lowest kept bit, then truncates.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (keep.astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, bf16: bool) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if bf16 else x


def rotate_f32(x: np.ndarray, c: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Split-half rotation of the last axis in float32 without fusion."""
    x = np.asarray(x, dtype=np.float32)
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    y1 = (x1 * c) - (x2 * s)
    y2 = (x2 * c) + (x1 * s)
    return np.concatenate([y1, y2], axis=-1).astype(np.float32)


class RebaseStream:
    """One (layer, stream) ring in the rebase-on-evict variant.

    Stores, per slot, the key already rotated to its current re-based index and
    the value as appended, both as float32 arrays holding storage-precision
    values; the bookkeeping is ``StreamLedger``'s.
    """

    def __init__(self, window: int, n_kv_heads: int, head_dim: int, bf16: bool,
                 theta: float = DEFAULT_THETA, next_pos: int = 0, next_slot: int | None = None,
                 exact: bool = False):
        self.led = StreamLedger(window, next_pos, next_slot)
        self.w, self.hkv, self.d, self.bf16, self.theta = window, n_kv_heads, head_dim, bf16, theta
        self.exact = exact                 # float64 storage and arithmetic (pins the bookkeeping)
        dt = np.float64 if exact else np.float32
        self.k = np.zeros((window, n_kv_heads, head_dim), dtype=dt)
        self.v = np.zeros((window, n_kv_heads, head_dim), dtype=dt)

    def _rot(self, x: np.ndarray, index, conj: bool) -> np.ndarray:
        """x [..., D] by R(index) (R(-index) when conj)."""
        if self.exact:
            idx = np.asarray(index, dtype=np.int64)
            return rotate(x, -idx if conj else idx, self.theta)
        c, s = coef_f32(index, self.d, self.theta)
        return to_storage(rotate_f32(x, c, -s if conj else s), self.bf16)

    def append(self, k_new: np.ndarray, v_new: np.ndarray) -> tuple[list[int], list[int]]:
        """Append n tokens (k_new, v_new [n, Hkv, D], already in storage precision)."""
        k_new = np.asarray(k_new)
        n = k_new.shape[0]
        l0 = self.led.length
        slots, evicted = self.led.append(n)
        l1 = self.led.length
        e = l0 + n - l1
        if e > 0 and l1 > n:            # survivors: re-based indices drop by e
            surv = [self.led.slot_of_live(r) for r in range(l1 - n)]
            self.k[surv] = self._rot(self.k[surv], e, conj=True)
        for j, slot in enumerate(slots):
            r = l1 - n + j
            self.k[slot] = self._rot(k_new[j], r, conj=False)
            self.v[slot] = v_new[j]
        return slots, evicted

    def window(self) -> tuple[np.ndarray, np.ndarray]:
        """Stored keys (rotated) and values of the live window, oldest first."""
        order = [self.led.slot_of_live(r) for r in range(self.led.length)]
        return self.k[order].astype(np.float64), self.v[order].astype(np.float64)

    def attention(self, q: np.ndarray, scale: float | None = None) -> np.ndarray:
        """The C newest tokens' queries q [C, Hq, D] over the stored window, float64."""
        q = np.asarray(q, dtype=np.float64)
        c, _, d = q.shape
        kw, vw = self.window()
        n = kw.shape[0]
        if not 1 <= c <= n:
            raise ValueError("need 1 <= C <= L")
        scale = default_scale(d) if scale is None else scale
        r_k = np.arange(n)
        r_q = n - c + np.arange(c)
        qr = rotate(q, r_q[:, None], self.theta)
        visible = r_k[None, :] <= r_q[:, None]
        return attend(qr, kw, vw, scale, visible)
