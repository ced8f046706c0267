"""A whole rolling cache (layers x streams), float64, built from ledger + attention.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

It mirrors the library's five operations - create, reset, append, decode and
chunk attention - with the plainest possible data structures: per touched
(layer, stream) pair a physical ring of W slots holding float64 copies of the
appended K/V rows (un-rotated, never modified after being written), and the
``StreamLedger`` that says which slot each token takes.  Decode and chunk
attention gather the live window oldest-first from the ring and call the
re-based attention of ``attention.py``.

Source: "Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
flowchart figure and section "Inside the Rolling KV Cache and Exact RoPE
Re-Basing" (fixed capacity, oldest-first eviction, re-based indices), plus the
reset after a completed utterance shown by the flowchart's node "Emit final
segment, reset utterance state".  The reset applies to every layer of a stream.

A pinned prompt prefix (the pages mention an audio-independent prompt prefix
prepared once and re-checked at every silence reset, "Audio8-ASR-Infinite-
Compressed", Linux CPU notes; they do not say how it meets re-basing) is kept
per pair outside the ring and never evicted.  Reading: attention runs over the
sequence [prefix; live window] with consecutive re-based indices, i.e. exactly
the method's re-based attention over that concatenation.  A reset leaves the
prefix in place; ``clear_prefix`` empties it.

Pairs are materialised lazily, so a test can follow a few (layer, stream) pairs
of a very large configuration.
"""

from __future__ import annotations

import numpy as np

from .attention import chunk_rebased
from .ledger import StreamLedger
from .rope import DEFAULT_THETA


class OracleCache:
    def __init__(self, n_layers: int, n_streams: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, window: int, theta: float = DEFAULT_THETA,
                 scale: float | None = None):
        if n_q_heads % n_kv_heads:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        self.n_layers, self.n_streams = n_layers, n_streams
        self.hq, self.hkv, self.d, self.window = n_q_heads, n_kv_heads, head_dim, window
        self.theta, self.scale = theta, scale
        self._start = [(0, 0) for _ in range(n_streams)]      # (next_pos, next_slot) at reset
        self._pairs: dict[tuple[int, int], tuple[StreamLedger, np.ndarray, np.ndarray]] = {}
        self._prefix: dict[tuple[int, int], tuple[np.ndarray, np.ndarray]] = {}

    # -- storage -----------------------------------------------------------
    def _pair(self, layer: int, b: int):
        key = (layer, b)
        if key not in self._pairs:
            p, s = self._start[b]
            led = StreamLedger(self.window, p, s)
            ring_k = np.zeros((self.window, self.hkv, self.d), dtype=np.float64)
            ring_v = np.zeros((self.window, self.hkv, self.d), dtype=np.float64)
            self._pairs[key] = (led, ring_k, ring_v)
        return self._pairs[key]

    def ledger(self, layer: int, b: int) -> StreamLedger:
        return self._pair(layer, b)[0]

    # -- operations ----------------------------------------------------------
    def reset(self, b0: int, next_pos, next_slot=None) -> None:
        for i, p in enumerate(next_pos):
            b = b0 + i
            s = int(p) % self.window if next_slot is None else int(next_slot[i])
            self._start[b] = (int(p), s)
            for layer in range(self.n_layers):
                if (layer, b) in self._pairs:
                    self._pairs[(layer, b)][0].reset(int(p), s)

    def append(self, layer: int, b0: int, k: np.ndarray, v: np.ndarray):
        """k, v [nb, n_new, Hkv, D]; returns (slots [nb][n_new], evicted [nb][n_new])."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        nb, n_new = k.shape[:2]
        slots, evicted = [], []
        for i in range(nb):
            led, ring_k, ring_v = self._pair(layer, b0 + i)
            s, e = led.append(n_new)
            for j, slot in enumerate(s):
                ring_k[slot] = k[i, j]
                ring_v[slot] = v[i, j]
            slots.append(s)
            evicted.append(e)
        return slots, evicted

    def rebuild(self, layer: int, b0: int, k: np.ndarray, v: np.ndarray) -> None:
        """Window re-prefill: k, v [nb, n, Hkv, D] (oldest first) become each
        stream's window, the last n positions (P unchanged), token j in slot j,
        the next token in slot n mod W ("audio8-asr-infinite-p150", section
        "Limitations"; see prefill.py).  The pinned prefix is kept."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        nb, n = k.shape[:2]
        if not 1 <= n <= self.window:
            raise ValueError("n out of [1, W]")
        for i in range(nb):
            led, ring_k, ring_v = self._pair(layer, b0 + i)
            if led.next_pos < n:
                raise ValueError("the window would start before position 0")
            ring_k[:n] = k[i]
            ring_v[:n] = v[i]
            led.length = n
            led.next_slot = n % self.window

    def append_prefix(self, layer: int, b0: int, k: np.ndarray, v: np.ndarray) -> None:
        """Pin k, v [nb, n_new, Hkv, D] after each stream's prefix (its window must be empty)."""
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        for i in range(k.shape[0]):
            if self._pair(layer, b0 + i)[0].length:
                raise RuntimeError("the prefix must precede the window")
            pk, pv = self.prefix_kv(layer, b0 + i)
            self._prefix[(layer, b0 + i)] = (np.concatenate([pk, k[i]]), np.concatenate([pv, v[i]]))

    def clear_prefix(self, b0: int, nb: int) -> None:
        for key in [key for key in self._prefix if b0 <= key[1] < b0 + nb]:
            del self._prefix[key]

    def prefix_kv(self, layer: int, b: int):
        empty = np.zeros((0, self.hkv, self.d), dtype=np.float64)
        return self._prefix.get((layer, b), (empty, empty))

    def window_kv(self, layer: int, b: int):
        """Live keys and values oldest first, [L, Hkv, D] each, and the origin."""
        led, ring_k, ring_v = self._pair(layer, b)
        idx = [led.slot_of_live(j) for j in range(led.length)]
        return ring_k[idx], ring_v[idx], led.origin

    def chunk(self, layer: int, b0: int, q: np.ndarray) -> np.ndarray:
        """q [nb, C, Hq, D] for the C newest tokens; returns [nb, C, Hq, D]."""
        q = np.asarray(q, dtype=np.float64)
        out = np.empty_like(q)
        for i in range(q.shape[0]):
            kw, vw, _ = self.window_kv(layer, b0 + i)
            if kw.shape[0] == 0:
                raise RuntimeError("attention over an empty window")
            pk, pv = self.prefix_kv(layer, b0 + i)
            out[i] = chunk_rebased(q[i], np.concatenate([pk, kw]), np.concatenate([pv, vw]), self.theta,
                                   self.scale)
        return out

    def decode(self, layer: int, b0: int, q: np.ndarray) -> np.ndarray:
        """q [nb, Hq, D] for the newest token; returns [nb, Hq, D]."""
        return self.chunk(layer, b0, np.asarray(q)[:, None])[:, 0]
