"""Ring bookkeeping model: which slot each new token takes, which position leaves.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Source: "Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
flowchart figure (nodes "Rolling KV cache, fixed capacity", "Token falls inside
the window?", "Evict oldest pair") and section "Inside the Rolling KV Cache and
Exact RoPE Re-Basing", second paragraph: the cache has a fixed capacity, and
once it is full every arriving key/value pair pushes out the oldest one, so the
store never grows.

Reading taken where the pages are silent (listed in the design notes):
* capacity W counts tokens; eviction is per token, oldest first (FIFO);
* the store is a ring of W slots; a stream's state is (P, L, S): the absolute
  position of its next token, the number of live tokens (<= W) and the slot the
  next token will occupy.  With S = P mod W at reset this is slot = pos mod W;
* a reset empties the window (L = 0) and sets P and S; slot contents are left
  as they are and are never read while they are not live.

Pinned by ``tests/test_oracle_ledger.py`` against an independent deque
simulation and against closed forms.
"""

from __future__ import annotations


class StreamLedger:
    """State of one (layer, stream) ring: P, L, S over a window of W slots."""

    __slots__ = ("window", "next_pos", "length", "next_slot")

    def __init__(self, window: int, next_pos: int = 0, next_slot: int | None = None):
        if window < 1:
            raise ValueError("window must be >= 1")
        self.window = int(window)
        self.reset(next_pos, next_slot)

    def reset(self, next_pos: int, next_slot: int | None = None) -> None:
        """Empty the window; the next token gets position next_pos, slot next_slot."""
        if next_pos < 0:
            raise ValueError("next_pos must be >= 0")
        if next_slot is None:
            next_slot = next_pos % self.window
        if not 0 <= next_slot < self.window:
            raise ValueError("next_slot out of range")
        self.next_pos = int(next_pos)
        self.length = 0
        self.next_slot = int(next_slot)

    def append(self, n_new: int) -> tuple[list[int], list[int]]:
        """Admit n_new tokens one after another, oldest-first eviction.

        Returns (slots, evicted): the slot each new token was written to and the
        absolute position that left the window to make room for it (-1 when the
        window still had room).
        """
        if n_new < 0:
            raise ValueError("n_new must be >= 0")
        slots, evicted = [], []
        for j in range(n_new):
            pos = self.next_pos + j
            slots.append(self.next_slot)
            if self.length == self.window:
                # the window is full: its oldest live token (position pos - W)
                # is the pair that leaves.
                evicted.append(pos - self.window)
            else:
                evicted.append(-1)
            self.next_slot = (self.next_slot + 1) % self.window
            self.length = min(self.length + 1, self.window)
        self.next_pos += n_new
        return slots, evicted

    # -- derived quantities ------------------------------------------------
    @property
    def origin(self) -> int:
        """Absolute position of the oldest live token: the window's zero."""
        return self.next_pos - self.length

    @property
    def oldest_slot(self) -> int:
        return (self.next_slot - self.length) % self.window

    def live_positions(self) -> list[int]:
        """Absolute positions of the live tokens, oldest first."""
        return list(range(self.origin, self.next_pos))

    def slot_of_live(self, k: int) -> int:
        """Slot of the k-th oldest live token (k = its re-based index)."""
        if not 0 <= k < self.length:
            raise IndexError(k)
        return (self.oldest_slot + k) % self.window

    def state(self) -> tuple[int, int, int]:
        return self.next_pos, self.length, self.next_slot


class CacheLedger:
    """Ledgers of every (layer, stream) pair of a cache."""

    def __init__(self, n_layers: int, n_streams: int, window: int):
        self.n_layers, self.n_streams, self.window = n_layers, n_streams, window
        self.rows = [[StreamLedger(window) for _ in range(n_streams)] for _ in range(n_layers)]

    def reset(self, b0: int, next_pos, next_slot=None) -> None:
        """Reset streams b0.. for every layer (a reset applies to the whole stack)."""
        for i, p in enumerate(next_pos):
            s = None if next_slot is None else next_slot[i]
            for layer in range(self.n_layers):
                self.rows[layer][b0 + i].reset(p, s)

    def append(self, layer: int, b0: int, nb: int, n_new: int):
        slots, evicted = [], []
        for b in range(b0, b0 + nb):
            s, e = self.rows[layer][b].append(n_new)
            slots.append(s)
            evicted.append(e)
        return slots, evicted

    def __getitem__(self, key):
        layer, b = key
        return self.rows[layer][b]
