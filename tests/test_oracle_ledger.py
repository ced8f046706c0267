"""Pins of the oracle's ring bookkeeping (CPU only).

The oracle ledger is checked against things it does not share code with:
* a hand-traced fixture (tests/golden/ledger_w3_hand.json);
* an independent simulation that keeps the live positions in a bounded deque
  (the plain meaning of "fixed capacity, the oldest pair leaves") and derives
  slots from the closed form slot(p) = (p + sigma) mod W, sigma = (S0 - P0) mod W;
* planted mistakes (evict the newest, forget to wrap) must fail those pins.
"""

import collections
import json
import os
import random

import pytest

from oracle.ledger import CacheLedger, StreamLedger

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def check_against_deque(ledger_cls, window, ops, p0=0, s0=None, full_every=1):
    """Run ``ops`` (('a', n) appends / ('r', pos, slot) resets) on ledger_cls and on
    a deque simulation; assert slots, evictions and state agree exactly.  The
    whole live set is compared after every ``full_every``-th append."""
    led = ledger_cls(window, p0, s0)
    live = collections.deque()
    pos = p0
    sigma = ((s0 if s0 is not None else p0 % window) - p0) % window
    for n_op, op in enumerate(ops):
        if op[0] == "r":
            _, pos, slot = op
            led.reset(pos, slot)
            live.clear()
            sigma = ((slot if slot is not None else pos % window) - pos) % window
            continue
        n = op[1]
        slots, evicted = led.append(n)
        exp_slots, exp_ev = [], []
        for _ in range(n):
            exp_slots.append((pos + sigma) % window)
            exp_ev.append(live.popleft() if len(live) == window else -1)
            live.append(pos)
            pos += 1
        assert slots == exp_slots
        assert evicted == exp_ev
        assert led.next_pos == pos
        assert led.length == len(live)
        assert led.oldest_slot == ((live[0] + sigma) % window if live else led.next_slot)
        if n_op % full_every == 0:
            assert led.live_positions() == list(live)
            for k in range(led.length):
                assert led.slot_of_live(k) == (live[k] + sigma) % window


def random_ops(rng, window, n_ops, max_chunk):
    ops = []
    for _ in range(n_ops):
        if rng.random() < 0.01:
            ops.append(("r", rng.randrange(0, 1 << 40), rng.choice([None, rng.randrange(window)])))
        else:
            ops.append(("a", rng.randint(0, max_chunk)))
    return ops


def test_hand_traced_fixture():
    with open(os.path.join(GOLDEN, "ledger_w3_hand.json")) as f:
        fx = json.load(f)
    led = StreamLedger(fx["window"])
    led.reset(fx["reset"]["next_pos"], fx["reset"]["next_slot"])
    for a in fx["appends"]:
        slots, evicted = led.append(a["n_new"])
        assert slots == a["slots"]
        assert evicted == a["evicted"]
    st = fx["final_state"]
    assert led.state() == (st["next_pos"], st["length"], st["next_slot"])
    assert led.live_positions() == fx["final_live_positions"]


@pytest.mark.parametrize("window", [1, 2, 3, 7, 64, 100, 1000])
def test_matches_deque_random(window):
    rng = random.Random(1234 + window)
    ops = random_ops(rng, window, 3000, max(1, min(window, 9)))
    check_against_deque(StreamLedger, window, ops, p0=rng.randrange(1 << 30), s0=rng.randrange(window))


def test_many_wraparounds_qwen_window():
    """100,000 single-token appends at W=4096 (about 24 wraps), as in the long stream."""
    check_against_deque(StreamLedger, 4096, [("a", 1)] * 100_000, full_every=4093)


def test_large_positions():
    w = 8192
    p0 = 2**62 - 3 * w
    check_against_deque(StreamLedger, w, [("a", 8)] * 3000, p0=p0, s0=5, full_every=511)


def test_cache_reset_applies_to_all_layers():
    c = CacheLedger(3, 2, 5)
    for layer in range(3):
        c.append(layer, 0, 2, 4)
    c.reset(1, [100], [2])
    for layer in range(3):
        assert c[layer, 1].state() == (100, 0, 2)
        assert c[layer, 0].state() == (4, 4, 4)


class EvictNewest(StreamLedger):
    """Planted mistake: when full, report the newest live position as evicted."""

    def append(self, n_new):
        slots, evicted = super().append(n_new)
        return slots, [(e + self.window - 1) if e >= 0 else e for e in evicted]


class NoWrap(StreamLedger):
    """Planted mistake: slots are not reduced mod W after the first pass."""

    def append(self, n_new):
        slots, evicted = [], []
        for j in range(n_new):
            slots.append(self.next_slot)
            evicted.append(self.next_pos + j - self.window if self.length == self.window else -1)
            self.next_slot = self.next_slot + 1 if self.next_slot + 1 < self.window else self.next_slot
            self.length = min(self.length + 1, self.window)
        self.next_pos += n_new
        return slots, evicted


@pytest.mark.parametrize("mutant", [EvictNewest, NoWrap])
def test_planted_mistakes_fail(mutant):
    with pytest.raises(AssertionError):
        check_against_deque(mutant, 7, [("a", 1)] * 40)
