"""CPU oracle for rolling-window decoder attention with exact RoPE re-basing.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code, table, constant generator or
pre/post-processing with the HIP library, and it never imports that library.

Everything here is plain numpy in float64 (integers as Python ints), written
from the pages' statement of the method:

* "Audio8 ASR Infinite: What It Actually Takes to Listen Forever" (blog),
  flowchart figure in "The Unbounded Stream Problem That Streaming ASR Never
  Really Solved" and section "Inside the Rolling KV Cache and Exact RoPE
  Re-Basing": a fixed-capacity cache that evicts its oldest key/value pair once
  full, and re-bases the rotary index of every surviving key and of the query
  to the window's new origin so query-key distances are unchanged.
* "Audio8-ASR-Infinite-mlx", section "Requires a patched mlx-audio-swift": the
  checkpoints use the split-half (rotate_half) rotary pairing, not the
  interleaved one.
* "Audio8-ASR-0.1B in audio.cpp", section "Architecture": RoPE theta 1e6.

Modules
-------
ledger     -- the ring bookkeeping model (slots, evicted positions, state).
rope       -- split-half rotary embedding at a given (re-based) index.
attention  -- re-based decode / chunk attention over the live window, and the
              brute-force attention at absolute positions it must equal.
model      -- a whole cache (layers x streams) built from the three above.
rebase     -- the rebase-on-evict comparison variant (keys stored rotated and
              re-rotated at every eviction, its float32/bf16 rounding emulated).
prefill    -- window re-prefill: a window's K/V re-derived from stored hidden
              states (the comparison with rebuilding instead of trimming).

Parity status of every function is pinned by tests under ``tests/`` marked
``not gpu``; none is "parity unpinned".
"""

from . import ledger, rope, attention, model, rebase, prefill  # noqa: F401
