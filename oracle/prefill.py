"""Window re-prefill: a window's keys and values re-derived from stored hidden
states, float64.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Source: "audio8-asr-infinite-p150", section "Limitations": that port keeps its
decoder's rolling context by re-prefilling the window - recomputing the cache
of the retained tokens - instead of trimming the cache as upstream does.  Here
only the part of a re-prefill that produces a layer's cache is modelled: the
key and value projections of the window's stored hidden states (the pages
give no projection details; the plainest reading of a decoder's K/V
projection is a bias-free linear map, K = H Wk^T and V = H Wv^T, with the
weights in a linear layer's [out_features][in_features] layout and output
feature kh * D + d being element d of KV head kh).  The rebuilt tokens become
the window: the last n positions, in order, oldest first.

Pinned by ``tests/test_oracle_prefill.py``: a hand-derived two-token fixture
(tests/golden/prefill_hand.json), identity weights giving the hidden states
back, linearity, and a rebuilt window attending exactly as the same tokens
appended one by one; a transposed weight must fail the fixture.
"""

from __future__ import annotations

import numpy as np


def project(hidden: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """hidden [n, H] times weight [F, H] transposed: [n, F], float64."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("hidden [n, H] and weight [F, H] expected")
    return h @ w.T


def rebuild_kv(hidden: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, n_kv_heads: int, head_dim: int):
    """Keys and values [n, Hkv, D] of a window re-derived from hidden [n, H]."""
    n = np.asarray(hidden).shape[0]
    k = project(hidden, w_k).reshape(n, n_kv_heads, head_dim)
    v = project(hidden, w_v).reshape(n, n_kv_heads, head_dim)
    return k, v
