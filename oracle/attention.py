"""Attention over the rolling window, float64: re-based form and brute force.

TEST INFRASTRUCTURE (see the package docstring): never used by the product path.

Source: "Audio8 ASR Infinite: What It Actually Takes to Listen Forever",
flowchart figure (nodes "Shift sliding origin forward, re-base all remaining
RoPE indices to new zero", "Relative distances between keys and queries
preserved exactly", "Attention over window") and section "Inside the Rolling KV
Cache and Exact RoPE Re-Basing", fourth paragraph: after an eviction the origin
moves forward and every surviving key's and the query's rotary index is measured
from the new origin; nothing is interpolated or rescaled.

Readings taken where the pages are silent (listed in the design notes):
* the origin is the absolute position of the oldest live token, so live keys
  carry indices 0 .. L-1 in age order and the query its own distance from the
  origin (decode: L - 1, it is the newest token);
* a query attends to its own key/value (append, then attend);
* several new positions per clock (a chunk) are all appended first; query c of
  a C-token chunk has index L - C + c and sees keys 0 .. L - C + c (causal
  inside the chunk, the whole older window before it);
* grouped-query attention maps query head h to key/value head h // (Hq / Hkv);
* scores are scaled by 1/sqrt(D) unless a scale is given.

``brute_force`` computes the same thing without any window bookkeeping: it takes
every token since the last reset with its absolute position, keeps the ones the
fixed capacity still holds, and rotates at absolute positions.  The re-based
result must equal it (in exact arithmetic they are the same number).

Pinned by ``tests/test_oracle_attention.py``.
"""

from __future__ import annotations

import math

import numpy as np

from .rope import DEFAULT_THETA, rotate


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend(q_rot: np.ndarray, k_rot: np.ndarray, v: np.ndarray, scale: float,
           visible: np.ndarray | None = None) -> np.ndarray:
    """softmax(scale * q k^T) v per query head, GQA head map h -> h // G.

    q_rot [Nq, Hq, D]; k_rot, v [Nk, Hkv, D]; visible [Nq, Nk] bool or None.
    Returns [Nq, Hq, D] float64.
    """
    nq, hq, d = q_rot.shape
    nk, hkv, _ = k_rot.shape
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    out = np.empty((nq, hq, d), dtype=np.float64)
    for h in range(hq):
        kh = h // g
        s = scale * (q_rot[:, h, :] @ k_rot[:, kh, :].T)          # [Nq, Nk]
        if visible is not None:
            s = np.where(visible, s, -np.inf)
        out[:, h, :] = _softmax_rows(s) @ v[:, kh, :]
    return out


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def chunk_rebased(q: np.ndarray, k_win: np.ndarray, v_win: np.ndarray,
                  theta: float = DEFAULT_THETA, scale: float | None = None) -> np.ndarray:
    """C new queries over a live window given oldest-first.

    q [C, Hq, D] are the queries of the C newest tokens (already in the window);
    k_win, v_win [L, Hkv, D] hold the L live tokens, oldest first, un-rotated.
    Key j carries re-based index j; query c carries L - C + c and sees keys
    0 .. L - C + c.
    """
    q = np.asarray(q, dtype=np.float64)
    k_win = np.asarray(k_win, dtype=np.float64)
    v_win = np.asarray(v_win, dtype=np.float64)
    c, _, d = q.shape
    n = k_win.shape[0]
    if not 1 <= c <= n:
        raise ValueError("need 1 <= C <= L")
    scale = default_scale(d) if scale is None else scale
    r_k = np.arange(n)
    r_q = n - c + np.arange(c)
    qr = rotate(q, r_q[:, None], theta)
    kr = rotate(k_win, r_k[:, None], theta)
    visible = r_k[None, :] <= r_q[:, None]
    return attend(qr, kr, v_win, scale, visible)


def decode_rebased(q: np.ndarray, k_win: np.ndarray, v_win: np.ndarray,
                   theta: float = DEFAULT_THETA, scale: float | None = None) -> np.ndarray:
    """One query (the newest token, index L - 1) over the window; q [Hq, D]."""
    return chunk_rebased(np.asarray(q)[None], k_win, v_win, theta, scale)[0]


def brute_force(q: np.ndarray, q_pos, hist_pos, hist_k, hist_v, next_pos: int,
                window: int, theta: float = DEFAULT_THETA,
                scale: float | None = None) -> np.ndarray:
    """Attention at absolute positions from the full history since the reset.

    q [Nq, Hq, D] at absolute positions q_pos [Nq]; hist_* hold every token
    appended since the last reset (positions hist_pos, any order), next_pos is
    the position the next token would take.  A fixed capacity of ``window``
    tokens keeps positions >= next_pos - window; a query sees kept keys at or
    before its own position.  Rotation uses the absolute positions themselves.
    """
    q = np.asarray(q, dtype=np.float64)
    hist_pos = np.asarray(hist_pos, dtype=np.int64)
    hist_k = np.asarray(hist_k, dtype=np.float64)
    hist_v = np.asarray(hist_v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    d = q.shape[-1]
    scale = default_scale(d) if scale is None else scale
    kept = hist_pos >= next_pos - window
    pos, k, v = hist_pos[kept], hist_k[kept], hist_v[kept]
    qr = rotate(q, q_pos[:, None], theta)
    kr = rotate(k, pos[:, None], theta)
    visible = pos[None, :] <= q_pos[:, None]
    return attend(qr, kr, v, scale, visible)
