"""Translation invariance of the GPU attention, through the C ABI.

The method re-bases every index to the window's origin, so the attention of a
window depends only on its contents, never on the absolute positions nor on
where the ring holds it ("Audio8 ASR Infinite: What It Actually Takes to Listen
Forever", section "Inside the Rolling KV Cache and Exact RoPE Re-Basing":
relative distances are preserved exactly, so the attention geometry does not
change as the stream advances).

* Bitwise: the MFMA kernels walk the ring in physical 32-slot tiles, so a
  window stored at ring offsets that differ by a multiple of 32 is cut into the
  same tiles, visits and key splits, and every key and query meets the same
  table rows.  Such windows, at any absolute positions (0 .. 2^40), must give
  bit-identical outputs: decode, fused append + decode, chunk and fused append
  + chunk, with two and with eight key splits, full and partly filled windows.
  The portable kernel walks in re-based order and must be bitwise invariant
  under any offset.
* Any offset: the MFMA kernels' tiles then hold different keys, so operand
  roundings and summation orders differ; the outputs must stay within a
  stated bound of each other, in bf16 units in the last place.
"""

import numpy as np
import pytest

from gpu_util import Twin, say

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 2, 128
POSITIONS = [0, 5_000_000, 2**24 + 3, 2**40 + 17]
# bound on the distance between outputs of the same window at unrelated ring
# offsets (MFMA kernels), in bf16 units in the last place at the magnitude of
# the row's largest output (measured on MI355X: at most 1.375 over decode,
# fused decode, chunk and fused chunk at W = 256 and 1024); see
# test_any_offset_within_stated_ulps
MAX_ULPS_ANY_OFFSET = 2


def rand(rng, *shape):
    import synth
    return synth.round_bf16(rng.standard_normal(shape).astype(np.float32))


def row_ulps(a, b):
    """|a - b| per output row (the last axis) in units of the bf16 spacing at
    that row's largest magnitude in a: 2^(floor(log2 max|a|) - 7)."""
    scale = np.max(np.abs(a), axis=-1, keepdims=True)
    ulp = np.exp2(np.floor(np.log2(np.maximum(scale, 1e-30))) - 7)
    return np.max(np.abs(a - b) / ulp)


def run_window(offsets, positions, w, fill, mode, portable, seed):
    """Streams fed the same tokens from the given start offsets / positions;
    returns the outputs of the last call, [stream, ...]."""
    n = len(offsets)
    rng = np.random.default_rng(seed)
    c = 1 if "decode" in mode else 8
    tw = Twin(1, n, HQ, HKV, D, w, 8, True, portable)
    tw.reset(0, positions, offsets)
    steps = fill // c
    out = None
    for t in range(steps):
        k = np.repeat(rand(rng, 1, c, HKV, D), n, axis=0)
        v = np.repeat(rand(rng, 1, c, HKV, D), n, axis=0)
        last = t == steps - 1
        if not last:
            tw.append(0, 0, k, v)
            continue
        if c == 1:
            q = np.repeat(rand(rng, 1, HQ, D), n, axis=0)
            if mode == "fused_decode":
                out = tw.append_decode(0, 0, k, v, q)
            else:
                tw.append(0, 0, k, v)
                out = tw.decode(0, 0, q)
        else:
            q = np.repeat(rand(rng, 1, c, HQ, D), n, axis=0)
            if mode == "fused_chunk":
                out = tw.append_chunk(0, 0, k, v, q)
            else:
                tw.append(0, 0, k, v)
                out = tw.chunk(0, 0, q)
    for b in range(n):
        tw.check_ring(0, b)
    tw.close()
    return out


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("mode", ["decode", "fused_decode", "chunk", "fused_chunk"])
@pytest.mark.parametrize("w,fill", [(256, 296), (1024, 1064), (1024, 720)])
def test_bitwise_invariance_offsets_32m(portable, mode, w, fill):
    say("invariance_32m", portable, mode, w, fill)
    offsets = [0, 32, 96, w - 32]
    out = run_window(offsets, POSITIONS, w, fill, mode, portable, seed=w + fill)
    for b in range(1, len(offsets)):
        assert np.array_equal(out[b], out[0]), (mode, offsets[b], float(np.max(np.abs(out[b] - out[0]))))


@pytest.mark.parametrize("mode", ["decode", "chunk"])
def test_portable_bitwise_invariance_any_offset(mode):
    say("portable invariance any offset", mode)
    offsets = [0, 9, 201, 77]
    out = run_window(offsets, POSITIONS, 256, 296, mode, True, seed=11)
    for b in range(1, len(offsets)):
        assert np.array_equal(out[b], out[0]), (mode, offsets[b])


@pytest.mark.parametrize("mode", ["decode", "fused_decode", "chunk", "fused_chunk"])
@pytest.mark.parametrize("w,fill", [(256, 296), (1024, 1064)])
def test_any_offset_within_stated_ulps(mode, w, fill):
    """Unrelated ring offsets (0, 9, 13, 77, 201 mod 32: 0, 9, 13, 13, 9):
    the same window's outputs differ by at most MAX_ULPS_ANY_OFFSET bf16 units
    in the last place of each output row's largest element."""
    offsets = [0, 9, 13, 77, 201]
    out = run_window(offsets, POSITIONS + [123_456_789], w, fill, mode, False, seed=3 * w + fill)
    worst_ulps, worst_abs = 0.0, 0.0
    for b in range(1, len(offsets)):
        worst_ulps = max(worst_ulps, float(row_ulps(out[0], out[b])))
        worst_abs = max(worst_abs, float(np.max(np.abs(out[b] - out[0]))))
    say("any offset", mode, w, "max ulps", worst_ulps, "max abs", worst_abs)
    assert worst_ulps <= MAX_ULPS_ANY_OFFSET, (worst_ulps, worst_abs)
