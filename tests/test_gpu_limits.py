"""GPU parity at the library's size limits: more streams in one call than one
launch carries (their state travels in the kernel arguments, 128 streams per
launch), and chunks longer than the 16 positions the split kernels take (those
run as one block per row group over the whole window, without key splits)."""

import numpy as np
import pytest

import synth
from gpu_util import Twin, say

pytestmark = pytest.mark.gpu


def draw(rng, shape, bf16=True):
    """N(0, 1) inputs, rounded to bf16 first when the cache is bf16 (both
    sides then see the same values)."""
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("portable", [False, True])
def test_more_streams_than_one_launch(portable):
    """130 streams in every call: a launch of 128 and one of 2.  Decode, chunk
    and the fused calls against the oracle, for every stream, from seeded
    ragged start states (some windows wrap, some are still filling)."""
    say("more_streams_than_one_launch", portable)
    nb, hq, hkv, d, w = 130, 4, 2, 64, 64
    rng = np.random.default_rng(130)
    tw = Twin(1, nb, hq, hkv, d, w, 4, True, portable)
    pos = rng.integers(0, 2**40, size=nb)
    slot = rng.integers(0, w, size=nb)
    tw.reset(0, pos.tolist(), slot.tolist())
    fill = rng.integers(1, 2 * w, size=nb)            # tokens before the first attention
    for t in range(int(fill.max())):
        live = [b for b in range(nb) if t < fill[b]]
        # appends in runs of consecutive streams (one call per run)
        runs, start = [], live[0]
        for a, b in zip(live, live[1:] + [None]):
            if b != a + 1:
                runs.append((start, a + 1))
                start = b
        for b0, b1 in runs:
            k = draw(rng, (b1 - b0, 1, hkv, d))
            v = draw(rng, (b1 - b0, 1, hkv, d))
            tw.append(0, b0, k, v)
    for step in range(3):
        q = draw(rng, (nb, hq, d))
        tw.decode(0, 0, q)
        k = draw(rng, (nb, 1, hkv, d))
        v = draw(rng, (nb, 1, hkv, d))
        tw.append_decode(0, 0, k, v, draw(rng, (nb, hq, d)))
        k = draw(rng, (nb, 4, hkv, d))
        v = draw(rng, (nb, 4, hkv, d))
        tw.append(0, 0, k, v)
        tw.chunk(0, 0, draw(rng, (nb, 4, hq, d)))
        k = draw(rng, (nb, 3, hkv, d))
        v = draw(rng, (nb, 3, hkv, d))
        tw.append_chunk(0, 0, k, v, draw(rng, (nb, 3, hq, d)))
    for b in (0, 1, 127, 128, 129):
        tw.check_state(0, b)
        tw.check_ring(0, b)
    say("worst", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("bf16", [True, False])
def test_chunks_longer_than_16(portable, bf16):
    """Chunks of 17, 20 and 32 positions (max_chunk 32) through fills and wraps,
    separate and fused, on a window of 96 slots."""
    say("chunks_longer_than_16", portable, bf16)
    hq, hkv, d, w = 8, 2, 64, 96
    rng = np.random.default_rng(17 + bf16)
    tw = Twin(1, 2, hq, hkv, d, w, 32, bf16, portable)
    tw.reset(0, [2**33 + 5, 3], [40, 0])
    for t, n in enumerate([20, 32, 17, 32, 20, 32, 17, 20, 32]):
        k = draw(rng, (2, n, hkv, d), bf16)
        v = draw(rng, (2, n, hkv, d), bf16)
        q = draw(rng, (2, n, hq, d), bf16)
        if t % 2:
            tw.append_chunk(0, 0, k, v, q)
        else:
            tw.append(0, 0, k, v)
            tw.chunk(0, 0, q)
    for b in range(2):
        tw.check_state(0, b)
        tw.check_ring(0, b)
    say("worst", tw.worst)
    tw.close()
