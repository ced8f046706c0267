"""GPU parity on small shapes and edge cases, through the C ABI, both kernel
policies (AUTO = MFMA decode where it applies, PORTABLE = VALU kernels).

Covers: partial windows, several wraparounds, windows that are not a multiple
of the 32-slot tile (1, 7, 33, 100), GQA groups 1/2/8/16, head dims 64/128,
bf16 and float32, ring offsets unrelated to positions, chunks (causal inside a
chunk) including a chunk of the whole window, resets in mid-stream, streams at
different fill levels in one batched call, error returns that change nothing,
run-to-run bitwise determinism, and ring readback equal to the inputs.
"""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
from gpu_util import Twin, say, to_device, empty_out

pytestmark = pytest.mark.gpu


def rand(rng, *shape, bf16=True):
    import synth
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,hq,hkv,d,bf16", [
    (1, 8, 8, 64, True), (7, 16, 2, 128, True), (33, 16, 2, 128, True), (100, 8, 8, 64, True),
    (64, 8, 8, 64, False), (96, 4, 1, 128, True), (64, 16, 1, 64, True), (40, 6, 3, 128, False),
])
def test_decode_stream_wraps(window, hq, hkv, d, bf16, portable):
    say("decode_stream_wraps", window, hq, hkv, d, bf16, portable)
    rng = np.random.default_rng(window * 31 + hq)
    tw = Twin(2, 3, hq, hkv, d, window, 1, bf16, portable)
    p0 = [0, 1_000_003, 2**24 - 5]
    s0 = [0, rng.integers(window), rng.integers(window)]
    tw.reset(0, p0, s0)
    steps = 3 * window + 5
    check = set(range(0, steps, max(1, steps // 12))) | {window - 1, window, window + 1, steps - 1}
    for t in range(steps):
        for layer in range(2):
            k = rand(rng, 3, 1, hkv, d, bf16=bf16)
            v = rand(rng, 3, 1, hkv, d, bf16=bf16)
            tw.append(layer, 0, k, v)
            if t in check:
                q = rand(rng, 3, hq, d, bf16=bf16)
                tw.decode(layer, 0, q)
    for layer in range(2):
        for b in range(3):
            tw.check_state(layer, b)
            tw.check_ring(layer, b)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,hq,hkv,d,bf16", [
    (1, 8, 8, 64, True), (7, 16, 2, 128, True), (33, 16, 2, 128, True), (100, 8, 8, 64, True),
    (64, 8, 8, 64, False), (96, 4, 1, 128, True), (256, 16, 2, 128, True),
])
def test_fused_append_decode_wraps(window, hq, hkv, d, bf16, portable):
    """a8r_append_decode_attn equals append + decode, across fills and wraps,
    mixed with separate appends and decodes on the same cache."""
    say("fused_append_decode", window, hq, hkv, d, bf16, portable)
    rng = np.random.default_rng(window * 7 + hq)
    tw = Twin(2, 3, hq, hkv, d, window, 1, bf16, portable)
    tw.reset(0, [5, 2**24 - 3, 77_777], [0, rng.integers(window), rng.integers(window)])
    steps = 3 * window + 7
    for t in range(steps):
        layer = t % 2
        k = rand(rng, 3, 1, hkv, d, bf16=bf16)
        v = rand(rng, 3, 1, hkv, d, bf16=bf16)
        q = rand(rng, 3, hq, d, bf16=bf16)
        if t % 5 == 4:
            tw.append(layer, 0, k, v)
            tw.decode(layer, 0, q)
        else:
            tw.append_decode(layer, 0, k, v, q)
    for layer in range(2):
        for b in range(3):
            tw.check_state(layer, b)
            tw.check_ring(layer, b)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,chunk,hq,hkv,d,bf16,nb", [
    (64, 8, 16, 2, 128, True, 3), (37, 5, 8, 8, 64, True, 2), (45, 16, 16, 2, 128, True, 2),
    (50, 3, 4, 2, 64, False, 2),                          # float32: the two-launch path
    (64, 12, 32, 2, 128, True, 2),                        # 192 query rows: the two-launch path
    (2048, 8, 16, 2, 128, True, 2), (1000, 6, 8, 1, 64, True, 3),   # many key splits
])
def test_fused_append_chunk(window, chunk, hq, hkv, d, bf16, nb, portable):
    """a8r_append_chunk_attn equals append + chunk through fills and wraps (new
    tokens crossing tile and split boundaries, sizes 1 and odd), mixed with
    separate appends and chunks on the same cache."""
    say("fused_append_chunk", window, chunk, hq, hkv, d, bf16, nb, portable)
    rng = np.random.default_rng(window * 3 + chunk)
    tw = Twin(2, nb, hq, hkv, d, window, chunk, bf16, portable)
    tw.reset(0, [2**24 - 3 * window + i for i in range(nb)], [int(rng.integers(window)) for _ in range(nb)])
    steps = min(3 * window // chunk + 5, 40) if window > 512 else 3 * window // chunk + 5
    for t in range(steps):
        layer = t % 2
        n = chunk if t % 4 else (1 if t % 8 == 0 else max(2, chunk - 3))
        k = rand(rng, nb, n, hkv, d, bf16=bf16)
        v = rand(rng, nb, n, hkv, d, bf16=bf16)
        q = rand(rng, nb, n, hq, d, bf16=bf16)
        if t % 7 == 6:
            tw.append(layer, 0, k, v)
            tw.chunk(layer, 0, q)
        else:
            tw.append_chunk(layer, 0, k, v, q)
    for layer in range(2):
        for b in range(nb):
            tw.check_state(layer, b)
            tw.check_ring(layer, b)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,chunk,hq,hkv,d,bf16", [
    (64, 8, 16, 2, 128, True), (37, 5, 8, 8, 64, True), (16, 16, 16, 2, 128, True),
    (50, 3, 4, 2, 64, False), (128, 8, 16, 2, 128, True),
    (64, 16, 32, 2, 128, True), (40, 12, 16, 1, 64, True),     # 256 and 192 query rows per KV head
    (512, 8, 16, 2, 128, True), (1000, 16, 32, 2, 64, True),   # several key splits (merged in the kernel)
])
def test_chunk_stream(window, chunk, hq, hkv, d, bf16, portable):
    say("chunk_stream", window, chunk, hq, hkv, d, bf16, portable)
    rng = np.random.default_rng(window + chunk)
    tw = Twin(1, 2, hq, hkv, d, window, chunk, bf16, portable)
    tw.reset(0, [2**24 - 3 * window, 77], [5 % window, 0])
    for t in range(4 * window // chunk + 3):
        n = chunk if t % 3 else max(1, chunk // 2)
        k = rand(rng, 2, n, hkv, d, bf16=bf16)
        v = rand(rng, 2, n, hkv, d, bf16=bf16)
        tw.append(0, 0, k, v)
        q = rand(rng, 2, n, hq, d, bf16=bf16)
        tw.chunk(0, 0, q)
    tw.check_state(0, 1)
    tw.check_ring(0, 0)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
def test_ragged_streams_and_reset_midstream(portable):
    say("ragged_streams_and_reset", portable)
    rng = np.random.default_rng(3)
    hq, hkv, d, w = 16, 2, 128, 96
    tw = Twin(2, 5, hq, hkv, d, w, 4, True, portable)
    # streams filled to different levels
    for b in range(5):
        for _ in range(b * 30 + 1):
            tw.append(0, b, rand(rng, 1, 1, hkv, d), rand(rng, 1, 1, hkv, d))
    tw.decode(0, 0, rand(rng, 5, hq, d))
    # reset streams 1..2 in the middle, refill a little, batched decode again
    tw.reset(1, [10**9, 5], [17, 3])
    for layer in range(2):
        tw.append(layer, 1, rand(rng, 2, 3, hkv, d), rand(rng, 2, 3, hkv, d))
    tw.decode(0, 0, rand(rng, 5, hq, d))
    tw.chunk(0, 1, rand(rng, 2, 3, hq, d))
    tw.decode(1, 1, rand(rng, 2, hq, d))
    # fused calls over the ragged batch: an empty window filling up (layer 1,
    # streams 0, 3, 4), partly filled and full windows in one launch
    for t in range(4):
        n = 4 if t % 2 else 1
        k, v = rand(rng, 5, n, hkv, d), rand(rng, 5, n, hkv, d)
        if n == 1:
            tw.append_decode(1, 0, k, v, rand(rng, 5, hq, d))
            tw.append_decode(0, 0, k, v, rand(rng, 5, hq, d))
        else:
            tw.append_chunk(1, 0, k, v, rand(rng, 5, n, hq, d))
            tw.append_chunk(0, 0, k, v, rand(rng, 5, n, hq, d))
    for b in range(5):
        tw.check_state(0, b)
        tw.check_state(1, b)
        tw.check_ring(0, b)
    tw.close()


def test_errors_leave_state_unchanged():
    say("errors_leave_state_unchanged")
    rng = np.random.default_rng(4)
    tw = Twin(2, 2, 16, 2, 128, 64, 8, True)
    c = tw.gpu
    q = to_device(rand(rng, 2, 16, 128), True)
    out = empty_out((2, 16, 128), True)
    with pytest.raises(a8r.A8RError) as e:
        c.decode_attn(0, 0, 2, q, out)               # empty window
    assert e.value.status == a8r.A8R_ESTATE
    tw.append(0, 0, rand(rng, 2, 3, 2, 128), rand(rng, 2, 3, 2, 128))
    before = [c.get_state(l, b) for l in range(2) for b in range(2)]
    k = to_device(rand(rng, 2, 9, 2, 128), True)
    bad = [
        (lambda: c.append_kv(0, 0, 2, 9, k, k), a8r.A8R_EINVAL),          # n_new > max_chunk
        (lambda: c.append_kv(2, 0, 1, 1, k, k), a8r.A8R_EINVAL),          # layer out of range
        (lambda: c.append_kv(0, 1, 2, 1, k, k), a8r.A8R_EINVAL),          # streams out of range
        (lambda: c.append_kv(0, 0, 1, 1, k.data_ptr() + 2, k), a8r.A8R_EINVAL),  # misaligned
        (lambda: c.chunk_attn(0, 0, 2, 4, q, out), a8r.A8R_ESTATE),       # n_new > L
        (lambda: c.decode_attn(1, 0, 1, q, out), a8r.A8R_ESTATE),         # layer 1 still empty
        (lambda: c.decode_attn(0, 0, 2, 0, out), a8r.A8R_EINVAL),         # null q
        (lambda: c.reset(0, [-5]), a8r.A8R_EINVAL),
        (lambda: c.reset(1, [5], [64]), a8r.A8R_EINVAL),
        (lambda: c.append_chunk_attn(0, 0, 2, 9, k, k, q, out), a8r.A8R_EINVAL),      # n_new > max_chunk
        (lambda: c.append_chunk_attn(0, 1, 2, 4, k, k, q, out), a8r.A8R_EINVAL),      # streams out of range
        (lambda: c.append_chunk_attn(0, 0, 2, 4, k, k, 0, out), a8r.A8R_EINVAL),      # null q
        (lambda: c.append_chunk_attn(0, 0, 2, 4, k.data_ptr() + 2, k, q, out), a8r.A8R_EINVAL),
        (lambda: c.append_decode_attn(0, 0, 2, k, k, q.data_ptr() + 2, out), a8r.A8R_EINVAL),
    ]
    for call, status in bad:
        with pytest.raises(a8r.A8RError) as e:
            call()
        assert e.value.status == status
    assert [c.get_state(l, b) for l in range(2) for b in range(2)] == before
    tw.decode(0, 0, rand(rng, 2, 16, 128))
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("streams,window", [(4, 512), (64, 256)])
def test_bitwise_deterministic(portable, streams, window):
    """Repeated calls give identical bits: 4 streams take the multi-split merge
    (the exchange tree over several levels), 64 streams the two-split exchange."""
    say("bitwise_deterministic", portable, streams, window)
    rng = np.random.default_rng(5)
    tw = Twin(1, streams, 16, 2, 128, window, 8, True, portable)
    tw.reset(0, [(b * 7919 + b * b * 2**20) % 2**30 for b in range(streams)],
             [(b * 97 + 7) % window for b in range(streams)])
    k = to_device(rand(rng, streams, 8, 2, 128), True)
    v = to_device(rand(rng, streams, 8, 2, 128), True)
    for _ in range(window // 8 + 30):
        tw.gpu.append_kv(0, 0, streams, 8, k, v, want_bookkeeping=False)
    q = to_device(rand(rng, streams, 16, 128), True)
    outs = [empty_out((streams, 16, 128), True) for _ in range(3)]
    for o in outs:
        tw.gpu.decode_attn(0, 0, streams, q, o)
    assert bool((outs[0] == outs[1]).all()) and bool((outs[0] == outs[2]).all())
    tw.close()


@pytest.mark.parametrize("window", [400, 700, 950, 1600, 2100])
def test_decode_merge_tree_split_counts(window):
    """One stream (two KV heads): the window is split 2, 4, 4, 8 and 16 ways (a
    quarter of its 32-slot tiles rounded down to a power of two, up to 16):
    merge trees of 1 to 4 levels; parity through fills and a wrap, and
    identical bits on repeated calls."""
    say("decode_merge_tree", window)
    rng = np.random.default_rng(window)
    tw = Twin(1, 1, 16, 2, 128, window, 1, True)
    tw.reset(0, [2**24 - window // 2], [window // 3])
    for t in range(window + 40):
        k, v = rand(rng, 1, 1, 2, 128), rand(rng, 1, 1, 2, 128)
        if t % 97 == 0 or t >= window + 37:
            tw.append_decode(0, 0, k, v, rand(rng, 1, 16, 128))
        else:
            tw.append(0, 0, k, v)
    q = to_device(rand(rng, 1, 16, 128), True)
    outs = [empty_out((1, 16, 128), True) for _ in range(3)]
    for o in outs:
        tw.gpu.decode_attn(0, 0, 1, q, o)
    assert bool((outs[0] == outs[1]).all()) and bool((outs[0] == outs[2]).all())
    say("worst err", tw.worst)
    tw.close()


def test_translation_invariance_within_tolerance():
    """Identical logical windows stored at different ring offsets and absolute
    positions give the same attention (to rounding)."""
    say("translation_invariance")
    rng = np.random.default_rng(6)
    hq, hkv, d, w = 16, 2, 128, 256
    tw = Twin(1, 3, hq, hkv, d, w, 1, True)
    tw.reset(0, [0, 5_000_000, 2**24 + 3], [0, 201, 77])
    ks = rand(rng, w + 40, 1, hkv, d)
    vs = rand(rng, w + 40, 1, hkv, d)
    for t in range(w + 40):
        k = np.repeat(ks[t][None], 3, axis=0)
        v = np.repeat(vs[t][None], 3, axis=0)
        tw.append(0, 0, k, v)
    q = np.repeat(rand(rng, 1, hq, d), 3, axis=0)
    out = tw.decode(0, 0, q)
    assert np.max(np.abs(out[0] - out[1])) < 4e-3
    assert np.max(np.abs(out[0] - out[2])) < 4e-3
    tw.close()


def test_policies_agree():
    say("policies_agree")
    rng = np.random.default_rng(7)
    args = (1, 2, 16, 2, 128, 300, 1, True)
    a, b = Twin(*args, portable=False), Twin(*args, portable=True)
    for tw in (a, b):
        tw.reset(0, [9, 99999], [3, 250])
    for _ in range(333):
        k, v = rand(rng, 2, 1, 2, 128), rand(rng, 2, 1, 2, 128)
        a.append(0, 0, k, v)
        b.append(0, 0, k, v)
    q = rand(rng, 2, 16, 128)
    oa, ob = a.decode(0, 0, q), b.decode(0, 0, q)
    assert np.max(np.abs(oa - ob)) < 2e-2
    a.close()
    b.close()


@pytest.mark.parametrize("window,hq,hkv,d", [
    (2048, 16, 2, 128), (4096, 32, 2, 128), (1024, 8, 1, 64), (4096, 8, 4, 128),
])
def test_decode_writes_only_its_rows(window, hq, hkv, d):
    """Decode and fused append + decode with eight key splits (three levels of
    the merge tree) write their output rows and nothing past them: the output
    is a view at the start of a larger buffer whose tail holds a sentinel, and
    the rows match the oracle.  Groups of 8 and 16 query heads per KV head
    give each thread of the merge a partial and a full share of elements."""
    say("decode_writes_only_its_rows", window, hq, hkv, d)
    from gpu_util import torch, to_host_f64
    t = torch()
    rng = np.random.default_rng(window + 7 * hq + d)
    nb = 2
    tw = Twin(1, nb, hq, hkv, d, window, 256, True, False)
    tw.reset(0, [3 * window + 11, 2**24 + 5], [int(rng.integers(window)), int(rng.integers(window))])
    for n in [256] * (window // 256 - 1) + [255]:          # window - 1 tokens
        tw.append(0, 0, rand(rng, nb, n, hkv, d), rand(rng, nb, n, hkv, d))
    sentinel = 0x7f7f                                       # bf16 bits of a huge finite value
    for step in range(3):
        q = rand(rng, nb, hq, d)
        big = t.full((nb + 3, hq, d), sentinel, dtype=t.int16, device="cuda")
        if step == 1:
            k, v = rand(rng, nb, 1, hkv, d), rand(rng, nb, 1, hkv, d)
            tw.gpu.append_decode_attn(0, 0, nb, to_device(k, True), to_device(v, True), to_device(q, True),
                                      big[:nb])
            tw.ora.append(0, 0, k, v)
        else:
            tw.gpu.decode_attn(0, 0, nb, to_device(q, True), big[:nb])
        tail = big[nb:].cpu().numpy()
        assert np.all(tail == sentinel), ("output written past its rows", step, int(np.sum(tail != sentinel)))
        tw._cmp(to_host_f64(big[:nb], True), tw.ora.decode(0, 0, q), ("decode", step))
    # one stream of the two: the other stream's rows stay untouched too
    q = rand(rng, 1, hq, d)
    big = t.full((4, hq, d), sentinel, dtype=t.int16, device="cuda")
    tw.gpu.decode_attn(0, 1, 1, to_device(q, True), big[:1])
    assert np.all(big[1:].cpu().numpy() == sentinel)
    tw._cmp(to_host_f64(big[:1], True), tw.ora.decode(0, 1, q), ("decode", "stream 1"))
    say("worst err", tw.worst)
    tw.close()
