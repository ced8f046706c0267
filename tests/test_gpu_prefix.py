"""GPU parity of the pinned prompt prefix, through the C ABI, both kernel
policies (AUTO = MFMA decode and chunk kernels, PORTABLE = VALU kernels).

Attention runs over [prefix; live window] with consecutive re-based indices
(the prefix at 0 .. F - 1, the window after it); the oracle (oracle/model.py)
is pinned to torch's float64 attention on that sequence and to a needle test
in tests/test_oracle_prefix.py.  Covered here:
* prefix lengths 1, 31, 32, 33, 100 (a partial tile, whole tiles, several
  tiles) with streams of one batch at different prefix lengths, including 0
  (the prefix kernel instance then walks streams without one);
* decode through fills and several wraparounds, fused append + decode, chunks
  of 2 .. 16 positions (several key splits at W = 512);
* a prefix built by several appends; reset keeps the prefix, clear_prefix
  removes it, a new prefix after a reset;
* export / import of a prepared prefix: the export equals the appended tokens
  bit for bit (K and V), and a second cache importing it gives bitwise the
  same attention;
* ring readback unchanged by the prefix (the prefix lives past the ring);
* errors: append to a non-empty window, beyond the capacity, a cache without
  prefix capacity, the rebase-on-evict mode.
"""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
import synth
from gpu_util import Twin, say, to_device, empty_out, current_stream

pytestmark = pytest.mark.gpu


def rand(rng, *shape, bf16=True):
    import synth
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,hq,hkv,d,bf16,prefixes", [
    (64, 16, 2, 128, True, [31, 0, 100]),
    (33, 8, 8, 64, True, [1, 32, 33]),
    (96, 16, 1, 128, True, [64, 5, 0]),
    (40, 6, 3, 128, False, [7, 0, 45]),
    (7, 16, 2, 128, True, [3, 40, 1]),
])
def test_prefix_decode_wraps(window, hq, hkv, d, bf16, prefixes, portable):
    say("prefix_decode_wraps", window, hq, hkv, d, bf16, prefixes, portable)
    rng = np.random.default_rng(window * 13 + sum(prefixes))
    tw = Twin(2, 3, hq, hkv, d, window, 1, bf16, portable, prefix_capacity=max(prefixes) + 8)
    tw.reset(0, [0, 1_000_003, 2**24 - 5], [0, int(rng.integers(window)), int(rng.integers(window))])
    for layer in range(2):
        for b, f in enumerate(prefixes):
            if f:
                # layer 1 gets its prefix in two appends
                cuts = [f] if layer == 0 or f == 1 else [f // 2, f - f // 2]
                for n in cuts:
                    tw.append_prefix(layer, b, rand(rng, 1, n, hkv, d, bf16=bf16), rand(rng, 1, n, hkv, d, bf16=bf16))
    steps = 3 * window + 5
    check = set(range(0, steps, max(1, steps // 10))) | {window - 1, window, window + 1, steps - 1}
    for t in range(steps):
        layer = t % 2
        k = rand(rng, 3, 1, hkv, d, bf16=bf16)
        v = rand(rng, 3, 1, hkv, d, bf16=bf16)
        q = rand(rng, 3, hq, d, bf16=bf16)
        if t % 3 == 0:
            tw.append_decode(layer, 0, k, v, q, check=t in check)
        else:
            tw.append(layer, 0, k, v)
            if t in check:
                tw.decode(layer, 0, q)
    for layer in range(2):
        for b in range(3):
            tw.check_state(layer, b)
            tw.check_ring(layer, b)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("window,chunk,hq,hkv,d,prefixes", [
    (64, 8, 16, 2, 128, [100, 31]),
    (37, 5, 8, 8, 64, [1, 0]),
    (512, 16, 16, 2, 128, [0, 250]),        # several key splits
    (40, 12, 16, 1, 64, [33, 64]),          # 192 query rows per KV head
])
def test_prefix_chunk(window, chunk, hq, hkv, d, prefixes, portable):
    say("prefix_chunk", window, chunk, hq, hkv, d, prefixes, portable)
    rng = np.random.default_rng(window + chunk + 1)
    tw = Twin(1, 2, hq, hkv, d, window, chunk, True, portable, prefix_capacity=max(prefixes))
    tw.reset(0, [2**24 - 3 * window, 77], [5 % window, 0])
    for b, f in enumerate(prefixes):
        if f:
            tw.append_prefix(0, b, rand(rng, 1, f, hkv, d), rand(rng, 1, f, hkv, d))
    for t in range(3 * window // chunk + 3):
        n = chunk if t % 3 else max(1, chunk // 2)
        k, v, q = rand(rng, 2, n, hkv, d), rand(rng, 2, n, hkv, d), rand(rng, 2, n, hq, d)
        if t % 2:                                   # one launch: append + attention
            tw.append_chunk(0, 0, k, v, q)
            continue
        tw.append(0, 0, k, v)
        if n == 1:
            tw.decode(0, 0, q[:, 0])
        else:
            tw.chunk(0, 0, q)
    tw.check_state(0, 1)
    tw.check_ring(0, 0)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("portable", [False, True])
def test_prefix_reset_clear_rebuild(portable):
    say("prefix_reset_clear_rebuild", portable)
    rng = np.random.default_rng(21)
    hq, hkv, d, w = 16, 2, 128, 96
    tw = Twin(1, 2, hq, hkv, d, w, 4, True, portable, prefix_capacity=80)
    tw.append_prefix(0, 0, rand(rng, 2, 50, hkv, d), rand(rng, 2, 50, hkv, d))

    def run(steps):
        for _ in range(steps):
            tw.append(0, 0, rand(rng, 2, 4, hkv, d), rand(rng, 2, 4, hkv, d))
        tw.decode(0, 0, rand(rng, 2, hq, d))
        tw.chunk(0, 0, rand(rng, 2, 4, hq, d))

    run(40)
    tw.reset(0, [123456, 2**24 + 7], [11, 95])       # the prefix stays
    assert tw.gpu.prefix_length(0, 0) == 50
    run(3)
    tw.reset(0, [0, 0], [0, 0])
    tw.append_prefix(0, 1, rand(rng, 1, 30, hkv, d), rand(rng, 1, 30, hkv, d))   # extended to 80
    run(30)
    tw.clear_prefix(0, 1)                              # stream 0 only
    assert tw.gpu.prefix_length(0, 0) == 0 and tw.gpu.prefix_length(0, 1) == 80
    run(5)
    tw.clear_prefix(1, 1)
    run(2)
    say("worst err", tw.worst)
    tw.close()


@pytest.mark.parametrize("bf16", [True, False])
def test_prefix_export_import(bf16):
    say("prefix_export_import", bf16)
    import torch
    rng = np.random.default_rng(25 + bf16)
    hq, hkv, d, w, f = 16, 2, 128, 80, 45
    cfgs = [a8r.make_config(2, 3, hq, hkv, d, w, 4, bf16, prefix_capacity=64) for _ in range(2)]
    a, b = (a8r.Cache(c, stream=current_stream()) for c in cfgs)
    pk, pv = rand(rng, 3, f, hkv, d, bf16=bf16), rand(rng, 3, f, hkv, d, bf16=bf16)
    kd, vd = to_device(pk, bf16), to_device(pv, bf16)
    a.append_prefix(1, 0, 3, f, kd, vd)
    ek, ev = torch.empty_like(kd), torch.empty_like(vd)
    a.export_prefix(1, 0, 3, f, ek, ev)
    got_k = synth.from_storage(ek.cpu().numpy().view(np.uint16) if bf16 else ek.cpu().numpy(), bf16)
    assert np.array_equal(got_k.view(np.uint32), pk.astype(np.float32).view(np.uint32))
    assert bool((ek == kd).all()) and bool((ev == vd).all())
    b.import_prefix(1, 0, 3, f, ek, ev)                  # import
    for c in (a, b):
        c.reset(0, [10, 2**24 - 7, 999], [3, 79, 40])
    outs = []
    for c in (a, b):
        r = np.random.default_rng(7)
        for _ in range(30):
            c.append_kv(1, 0, 3, 4, to_device(rand(r, 3, 4, hkv, d, bf16=bf16), bf16),
                        to_device(rand(r, 3, 4, hkv, d, bf16=bf16), bf16))
        o = empty_out((3, hq, d), bf16)
        c.decode_attn(1, 0, 3, to_device(rand(r, 3, hq, d, bf16=bf16), bf16), o)
        o2 = empty_out((3, 4, hq, d), bf16)
        c.chunk_attn(1, 0, 3, 4, to_device(rand(r, 3, 4, hq, d, bf16=bf16), bf16), o2)
        outs.append((o, o2))
    assert bool((outs[0][0] == outs[1][0]).all()) and bool((outs[0][1] == outs[1][1]).all())
    with pytest.raises(a8r.A8RError) as e:
        a.export_prefix(0, 0, 3, f, ek, ev)              # layer 0 has no prefix
    assert e.value.status == a8r.A8R_EINVAL
    with pytest.raises(a8r.A8RError) as e:
        a.export_prefix(1, 0, 3, f - 1, ek, ev)          # wrong length
    assert e.value.status == a8r.A8R_EINVAL
    a.close()
    b.close()


def test_prefix_errors():
    say("prefix_errors")
    rng = np.random.default_rng(22)
    tw = Twin(2, 2, 16, 2, 128, 64, 8, True, prefix_capacity=40)
    c = tw.gpu
    k = to_device(rand(rng, 2, 41, 2, 128), True)
    tw.append_prefix(0, 0, rand(rng, 2, 30, 2, 128), rand(rng, 2, 30, 2, 128))
    tw.append(0, 0, rand(rng, 2, 3, 2, 128), rand(rng, 2, 3, 2, 128))
    bad = [
        (lambda: c.append_prefix(0, 0, 1, 1, k, k), a8r.A8R_ESTATE),       # the window is not empty
        (lambda: c.append_prefix(1, 0, 1, 41, k, k), a8r.A8R_EINVAL),      # beyond the capacity
        (lambda: c.append_prefix(1, 0, 1, 0, k, k), a8r.A8R_EINVAL),       # n_new < 1
        (lambda: c.append_prefix(2, 0, 1, 1, k, k), a8r.A8R_EINVAL),       # layer out of range
        (lambda: c.append_prefix(1, 1, 2, 1, k, k), a8r.A8R_EINVAL),       # streams out of range
        (lambda: c.append_prefix(1, 0, 1, 1, k.data_ptr() + 2, k), a8r.A8R_EINVAL),   # misaligned
    ]
    for call, status in bad:
        with pytest.raises(a8r.A8RError) as e:
            call()
        assert e.value.status == status
    assert [c.prefix_length(l, b) for l in range(2) for b in range(2)] == [30, 30, 0, 0]
    tw.decode(0, 0, rand(rng, 2, 16, 128))
    tw.close()
    # no prefix capacity
    plain = a8r.Cache(a8r.make_config(1, 1, 16, 2, 128, 64, 1, True), stream=current_stream())
    with pytest.raises(a8r.A8RError) as e:
        plain.append_prefix(0, 0, 1, 1, k, k)
    assert e.value.status == a8r.A8R_EUNSUPPORTED
    plain.close()
    # the rebase-on-evict variant has no prefix
    with pytest.raises(a8r.A8RError) as e:
        a8r.Cache(a8r.make_config(1, 1, 16, 2, 128, 64, 1, True, rebase_on_evict=True, prefix_capacity=8),
                  stream=current_stream())
    assert e.value.status == a8r.A8R_EUNSUPPORTED


@pytest.mark.parametrize("portable", [False, True])
def test_prefix_bitwise_deterministic(portable):
    say("prefix_bitwise_deterministic", portable)
    rng = np.random.default_rng(23)
    streams, w = 8, 512
    tw = Twin(1, streams, 16, 2, 128, w, 8, True, portable, prefix_capacity=96)
    for b in range(streams):
        f = (b * 37) % 97
        if f:
            tw.gpu.append_prefix(0, b, 1, f, to_device(rand(rng, 1, f, 2, 128), True),
                                 to_device(rand(rng, 1, f, 2, 128), True))
    k = to_device(rand(rng, streams, 8, 2, 128), True)
    v = to_device(rand(rng, streams, 8, 2, 128), True)
    for _ in range(w // 8 + 30):
        tw.gpu.append_kv(0, 0, streams, 8, k, v, want_bookkeeping=False)
    q = to_device(rand(rng, streams, 16, 128), True)
    outs = [empty_out((streams, 16, 128), True) for _ in range(3)]
    for o in outs:
        tw.gpu.decode_attn(0, 0, streams, q, o)
    assert bool((outs[0] == outs[1]).all()) and bool((outs[0] == outs[2]).all())
    tw.close()


def test_prefix_3b_shape():
    """The 3B-class shape (16 / 2 heads, D = 128, W = 4096) with a 256-token
    prefix, 4 streams at different fills, decode and 16-position chunks."""
    say("prefix_3b_shape")
    rng = np.random.default_rng(24)
    hq, hkv, d, w = 16, 2, 128, 4096
    tw = Twin(1, 4, hq, hkv, d, w, 16, True, prefix_capacity=256)
    tw.reset(0, [0, 2**24 - 1000, 77, 5_000_000], [0, 4000, 1234, 17])
    tw.append_prefix(0, 0, rand(rng, 4, 256, hkv, d), rand(rng, 4, 256, hkv, d))
    for t in range(w // 16 + 40):
        tw.append(0, 0, rand(rng, 4, 16, hkv, d), rand(rng, 4, 16, hkv, d))
        if t in (3, w // 16 - 1, w // 16 + 39):
            tw.decode(0, 0, rand(rng, 4, hq, d))
            tw.chunk(0, 0, rand(rng, 4, 16, hq, d))
    say("worst err", tw.worst)
    tw.close()


def test_prefix_streaming_launch():
    """10 streams of the 3B-class shape (W = 4096): the launch's windows (42 MB)
    exceed the L2, so decode takes the instance with streaming K/V loads, here
    with a 64-token prefix; decode and fused decode against the oracle."""
    say("prefix_streaming_launch")
    rng = np.random.default_rng(26)
    hq, hkv, d, w, nb = 16, 2, 128, 4096, 10
    tw = Twin(1, nb, hq, hkv, d, w, 512, True, prefix_capacity=64)
    tw.reset(0, [1000 * b + 3 for b in range(nb)], [(b * 613) % w for b in range(nb)])
    tw.append_prefix(0, 0, rand(rng, nb, 64, hkv, d), rand(rng, nb, 64, hkv, d))
    for _ in range(8):
        tw.append(0, 0, rand(rng, nb, 512, hkv, d), rand(rng, nb, 512, hkv, d))
    tw.decode(0, 0, rand(rng, nb, hq, d))
    for _ in range(3):
        tw.append_decode(0, 0, rand(rng, nb, 1, hkv, d), rand(rng, nb, 1, hkv, d), rand(rng, nb, hq, d))
    say("worst err", tw.worst)
    tw.close()

