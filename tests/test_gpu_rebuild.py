"""GPU parity of the window re-prefill (a8r_rebuild_window) through the C ABI.

The window of a batch of streams is rebuilt from stored hidden states with
seeded synthetic projection weights ("audio8-asr-infinite-p150", section
"Limitations": the rolling context rebuilt by re-prefilling instead of
trimming).  Checked against oracle/prefill.py:
* every rebuilt K and V element against the float64 projection of the same
  bf16 inputs, within the bound of a float32 accumulation of `hidden` products
  followed by one bf16 rounding: |gpu - exact| <= hidden * 2^-24 * sum|h w| +
  2^-8 |gpu| (the fraction equal to the exact value rounded to nearest even is
  reported);
* the state afterwards, (P, n, n mod W), bit for bit, on the host and device;
* decode and chunk attention over the rebuilt window, then appends and decode
  steps continuing from it (the appended tokens bit for bit in the ring), within
  the bf16 tolerance of the oracle's window (the exact projection rounded to
  bf16);
* full and ragged windows (n = W, n not a multiple of 8 or 256, n = 1), hidden
  sizes of one to eight 64-wide k steps, D = 128 and D = 64, several streams of
  one batch, a pinned prefix kept;
* errors that change nothing: n > W, a window before position 0, hidden sizes
  not a multiple of 64, float32 caches, the rebase-on-evict mode.
"""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
import synth
from gpu_util import Twin, say, to_device, empty_out
from oracle.prefill import rebuild_kv

pytestmark = pytest.mark.gpu


def rand_bf16(rng, *shape, scale=1.0):
    return synth.round_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def check_projection(got, exact, bound):
    """got: bf16 values (float64), exact: float64 projection, bound: per-element
    accumulation bound; returns the fraction equal to RNE(exact)."""
    err = np.abs(got - exact)
    lim = bound + np.abs(got) * 2.0**-8
    assert np.all(err <= lim), float(np.max(err - lim))
    rne = synth.round_bf16(exact.astype(np.float32)).astype(np.float64)   # exact -> float32 -> bf16
    return float(np.mean(got == rne))


@pytest.mark.parametrize("hq,hkv,d,w,hidden,n,nb,prefix", [
    (16, 2, 128, 512, 256, 512, 3, 0),
    (16, 2, 128, 512, 256, 300, 3, 0),
    (8, 2, 64, 256, 128, 131, 2, 0),
    (16, 2, 128, 384, 512, 200, 2, 20),
    (16, 2, 128, 256, 64, 1, 2, 0),                   # one token, one 64-wide k step
    (8, 2, 64, 1024, 192, 1000, 1, 0),                # four 256-token tiles, the last ragged; three k steps
])
def test_rebuild_matches_projection(hq, hkv, d, w, hidden, n, nb, prefix):
    say("rebuild", hq, hkv, d, w, hidden, n, nb, prefix)
    import torch
    rng = np.random.default_rng(w + n + hidden)
    tw = Twin(2, nb, hq, hkv, d, w, 8, True, prefix_capacity=prefix)
    tw.reset(0, [10_000 + 977 * b for b in range(nb)], [(41 * b) % w for b in range(nb)])
    if prefix:
        tw.append_prefix(1, 0, rand_bf16(rng, nb, prefix, hkv, d), rand_bf16(rng, nb, prefix, hkv, d))
    for _ in range(w // 8 + 3):                       # a full, wrapped window of other tokens
        tw.append(1, 0, rand_bf16(rng, nb, 8, hkv, d), rand_bf16(rng, nb, 8, hkv, d))
    h = rand_bf16(rng, nb, n, hidden)
    wk = rand_bf16(rng, hkv * d, hidden, scale=hidden ** -0.5)
    wv = rand_bf16(rng, hkv * d, hidden, scale=hidden ** -0.5)
    tw.gpu.rebuild_window(1, 0, nb, n, hidden, to_device(h, True), to_device(wk, True), to_device(wv, True))
    ks, vs = [], []
    frac = []
    for b in range(nb):
        k, v = rebuild_kv(h[b], wk, wv, hkv, d)
        bk = np.abs(h[b].astype(np.float64)) @ np.abs(wk.astype(np.float64)).T * hidden * 2.0**-24
        bv = np.abs(h[b].astype(np.float64)) @ np.abs(wv.astype(np.float64)).T * hidden * 2.0**-24
        rk, rv = tw.gpu.read_ring(1, b)
        gk = synth.bf16_to_f32(rk[:n]).astype(np.float64)
        gv = synth.bf16_to_f32(rv[:n]).astype(np.float64)
        frac.append(check_projection(gk, k, bk.reshape(n, hkv, d)))
        frac.append(check_projection(gv, v, bv.reshape(n, hkv, d)))
        ks.append(synth.round_bf16(k.astype(np.float32)))
        vs.append(synth.round_bf16(v.astype(np.float32)))
    say("fraction equal to the rounded exact projection", min(frac))
    tw.ora.rebuild(1, 0, np.stack(ks), np.stack(vs))
    for b in range(nb):
        tw.check_state(1, b)
        assert tw.gpu.get_state(1, b)[1:] == (n, n % w)
    tw.decode(1, 0, rand_bf16(rng, nb, hq, d))
    if n >= 8:
        tw.chunk(1, 0, rand_bf16(rng, nb, 8, hq, d))
    for _ in range(5):                                 # the stream goes on from the rebuilt window
        tw.append_decode(1, 0, rand_bf16(rng, nb, 1, hkv, d), rand_bf16(rng, nb, 1, hkv, d),
                         rand_bf16(rng, nb, hq, d))
    for b in range(nb):
        # the appended tokens bit for bit (the rebuilt ones were held to the
        # projection bound above: the oracle's window keeps the exact values
        # rounded once, which the float32 accumulation may miss by one ulp)
        rk, rv = tw.gpu.read_ring(1, b)
        _, ring_k, ring_v = tw.ora._pair(1, b)
        new = [(n + j) % w for j in range(5)]
        assert np.array_equal(synth.bf16_to_f32(rk[new]), ring_k[new].astype(np.float32))
        assert np.array_equal(synth.bf16_to_f32(rv[new]), ring_v[new].astype(np.float32))
        tw.check_state(1, b)
    tw.close()


def test_rebuild_errors_change_nothing():
    say("rebuild errors")
    rng = np.random.default_rng(9)
    hq, hkv, d, w, hidden = 16, 2, 128, 256, 128
    tw = Twin(1, 2, hq, hkv, d, w, 4, True)
    tw.reset(0, [100, 5000])
    for _ in range(30):
        tw.append(0, 0, rand_bf16(rng, 2, 4, hkv, d), rand_bf16(rng, 2, 4, hkv, d))
    before = [tw.gpu.get_state(0, b) for b in range(2)]
    h = to_device(rand_bf16(rng, 2, w + 1, hidden), True)
    wk = to_device(rand_bf16(rng, hkv * d, hidden), True)
    for n, hid in ((w + 1, hidden),        # more than the window
                   (0, hidden),            # an empty window
                   (16, 96)):              # hidden size not a multiple of 64
        with pytest.raises(a8r.A8RError) as e:
            tw.gpu.rebuild_window(0, 0, 2, n, hid, h, wk, wk)
        assert e.value.status == a8r.A8R_EINVAL
    # a window reaching before position 0: stream 0 is at position 220
    with pytest.raises(a8r.A8RError) as e:
        tw.gpu.rebuild_window(0, 0, 2, 221, hidden, h, wk, wk)
    assert e.value.status == a8r.A8R_EINVAL
    assert [tw.gpu.get_state(0, b) for b in range(2)] == before
    tw.decode(0, 0, rand_bf16(rng, 2, hq, d))
    tw.close()
    for kwargs, status in (({"bf16": False}, a8r.A8R_EUNSUPPORTED), ({"rebase_on_evict": True}, a8r.A8R_EUNSUPPORTED)):
        bf16 = kwargs.get("bf16", True)
        cfg = a8r.make_config(1, 1, hq, hkv, d, w, 4, bf16, rebase_on_evict=kwargs.get("rebase_on_evict", False))
        c = a8r.Cache(cfg)
        c.reset(0, [1000])
        hh = to_device(rand_bf16(rng, 1, 8, hidden), True)
        with pytest.raises(a8r.A8RError) as e:
            c.rebuild_window(0, 0, 1, 8, hidden, hh, wk, wk)
        assert e.value.status == status
        c.close()
