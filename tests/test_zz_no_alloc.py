"""a8r_chunk_attn_static, the chunk attention whose split partials live in the
library's static device array (for callers that cannot allocate), against
a8r_chunk_attn through the C ABI: bit-identical outputs on two calls in a row,
the second with a smaller input, on the MFMA chunk kernel and on the portable
kernel, and a call needing more than the array holds rejected with EINVAL
before any side effect.  The outputs are also held to the oracle's bf16 /
float32 tolerance."""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
from gpu_util import Twin, say, to_device, empty_out, to_host_f64

pytestmark = pytest.mark.gpu


def rand(rng, *shape, bf16=True):
    import synth
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("bf16,portable", [(True, False), (True, True), (False, True)])
def test_static_scratch_matches_chunk_attn(bf16, portable):
    say("no_alloc chunk", bf16, portable)
    rng = np.random.default_rng(71 + 2 * bf16 + portable)
    hq, hkv, d, w = 16, 2, 128, 1024
    tw = Twin(1, 24, hq, hkv, d, w, 16, bf16, portable)
    tw.reset(0, [(b * 7919 + 2**24 - 300) for b in range(24)], [(b * 37) % w for b in range(24)])
    for _ in range(w // 16 + 9):
        tw.append(0, 0, rand(rng, 24, 16, hkv, d, bf16=bf16), rand(rng, 24, 16, hkv, d, bf16=bf16))
    # first call: all 24 streams, 16 queries; second: 6 streams, 4 queries
    for b0, nb, n in ((0, 24, 16), (9, 6, 4)):
        q = rand(rng, nb, n, hq, d, bf16=bf16)
        qd = to_device(q, bf16)
        ref = empty_out((nb, n, hq, d), bf16)
        got = empty_out((nb, n, hq, d), bf16)
        tw.gpu.chunk_attn(0, b0, nb, n, qd, ref)
        tw.gpu.chunk_attn_static(0, b0, nb, n, qd, got)
        assert bool((got == ref).all()), (b0, nb, n)
        exp = tw.ora.chunk(0, b0, q)
        err = float(np.max(np.abs(to_host_f64(got, bf16) - exp)))
        assert err <= tw.tol, (b0, nb, n, err)
    tw.close()


def test_static_scratch_rejects_oversize():
    say("no_alloc oversize")
    rng = np.random.default_rng(5)
    hq, hkv, d, w = 16, 8, 128, 32
    cfg = a8r.make_config(1, 128, hq, hkv, d, w, 16, True)
    c = a8r.Cache(cfg)
    c.reset(0, list(range(128)))
    k = to_device(rand(rng, 128, 16, hkv, d), True)
    c.append_kv(0, 0, 128, 16, k, k)
    before = [c.get_state(0, b) for b in range(128)]
    q = to_device(rand(rng, 128, 16, hq, d), True)
    out = empty_out((128, 16, hq, d), True)
    # 128 streams x 8 KV heads x 16 splits x 32 rows x 130 floats: 272 MB > 64 MiB
    with pytest.raises(a8r.A8RError) as e:
        c.chunk_attn_static(0, 0, 128, 16, q, out)
    assert e.value.status == a8r.A8R_EINVAL
    with pytest.raises(a8r.A8RError) as e:
        c.chunk_attn_static(0, 0, 4, 1, q, out)                # one query: a8r_decode_attn
    assert e.value.status == a8r.A8R_EINVAL
    assert [c.get_state(0, b) for b in range(128)] == before
    # a smaller batch of the same cache fits and matches a8r_chunk_attn
    ref = empty_out((8, 16, hq, d), True)
    got = empty_out((8, 16, hq, d), True)
    c.chunk_attn(0, 0, 8, 16, q, ref)
    c.chunk_attn_static(0, 0, 8, 16, q, got)
    assert bool((got == ref).all())
    c.close()
