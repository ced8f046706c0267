"""The boundary's placement options on the GPU: a cache living in a
caller-owned workspace behaves bit for bit like one the library allocates, a
workspace too small or misaligned is refused before anything is touched, and
a cache moved to another stream with a8r_set_stream keeps its results."""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
import synth
from gpu_util import Twin, current_stream, say, to_device

pytestmark = pytest.mark.gpu


def draw(rng, shape):
    return synth.round_bf16(rng.standard_normal(shape).astype(np.float32))


def run_sequence(cache, rng, nb, hq, hkv, d, chunk, torch):
    """A fixed mix of appends, decodes, chunks and fused calls; returns every
    output's bits."""
    outs = []
    cache.reset(0, [2**30 + 7 * b for b in range(nb)], [(5 * b) % 96 for b in range(nb)])
    for t in range(40):
        layer = t % 2
        k, v = draw(rng, (nb, chunk, hkv, d)), draw(rng, (nb, chunk, hkv, d))
        q = draw(rng, (nb, chunk, hq, d))
        qd, kd, vd = to_device(q, True), to_device(k, True), to_device(v, True)
        out = torch.empty((nb, chunk, hq, d), dtype=torch.int16, device="cuda")
        if t % 4 == 0:
            cache.append_kv(layer, 0, nb, chunk, kd, vd)
            cache.chunk_attn(layer, 0, nb, chunk, qd, out)
        elif t % 4 == 1:
            cache.append_chunk_attn(layer, 0, nb, chunk, kd, vd, qd, out)
        elif t % 4 == 2:
            k1, v1 = to_device(k[:, :1], True), to_device(v[:, :1], True)
            q1 = to_device(q[:, 0], True)
            out = torch.empty((nb, hq, d), dtype=torch.int16, device="cuda")
            cache.append_decode_attn(layer, 0, nb, k1, v1, q1, out)
        else:
            cache.append_kv(layer, 0, nb, 1, to_device(k[:, :1], True), to_device(v[:, :1], True))
            out = torch.empty((nb, hq, d), dtype=torch.int16, device="cuda")
            cache.decode_attn(layer, 0, nb, to_device(q[:, 0], True), out)
        outs.append(out.cpu().numpy().copy())
    return outs


def test_caller_workspace_is_bitwise_the_same_cache():
    """Every output, the state and both rings of a cache placed in a torch
    workspace equal those of a cache the library allocates."""
    import torch
    say("caller_workspace")
    nb, hq, hkv, d, w, chunk = 3, 16, 2, 128, 96, 8
    cfg = a8r.make_config(2, nb, hq, hkv, d, w, chunk, True)
    need = a8r.workspace_bytes(cfg)
    assert need > 0
    ws = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws_ptr = ws.data_ptr() + off
    own = a8r.Cache(cfg, stream=current_stream())
    placed = a8r.Cache(cfg, stream=current_stream(), workspace=ws_ptr, ws_bytes=need)
    a = run_sequence(own, np.random.default_rng(5), nb, hq, hkv, d, chunk, torch)
    b = run_sequence(placed, np.random.default_rng(5), nb, hq, hkv, d, chunk, torch)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    for layer in range(2):
        for s in range(nb):
            assert own.get_state(layer, s) == placed.get_state(layer, s)
            ka, va = own.read_ring(layer, s)
            kb, vb = placed.read_ring(layer, s)
            assert np.array_equal(ka, kb) and np.array_equal(va, vb)
    placed.close()
    own.close()
    del ws


def test_workspace_too_small_or_misaligned_is_refused():
    import torch
    say("workspace_refused")
    cfg = a8r.make_config(1, 2, 8, 2, 64, 64, 4, True)
    need = a8r.workspace_bytes(cfg)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    base = ws.data_ptr() + (-ws.data_ptr()) % 256
    with pytest.raises(a8r.A8RError) as e:
        a8r.Cache(cfg, stream=current_stream(), workspace=base, ws_bytes=need - 1)
    assert e.value.status == 2                    # A8R_ENOMEM
    with pytest.raises(a8r.A8RError) as e:
        a8r.Cache(cfg, stream=current_stream(), workspace=base + 16, ws_bytes=need)
    assert e.value.status == 1                    # A8R_EINVAL
    del ws


def test_set_stream_keeps_results():
    """Half the calls on the creating stream, half on a second stream after
    a8r_set_stream (ordered by a synchronize), all against the oracle."""
    import torch
    say("set_stream")
    rng = np.random.default_rng(11)
    nb, hq, hkv, d, w = 2, 8, 2, 64, 80
    tw = Twin(1, nb, hq, hkv, d, w, 4, True)
    tw.reset(0, [12345, 2**35], [3, 70])
    side = torch.cuda.Stream()
    for t in range(60):
        if t == 30:
            torch.cuda.synchronize()
            tw.gpu.set_stream(side.cuda_stream)
        with torch.cuda.stream(side if t >= 30 else torch.cuda.current_stream()):
            k, v = draw(rng, (nb, 2, hkv, d)), draw(rng, (nb, 2, hkv, d))
            tw.append_chunk(0, 0, k, v, draw(rng, (nb, 2, hq, d)))
            k, v = draw(rng, (nb, 1, hkv, d)), draw(rng, (nb, 1, hkv, d))
            tw.append_decode(0, 0, k, v, draw(rng, (nb, hq, d)))
    torch.cuda.synchronize()
    for b in range(nb):
        tw.check_state(0, b)
        tw.check_ring(0, b)
    tw.close()
