"""GPU parity on the five synthetic workloads, through the C ABI.

* tiny_mha_fp32   every one of the 256 steps against the oracle (float32, 1e-5);
* audio8_0p1b     all 8192 steps appended on all 8 layers; attention checked on
                  every 64th step and around every wraparound;
* qwen3b_single   all 100,000 steps (about 24 wraps) on layers 0 and 35 of the
                  36-layer cache, bookkeeping at every step, attention at every
                  wraparound +-2 and 30 seeded random steps;
* qwen3b_batch64  the benchmark's configuration at full size (36 layers, 64
                  streams, W = 4096, seeded start positions and ring offsets,
                  9.66 GB of ring): batched append + decode calls over all 64
                  streams, outputs of 9 sampled (layer, stream) pairs checked;
* qwen3b_chunk8   full size (16 streams, W = 8192, positions crossing 2**24),
                  batched 8-token append + chunk attention (one fused call, as
                  the benchmark runs it, and the two calls), sampled pairs checked;
* qwen3b_chunk12/16  the same at 12 and 16 positions per call.
Inputs are the seeded N(0, 1) draws of ``synth``; unsampled pairs of the full
size workloads are filled with other device-side random values that are never
compared (only their finiteness is).
"""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
import synth
from gpu_util import Twin, say, to_device, empty_out, to_host_f64, current_stream, TOL_BF16
from oracle.model import OracleCache

pytestmark = pytest.mark.gpu
W_ = synth.WORKLOADS


def draw(wl, layer, stream, kind, pos0, count, heads):
    return synth.draw(wl.workload_id, layer, stream, kind, pos0, count, heads, wl.head_dim, wl.bf16)


def test_tiny_mha_fp32_every_step():
    wl = W_["tiny_mha_fp32"]
    say("tiny_mha_fp32")
    tw = Twin(wl.n_layers, wl.n_streams, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window,
              1, wl.bf16)
    for t in range(wl.steps):
        k = draw(wl, 0, 0, synth.KIND_K, t, 1, wl.n_kv_heads)[None]
        v = draw(wl, 0, 0, synth.KIND_V, t, 1, wl.n_kv_heads)[None]
        tw.append(0, 0, k, v)
        tw.check_state(0, 0)
        q = draw(wl, 0, 0, synth.KIND_Q, t, 1, wl.n_q_heads)
        tw.decode(0, 0, q)
    tw.check_ring(0, 0)
    say("worst err", tw.worst)
    assert tw.worst <= 1e-5
    tw.close()


def _run_long_stream(wl, layers, steps, check_steps):
    tw = Twin(wl.n_layers, 1, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, 1, wl.bf16)
    kd, vd, kh, vh = {}, {}, {}, {}
    for layer in layers:
        kh[layer] = draw(wl, layer, 0, synth.KIND_K, 0, steps, wl.n_kv_heads)
        vh[layer] = draw(wl, layer, 0, synth.KIND_V, 0, steps, wl.n_kv_heads)
        kd[layer] = to_device(kh[layer], wl.bf16)
        vd[layer] = to_device(vh[layer], wl.bf16)
    for t in range(steps):
        for layer in layers:
            slots, ev = tw.gpu.append_kv(layer, 0, 1, 1, kd[layer][t:t + 1], vd[layer][t:t + 1])
            s_ref, e_ref = tw.ora.append(layer, 0, kh[layer][t][None, None], vh[layer][t][None, None])
            assert slots[0, 0] == s_ref[0][0] and ev[0, 0] == e_ref[0][0], (t, layer)
            if t in check_steps:
                q = draw(wl, layer, 0, synth.KIND_Q, t, 1, wl.n_q_heads)
                tw.decode(layer, 0, q)
                tw.check_state(layer, 0)
    for layer in layers:
        tw.check_ring(layer, 0)
    say("worst err", tw.worst)
    tw.close()


def test_audio8_0p1b_all_steps():
    wl = W_["audio8_0p1b"]
    say("audio8_0p1b")
    w = wl.window
    checks = set(range(0, wl.steps, 64))
    for k in range(1, wl.steps // w + 1):
        checks |= {k * w - 2, k * w - 1, k * w, k * w + 1}
    checks = {c for c in checks if 0 <= c < wl.steps}
    _run_long_stream(wl, list(range(wl.n_layers)), wl.steps, checks)


def test_qwen3b_single_100k_steps():
    wl = W_["qwen3b_single"]
    say("qwen3b_single")
    w = wl.window
    rng = np.random.default_rng(2)
    checks = set(int(x) for x in rng.integers(0, wl.steps, 30))
    for k in range(1, wl.steps // w + 1):
        checks |= {k * w - 2, k * w - 1, k * w, k * w + 1, k * w + 2}
    checks = {c for c in checks if 0 <= c < wl.steps}
    _run_long_stream(wl, [0, wl.n_layers - 1], wl.steps, checks)


def _full_size(wl, sampled_layers, sampled_streams, n_steps, chunk, fused=False):
    """Fill every (layer, stream) of the workload, then run batched steps as the
    benchmark does; compare the sampled pairs with the oracle."""
    import torch
    p0, r0 = synth.start_states(wl)
    w, hkv, hq, d = wl.window, wl.n_kv_heads, wl.n_q_heads, wl.head_dim
    B, NL = wl.n_streams, wl.n_layers
    cfg = a8r.make_config(NL, B, hq, hkv, d, w, max(chunk, w), wl.bf16)
    cache = a8r.Cache(cfg, stream=current_stream())
    ora = OracleCache(NL, B, hq, hkv, d, w)
    n_pre = np.minimum(p0, w)
    start = p0 - n_pre
    slot0 = (r0 - n_pre) % w
    cache.reset(0, start, slot0)
    ora.reset(0, start, slot0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    junk = torch.randn((B, w, hkv, d), device="cuda", generator=gen).to(torch.bfloat16).view(torch.int16)
    sampled = {(l, b) for l in sampled_layers for b in sampled_streams}
    say("prefill", wl.name)
    for layer in range(NL):
        for b in range(B):
            n = int(n_pre[b])
            if n == 0:
                continue
            if (layer, b) in sampled:
                k = draw(wl, layer, b, synth.KIND_K, int(start[b]), n, hkv)
                v = draw(wl, layer, b, synth.KIND_V, int(start[b]), n, hkv)
                cache.append_kv(layer, b, 1, n, to_device(k[None], True), to_device(v[None], True),
                                want_bookkeeping=False)
                ora.append(layer, b, k[None], v[None])
            else:
                cache.append_kv(layer, b, 1, n, junk[b:b + 1, :n], junk[(b + 1) % B:(b + 1) % B + 1, :n],
                                want_bookkeeping=False)
    for layer in sampled_layers:
        for b in sampled_streams:
            assert cache.get_state(layer, b) == ora.ledger(layer, b).state()
    say("steps", wl.name)
    pos = p0.copy()
    worst = 0.0
    for step in range(n_steps):
        for layer in range(NL):
            kj = torch.randn((B, chunk, hkv, d), device="cuda", generator=gen).to(torch.bfloat16)
            vj = torch.randn((B, chunk, hkv, d), device="cuda", generator=gen).to(torch.bfloat16)
            qj = torch.randn((B, chunk, hq, d), device="cuda", generator=gen).to(torch.bfloat16)
            kj, vj, qj = kj.view(torch.int16), vj.view(torch.int16), qj.view(torch.int16)
            host = {}
            if layer in sampled_layers:
                for b in sampled_streams:
                    k = draw(wl, layer, b, synth.KIND_K, int(pos[b]), chunk, hkv)
                    v = draw(wl, layer, b, synth.KIND_V, int(pos[b]), chunk, hkv)
                    q = draw(wl, layer, b, synth.KIND_Q, int(pos[b]), chunk, hq)
                    kj[b] = to_device(k, True)
                    vj[b] = to_device(v, True)
                    qj[b] = to_device(q, True)
                    host[b] = q
                    ora.append(layer, b, k[None], v[None])
            if fused and chunk == 1:
                out = empty_out((B, hq, d), True)
                slots, ev = cache.append_decode_attn(layer, 0, B, kj, vj, qj[:, 0], out)
            elif fused:
                out = empty_out((B, chunk, hq, d), True)
                slots, ev = cache.append_chunk_attn(layer, 0, B, chunk, kj, vj, qj, out)
            else:
                slots, ev = cache.append_kv(layer, 0, B, chunk, kj, vj)
            for b in host:
                led = ora.ledger(layer, b)
                exp_slots = [(led.next_slot - chunk + j) % w for j in range(chunk)]
                assert list(slots[b]) == exp_slots
            if fused:
                pass
            elif chunk == 1:
                out = empty_out((B, hq, d), True)
                cache.decode_attn(layer, 0, B, qj[:, 0], out)
            else:
                out = empty_out((B, chunk, hq, d), True)
                cache.chunk_attn(layer, 0, B, chunk, qj, out)
            got = to_host_f64(out, True)
            assert np.all(np.isfinite(got))
            for b, q in host.items():
                exp = ora.chunk(layer, b, q[None])[0]
                g = got[b] if chunk > 1 else got[b][None]
                err = float(np.max(np.abs(g - exp)))
                worst = max(worst, err)
                assert err <= TOL_BF16, (wl.name, step, layer, b, err)
        pos += chunk
    for layer in sampled_layers:
        for b in sampled_streams:
            assert cache.get_state(layer, b) == ora.ledger(layer, b).state()
    say("worst err", worst)
    cache.close()


@pytest.mark.parametrize("fused", [True, False])
def test_qwen3b_batch64_full_size(fused):
    """The benchmark's launch configuration (fused append + decode by default)."""
    wl = W_["qwen3b_batch64"]
    _full_size(wl, [0, 17, 35], [0, 13, 63], 3, 1, fused)


@pytest.mark.parametrize("fused", [True, False])
def test_qwen3b_chunk8_full_size(fused):
    """Fused append + chunk (the benchmark's step) and the two separate calls."""
    wl = W_["qwen3b_chunk8"]
    _full_size(wl, [0, 35], [0, 9, 15], 2, 8, fused)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", ["qwen3b_chunk12", "qwen3b_chunk16"])
def test_qwen3b_clock_variants_full_size(name, fused):
    """The 120 ms and 160 ms clocks: 12 and 16 new positions per call (96 and
    128 query rows per KV head)."""
    wl = W_[name]
    _full_size(wl, [0, 35], [0, 7, 15], 2, wl.chunk, fused)
