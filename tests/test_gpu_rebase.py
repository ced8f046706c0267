"""GPU parity and drift measurement of the rebase-on-evict comparison variant
(A8R_REBASE_ON_EVICT), through the C ABI.

* stored keys: after appends with evictions (single tokens and chunks, several
  wraps, bf16 and float32, D = 64 and 128) the K ring read back equals the
  oracle's emulation (oracle/rebase.py) bit for bit: every re-rotation of every
  key rounds exactly as the oracle's float32 arithmetic does;
* attention over the stored keys (MFMA decode, portable decode and chunk, fused
  append + decode) matches the oracle's variant attention within the usual
  tolerance;
* drift: one 3B-shaped stream (W = 4096, D = 128, 16/2 heads) run for 100,000
  steps in both cache modes, its decode output compared with the exact
  re-based attention of the oracle at the end of every window.  The method's error stays at
  bf16 rounding; the variant's grows with the number of re-rotations its keys
  have been through (printed; the test asserts that it grows past the method's).
"""

import numpy as np
import pytest

import rolling_kv_cache_ring_amd as a8r
import synth
import oracle.attention as att
import oracle.rebase as rb
from gpu_util import say, to_device, empty_out, to_host_f64, current_stream, TOL_BF16, TOL_F32

pytestmark = pytest.mark.gpu


def _rand(rng, shape, bf16):
    x = rng.standard_normal(shape).astype(np.float32)
    return synth.round_bf16(x) if bf16 else x


class VariantTwin:
    def __init__(self, n_streams, hq, hkv, d, w, max_chunk, bf16, portable=False, p0=None, s0=None):
        cfg = a8r.make_config(1, n_streams, hq, hkv, d, w, max_chunk, bf16, portable=portable,
                              rebase_on_evict=True)
        self.gpu = a8r.Cache(cfg, stream=current_stream())
        p0 = p0 or [0] * n_streams
        s0 = s0 if s0 is not None else [p % w for p in p0]
        self.gpu.reset(0, p0, s0)
        self.ora = [rb.RebaseStream(w, hkv, d, bf16, next_pos=p0[b], next_slot=s0[b]) for b in range(n_streams)]
        self.bf16, self.hq, self.hkv, self.d, self.w = bf16, hq, hkv, d, w
        self.worst = 0.0

    def append(self, k, v):                        # k, v [B, n, Hkv, D] host float32
        b_n, n = k.shape[0], k.shape[1]
        self.gpu.append_kv(0, 0, b_n, n, to_device(k, self.bf16), to_device(v, self.bf16))
        for b in range(b_n):
            self.ora[b].append(k[b], v[b])

    def attend(self, q, fused_kv=None):            # q [B, C, Hq, D]
        b_n, c = q.shape[0], q.shape[1]
        tol = TOL_BF16 if self.bf16 else TOL_F32
        if fused_kv is not None:
            k, v = fused_kv
            if c == 1:
                out = empty_out((b_n, self.hq, self.d), self.bf16)
                self.gpu.append_decode_attn(0, 0, b_n, to_device(k, self.bf16), to_device(v, self.bf16),
                                            to_device(q[:, 0], self.bf16), out)
                got = to_host_f64(out, self.bf16)[:, None]
            else:
                out = empty_out((b_n, c, self.hq, self.d), self.bf16)
                self.gpu.append_chunk_attn(0, 0, b_n, c, to_device(k, self.bf16), to_device(v, self.bf16),
                                           to_device(q, self.bf16), out)
                got = to_host_f64(out, self.bf16)
            for b in range(b_n):
                self.ora[b].append(k[b], v[b])
        elif c == 1:
            out = empty_out((b_n, self.hq, self.d), self.bf16)
            self.gpu.decode_attn(0, 0, b_n, to_device(q[:, 0], self.bf16), out)
            got = to_host_f64(out, self.bf16)[:, None]
        else:
            out = empty_out((b_n, c, self.hq, self.d), self.bf16)
            self.gpu.chunk_attn(0, 0, b_n, c, to_device(q, self.bf16), out)
            got = to_host_f64(out, self.bf16)
        for b in range(b_n):
            exp = self.ora[b].attention(q[b])
            err = float(np.max(np.abs(got[b] - exp)))
            self.worst = max(self.worst, err)
            assert err <= tol, (b, err)

    def check_ring(self):
        for b, o in enumerate(self.ora):
            k, v = self.gpu.read_ring(0, b)
            live = [o.led.slot_of_live(j) for j in range(o.led.length)]
            kk = synth.from_storage(k, self.bf16)
            vv = synth.from_storage(v, self.bf16)
            assert np.array_equal(kk[live].view(np.uint32), o.k[live].astype(np.float32).view(np.uint32)), b
            assert np.array_equal(vv[live], o.v[live].astype(np.float32)), b

    def close(self):
        self.gpu.close()


@pytest.mark.parametrize("portable", [False, True])
@pytest.mark.parametrize("w,chunks,hq,hkv,d,bf16", [
    (64, [1], 16, 2, 128, True), (96, [1, 5, 1, 8], 8, 8, 64, True), (48, [3], 4, 2, 64, False),
    (300, [1, 16, 2], 16, 2, 128, True), (33, [1], 16, 1, 128, False),
])
def test_rebase_ring_and_attention(w, chunks, hq, hkv, d, bf16, portable):
    say("rebase ring", w, chunks, hq, hkv, d, bf16, portable)
    rng = np.random.default_rng(w * 7 + d)
    tw = VariantTwin(2, hq, hkv, d, w, max(chunks), bf16, portable, p0=[0, 2**24 - w // 2], s0=[0, 5 % w])
    t = 0
    while tw.ora[0].led.next_pos < 3 * w + 7:
        n = chunks[t % len(chunks)]
        k, v = _rand(rng, (2, n, hkv, d), bf16), _rand(rng, (2, n, hkv, d), bf16)
        tw.append(k, v)
        if t % 3 == 0 or n > 1:
            tw.attend(_rand(rng, (2, n, hq, d), bf16))
        t += 1
    tw.check_ring()
    say("worst err", tw.worst)
    tw.close()


def test_rebase_fused_append_decode():
    say("rebase fused append+decode")
    rng = np.random.default_rng(11)
    hq, hkv, d, w = 16, 2, 128, 80
    tw = VariantTwin(3, hq, hkv, d, w, 1, True)
    for t in range(2 * w + 9):
        k, v = _rand(rng, (3, 1, hkv, d), True), _rand(rng, (3, 1, hkv, d), True)
        tw.attend(_rand(rng, (3, 1, hq, d), True), fused_kv=(k, v))
    tw.check_ring()
    tw.close()


def test_rebase_fused_append_chunk():
    """In this mode a8r_append_chunk_attn runs as append + re-rotation + chunk."""
    say("rebase fused append+chunk")
    rng = np.random.default_rng(12)
    hq, hkv, d, w = 16, 2, 128, 80
    tw = VariantTwin(2, hq, hkv, d, w, 8, True, p0=[3, 2**24 - 5], s0=[0, 17])
    for t in range(3 * w // 6 + 4):
        n = 8 if t % 3 else 3
        k, v = _rand(rng, (2, n, hkv, d), True), _rand(rng, (2, n, hkv, d), True)
        tw.attend(_rand(rng, (2, n, hq, d), True), fused_kv=(k, v))
    tw.check_ring()
    tw.close()


def test_rebase_streaming_launch():
    """10 streams of the 3B-class shape (W = 4096, 42 MB of windows per launch):
    decode takes the instance with streaming K/V loads; the stored keys after a
    full window and evicting appends bit for bit, and attention within
    tolerance."""
    say("rebase streaming launch")
    rng = np.random.default_rng(13)
    hq, hkv, d, w, nb = 16, 2, 128, 4096, 10
    tw = VariantTwin(nb, hq, hkv, d, w, 512, True, p0=[5 * b for b in range(nb)],
                     s0=[(b * 977) % w for b in range(nb)])
    for _ in range(8):
        tw.append(_rand(rng, (nb, 512, hkv, d), True), _rand(rng, (nb, 512, hkv, d), True))
    tw.attend(_rand(rng, (nb, 1, hq, d), True))
    for _ in range(2):
        tw.append(_rand(rng, (nb, 1, hkv, d), True), _rand(rng, (nb, 1, hkv, d), True))
        tw.attend(_rand(rng, (nb, 1, hq, d), True))
    tw.check_ring()
    say("worst err", tw.worst)
    tw.close()


def test_drift_3b_stream_100k_steps():
    """Both cache modes on one 3B-shaped stream (W = 4096) for 100,000 decode
    steps (24.4 wraps), with the decode output compared to the exact re-based
    attention of the oracle at the end of every window and at the last step.
    The method's error stays at bf16 rounding; the variant's grows with the
    re-rotations its keys have been through ("Audio8 ASR Infinite: What It
    Actually Takes to Listen Forever", section "Failure Modes That Only Appear
    on Day Three of a Session": error entering at every cache boundary)."""
    hq, hkv, d, w = 16, 2, 128, 4096
    steps = 100_000
    rng = np.random.default_rng(12)
    L = a8r.lib()
    caches = {}
    for name, mode in (("rotate_on_read", False), ("rebase_on_evict", True)):
        cfg = a8r.make_config(1, 1, hq, hkv, d, w, 1, True, rebase_on_evict=mode)
        caches[name] = a8r.Cache(cfg, stream=current_stream())
    checks = set(range(w - 1, steps, w)) | {steps - 1}
    out = {n: empty_out((1, hq, d), True) for n in caches}
    errs = {n: [] for n in caches}
    block = w                                       # inputs drawn one window at a time
    prev_k = np.zeros((0, hkv, d), np.float32)      # the last W tokens before the block
    prev_v = np.zeros((0, hkv, d), np.float32)
    row = hkv * d * 2
    for t0 in range(0, steps, block):
        n = min(block, steps - t0)
        ks, vs = _rand(rng, (n, hkv, d), True), _rand(rng, (n, hkv, d), True)
        kd, vd = to_device(ks, True), to_device(vs, True)
        for j in range(n):
            t = t0 + j
            for c in caches.values():
                st = L.a8r_append_kv(c.handle, 0, 0, 1, 1, kd.data_ptr() + j * row, vd.data_ptr() + j * row,
                                     None, None)
                assert st == 0, L.a8r_last_error()
            if t in checks:
                q = _rand(rng, (1, hq, d), True)
                qd = to_device(q, True)
                for name, c in caches.items():
                    c.decode_attn(0, 0, 1, qd, out[name])
                lk = np.concatenate([prev_k, ks[: j + 1]])[-w:]     # the live window
                lv = np.concatenate([prev_v, vs[: j + 1]])[-w:]
                exact = att.decode_rebased(q[0], lk, lv)
                for name in caches:
                    got = to_host_f64(out[name], True)[0]
                    errs[name].append(float(np.max(np.abs(got - exact))))
                say("step", t + 1, {nm: round(e[-1], 5) for nm, e in errs.items()})
        prev_k = np.concatenate([prev_k, ks])[-w:]
        prev_v = np.concatenate([prev_v, vs])[-w:]
    for c in caches.values():
        c.close()
    say("drift (max |out - exact|) at steps", sorted(x + 1 for x in checks), errs)
    assert max(errs["rotate_on_read"]) <= TOL_BF16
    assert errs["rebase_on_evict"][-1] > 2 * max(errs["rotate_on_read"])
