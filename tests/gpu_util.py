"""Helpers for GPU parity tests: drive the HIP cache (through the C ABI) and the
oracle side by side on the same seeded inputs.

Tolerances (max |oracle_fp64 - gpu|, unit-variance inputs):
  float32 path: 1e-5;  bf16 path: 2e-2.
Bookkeeping (slots, evicted positions, per-pair state) and ring contents are
compared bit for bit.
"""

from __future__ import annotations

import sys

import numpy as np

import rolling_kv_cache_ring_amd as a8r
import synth
from oracle.model import OracleCache

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def torch():
    import torch as _t
    return _t


def say(*msg):
    print("[gpu]", *msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, bf16: bool):
    """float32 values (bf16-representable when bf16) -> device tensor of storage bits."""
    t = torch()
    st = synth.to_storage(x, bf16)
    if bf16:
        return t.from_numpy(np.ascontiguousarray(st).view(np.int16)).cuda()
    return t.from_numpy(np.ascontiguousarray(st)).cuda()


def empty_out(shape, bf16: bool):
    t = torch()
    return t.empty(shape, dtype=t.int16 if bf16 else t.float32, device="cuda")


def to_host_f64(x, bf16: bool) -> np.ndarray:
    a = x.detach().cpu().numpy()
    if bf16:
        return synth.bf16_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


def current_stream() -> int:
    return torch().cuda.current_stream().cuda_stream


class Twin:
    """One HIP cache and one oracle cache fed identical inputs."""

    def __init__(self, n_layers, n_streams, hq, hkv, d, window, max_chunk=1, bf16=True,
                 portable=False, theta=1.0e6, prefix_capacity=0):
        self.shape = (n_layers, n_streams, hq, hkv, d, window)
        self.bf16 = bf16
        self.hq, self.hkv, self.d, self.window = hq, hkv, d, window
        self.cfg = a8r.make_config(n_layers, n_streams, hq, hkv, d, window, max_chunk, bf16, theta,
                                   portable=portable, prefix_capacity=prefix_capacity)
        self.gpu = a8r.Cache(self.cfg, stream=current_stream())
        self.ora = OracleCache(n_layers, n_streams, hq, hkv, d, window, theta)
        self.tol = TOL_BF16 if bf16 else TOL_F32
        self.worst = 0.0

    def close(self):
        self.gpu.close()

    def reset(self, b0, pos, slot=None):
        self.gpu.reset(b0, pos, slot)
        self.ora.reset(b0, pos, slot)

    def append(self, layer, b0, k, v):
        """k, v float32 [nb, n, Hkv, D]; checks slots / evicted bit-exactly."""
        nb, n = k.shape[:2]
        kd, vd = to_device(k, self.bf16), to_device(v, self.bf16)
        slots, ev = self.gpu.append_kv(layer, b0, nb, n, kd, vd)
        s_ref, e_ref = self.ora.append(layer, b0, k, v)
        assert np.array_equal(slots, np.array(s_ref, dtype=np.int32)), (slots, s_ref)
        assert np.array_equal(ev, np.array(e_ref, dtype=np.int64)), (ev, e_ref)
        return kd, vd

    def append_prefix(self, layer, b0, k, v):
        """k, v float32 [nb, n, Hkv, D]: pinned prefix tokens of streams b0 .. b0 + nb - 1."""
        nb, n = k.shape[:2]
        self.gpu.append_prefix(layer, b0, nb, n, to_device(k, self.bf16), to_device(v, self.bf16))
        self.ora.append_prefix(layer, b0, k, v)
        for i in range(nb):
            assert self.gpu.prefix_length(layer, b0 + i) == self.ora.prefix_kv(layer, b0 + i)[0].shape[0]

    def clear_prefix(self, b0, nb):
        self.gpu.clear_prefix(b0, nb)
        self.ora.clear_prefix(b0, nb)

    def check_state(self, layer, b):
        got = self.gpu.get_state(layer, b)
        exp = self.ora.ledger(layer, b).state()
        assert got == exp, (layer, b, got, exp)

    def decode(self, layer, b0, q, check=True):
        nb = q.shape[0]
        out = empty_out((nb, self.hq, self.d), self.bf16)
        self.gpu.decode_attn(layer, b0, nb, to_device(q, self.bf16), out)
        got = to_host_f64(out, self.bf16)
        if check:
            exp = self.ora.decode(layer, b0, q)
            self._cmp(got, exp, ("decode", layer, b0))
        return got

    def append_decode(self, layer, b0, k, v, q, check=True):
        """a8r_append_decode_attn: k, v [nb, 1, Hkv, D], q [nb, Hq, D]."""
        nb = q.shape[0]
        out = empty_out((nb, self.hq, self.d), self.bf16)
        slots, ev = self.gpu.append_decode_attn(layer, b0, nb, to_device(k, self.bf16), to_device(v, self.bf16),
                                                to_device(q, self.bf16), out)
        s_ref, e_ref = self.ora.append(layer, b0, k, v)
        assert np.array_equal(slots, np.array(s_ref, dtype=np.int32)), (slots, s_ref)
        assert np.array_equal(ev, np.array(e_ref, dtype=np.int64)), (ev, e_ref)
        got = to_host_f64(out, self.bf16)
        if check:
            exp = self.ora.decode(layer, b0, q)
            self._cmp(got, exp, ("append_decode", layer, b0))
        return got

    def append_chunk(self, layer, b0, k, v, q, check=True):
        """a8r_append_chunk_attn: k, v [nb, n, Hkv, D], q [nb, n, Hq, D]."""
        nb, n = q.shape[:2]
        out = empty_out((nb, n, self.hq, self.d), self.bf16)
        slots, ev = self.gpu.append_chunk_attn(layer, b0, nb, n, to_device(k, self.bf16), to_device(v, self.bf16),
                                               to_device(q, self.bf16), out)
        s_ref, e_ref = self.ora.append(layer, b0, k, v)
        assert np.array_equal(slots, np.array(s_ref, dtype=np.int32)), (slots, s_ref)
        assert np.array_equal(ev, np.array(e_ref, dtype=np.int64)), (ev, e_ref)
        got = to_host_f64(out, self.bf16)
        if check:
            exp = self.ora.chunk(layer, b0, q)
            self._cmp(got, exp, ("append_chunk", layer, b0))
        return got

    def chunk(self, layer, b0, q, check=True):
        nb, n = q.shape[:2]
        out = empty_out((nb, n, self.hq, self.d), self.bf16)
        self.gpu.chunk_attn(layer, b0, nb, n, to_device(q, self.bf16), out)
        got = to_host_f64(out, self.bf16)
        if check:
            exp = self.ora.chunk(layer, b0, q)
            self._cmp(got, exp, ("chunk", layer, b0))
        return got

    def _cmp(self, got, exp, what):
        assert np.all(np.isfinite(got)), what
        err = float(np.max(np.abs(got - exp)))
        self.worst = max(self.worst, err)
        assert err <= self.tol, (what, err, self.tol)

    def check_ring(self, layer, b):
        """Ring readback equals the appended tokens on every live slot, bit for
        bit, K and V alike: the ring is a copy of what was appended, at the
        slots the oracle ledger assigns."""
        k, v = self.gpu.read_ring(layer, b)
        led = self.ora.ledger(layer, b)
        _, ring_k, ring_v = self.ora._pair(layer, b)
        live = [led.slot_of_live(j) for j in range(led.length)]
        kk = synth.from_storage(k, self.bf16)
        vv = synth.from_storage(v, self.bf16)
        # the oracle holds the appended float32 values widened exactly to float64
        assert np.array_equal(kk[live].view(np.uint32), ring_k[live].astype(np.float32).view(np.uint32))
        assert np.array_equal(vv[live].view(np.uint32), ring_v[live].astype(np.float32).view(np.uint32))
