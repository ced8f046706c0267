"""Python binding of the a8r C ABI (rolling-window attention with exact RoPE re-basing).

Argument marshalling only: every step of the path runs in the HIP library
``liba8r.so`` built next to this file.  Device buffers are passed as raw device
addresses (``torch.Tensor.data_ptr()`` of CUDA tensors works); the library
never sees torch types.  If the library is missing, importing this package
still works but every call raises ``LibraryNotBuilt`` - there is no fallback.

The names mirror ``include/a8r.h``: ``cache_create``, ``reset``, ``append_kv``,
``decode_attn``, ``chunk_attn``, ``get_state``, ``read_ring``, ``cache_destroy``
and the host-only ``Ledger``.  ``Cache`` is a thin object wrapper.
"""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liba8r.so")

A8R_OK, A8R_EINVAL, A8R_ENOMEM, A8R_EDEVICE, A8R_ESTATE, A8R_EUNSUPPORTED = range(6)
A8R_F32, A8R_BF16 = 0, 1
A8R_KERNELS_AUTO, A8R_KERNELS_PORTABLE = 0, 1
A8R_ROTATE_ON_READ, A8R_REBASE_ON_EVICT = 0, 1
STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "ENOMEM", 3: "EDEVICE", 4: "ESTATE", 5: "EUNSUPPORTED"}

EXPORTED = [
    "a8r_workspace_bytes", "a8r_cache_create", "a8r_cache_destroy", "a8r_set_stream", "a8r_reset",
    "a8r_append_kv", "a8r_decode_attn", "a8r_chunk_attn", "a8r_chunk_attn_static", "a8r_append_decode_attn",
    "a8r_append_chunk_attn",
    "a8r_get_state", "a8r_read_ring", "a8r_rebuild_window", "a8r_append_prefix", "a8r_export_prefix", "a8r_import_prefix", "a8r_clear_prefix",
    "a8r_prefix_length",
    "a8r_last_error", "a8r_ledger_create", "a8r_ledger_destroy", "a8r_ledger_reset",
    "a8r_ledger_append", "a8r_ledger_get", "a8r_version",
]


class LibraryNotBuilt(RuntimeError):
    pass


class A8RError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"a8r {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_streams", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("kernel_policy", ctypes.c_int32), ("cache_mode", ctypes.c_int32),
        ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
        ("reserved_f", ctypes.c_float), ("prefix_capacity", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


_lib = None
_c_void_p = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The loaded library; raises LibraryNotBuilt if liba8r.so is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(f"{LIB_PATH} not found: build it with "
                              "`python -m rolling_kv_cache_ring_amd.build`")
    # PyTorch wheels for ROCm ship their own HIP runtime under the same soname
    # as the system's; whichever is loaded first serves the whole process.
    # Loading the library before PyTorch would bring in a second HIP/HSA
    # runtime beside PyTorch's, and the second to open the GPU finds none, so
    # PyTorch (when installed) is imported first.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    L.a8r_workspace_bytes.argtypes = [ctypes.POINTER(Config)]
    L.a8r_workspace_bytes.restype = ctypes.c_size_t
    L.a8r_cache_create.argtypes = [ctypes.POINTER(Config), _c_void_p, _c_void_p, ctypes.c_size_t,
                                   ctypes.POINTER(_c_void_p)]
    L.a8r_cache_create.restype = st
    L.a8r_cache_destroy.argtypes = [_c_void_p]
    L.a8r_cache_destroy.restype = None
    L.a8r_set_stream.argtypes = [_c_void_p, _c_void_p]
    L.a8r_set_stream.restype = st
    L.a8r_reset.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _i64p, _i32p]
    L.a8r_reset.restype = st
    L.a8r_append_kv.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                _c_void_p, _c_void_p, _i32p, _i64p]
    L.a8r_append_kv.restype = st
    L.a8r_decode_attn.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _c_void_p, _c_void_p]
    L.a8r_decode_attn.restype = st
    L.a8r_chunk_attn.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                 _c_void_p, _c_void_p]
    L.a8r_chunk_attn.restype = st
    L.a8r_chunk_attn_static.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        _c_void_p, _c_void_p]
    L.a8r_chunk_attn_static.restype = st
    L.a8r_rebuild_window.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, _c_void_p, _c_void_p, _c_void_p]
    L.a8r_rebuild_window.restype = st
    L.a8r_append_decode_attn.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32p, _i64p]
    L.a8r_append_decode_attn.restype = st
    L.a8r_append_chunk_attn.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32p, _i64p]
    L.a8r_append_chunk_attn.restype = st
    L.a8r_append_prefix.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _c_void_p, _c_void_p]
    L.a8r_append_prefix.restype = st
    L.a8r_export_prefix.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _c_void_p, _c_void_p]
    L.a8r_export_prefix.restype = st
    L.a8r_import_prefix.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _c_void_p, _c_void_p]
    L.a8r_import_prefix.restype = st
    L.a8r_clear_prefix.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32]
    L.a8r_clear_prefix.restype = st
    L.a8r_prefix_length.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _i32p]
    L.a8r_prefix_length.restype = st
    L.a8r_get_state.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _i64p, _i32p, _i32p]
    L.a8r_get_state.restype = st
    L.a8r_read_ring.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _c_void_p, _c_void_p]
    L.a8r_read_ring.restype = st
    L.a8r_last_error.argtypes = []
    L.a8r_last_error.restype = ctypes.c_char_p
    L.a8r_version.argtypes = []
    L.a8r_version.restype = ctypes.c_char_p
    L.a8r_ledger_create.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(_c_void_p)]
    L.a8r_ledger_create.restype = st
    L.a8r_ledger_destroy.argtypes = [_c_void_p]
    L.a8r_ledger_destroy.restype = None
    L.a8r_ledger_reset.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _i64p, _i32p]
    L.a8r_ledger_reset.restype = st
    L.a8r_ledger_append.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    _i32p, _i64p]
    L.a8r_ledger_append.restype = st
    L.a8r_ledger_get.argtypes = [_c_void_p, ctypes.c_int32, ctypes.c_int32, _i64p, _i32p, _i32p]
    L.a8r_ledger_get.restype = st
    _lib = L
    return L


def _check(status: int) -> None:
    if status != A8R_OK:
        raise A8RError(status, lib().a8r_last_error().decode())


def _ptr(x):
    """Device/host address of a tensor, numpy array, int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot take the address of {type(x)}")


def _i64_array(vals):
    a = np.ascontiguousarray(np.asarray(vals, dtype=np.int64))
    return a, a.ctypes.data_as(_i64p)


def _i32_array(vals):
    a = np.ascontiguousarray(np.asarray(vals, dtype=np.int32))
    return a, a.ctypes.data_as(_i32p)


def make_config(n_layers, n_streams, n_q_heads, n_kv_heads, head_dim, window, max_chunk=1,
                bf16=True, rope_theta=1.0e6, softmax_scale=0.0, portable=False,
                rebase_on_evict=False, prefix_capacity=0) -> Config:
    return Config(n_layers, n_streams, n_q_heads, n_kv_heads, head_dim, window, max_chunk,
                  A8R_BF16 if bf16 else A8R_F32,
                  A8R_KERNELS_PORTABLE if portable else A8R_KERNELS_AUTO,
                  A8R_REBASE_ON_EVICT if rebase_on_evict else A8R_ROTATE_ON_READ,
                  float(rope_theta), float(softmax_scale), 0.0, int(prefix_capacity), 0)


def workspace_bytes(cfg: Config) -> int:
    return int(lib().a8r_workspace_bytes(ctypes.byref(cfg)))


def version() -> str:
    return lib().a8r_version().decode()


# ---- C-ABI mirrors ---------------------------------------------------------------

def cache_create(cfg: Config, stream: int | None = None, workspace=None, ws_bytes: int = 0) -> int:
    h = _c_void_p()
    _check(lib().a8r_cache_create(ctypes.byref(cfg), stream, _ptr(workspace), ws_bytes, ctypes.byref(h)))
    return h.value


def cache_destroy(handle: int) -> None:
    lib().a8r_cache_destroy(handle)


def set_stream(handle: int, stream: int | None) -> None:
    _check(lib().a8r_set_stream(handle, stream))


def reset(handle: int, b0: int, next_pos, next_slot=None) -> None:
    pos, pos_p = _i64_array(next_pos)
    slot_p = None
    if next_slot is not None:
        slot, slot_p = _i32_array(next_slot)
    _check(lib().a8r_reset(handle, b0, len(pos), pos_p, slot_p))


def append_kv(handle: int, layer: int, b0: int, nb: int, n_new: int, k, v, want_bookkeeping=True):
    """Returns (slots [nb, n_new] int32, evicted [nb, n_new] int64) or (None, None)."""
    if want_bookkeeping:
        slots = np.empty((nb, n_new), dtype=np.int32)
        ev = np.empty((nb, n_new), dtype=np.int64)
        _check(lib().a8r_append_kv(handle, layer, b0, nb, n_new, _ptr(k), _ptr(v),
                                   slots.ctypes.data_as(_i32p), ev.ctypes.data_as(_i64p)))
        return slots, ev
    _check(lib().a8r_append_kv(handle, layer, b0, nb, n_new, _ptr(k), _ptr(v), None, None))
    return None, None


def decode_attn(handle: int, layer: int, b0: int, nb: int, q, out) -> None:
    _check(lib().a8r_decode_attn(handle, layer, b0, nb, _ptr(q), _ptr(out)))


def chunk_attn(handle: int, layer: int, b0: int, nb: int, n_new: int, q, out) -> None:
    _check(lib().a8r_chunk_attn(handle, layer, b0, nb, n_new, _ptr(q), _ptr(out)))


def chunk_attn_static(handle: int, layer: int, b0: int, nb: int, n_new: int, q, out) -> None:
    """a8r_chunk_attn with the split partials in the library's static device array."""
    _check(lib().a8r_chunk_attn_static(handle, layer, b0, nb, n_new, _ptr(q), _ptr(out)))


def rebuild_window(handle: int, layer: int, b0: int, nb: int, n: int, hidden_dim: int, hidden, w_k, w_v) -> None:
    """a8r_rebuild_window: the window re-derived from stored hidden states."""
    _check(lib().a8r_rebuild_window(handle, layer, b0, nb, n, hidden_dim, _ptr(hidden), _ptr(w_k), _ptr(w_v)))


def append_decode_attn(handle: int, layer: int, b0: int, nb: int, k, v, q, out, want_bookkeeping=True):
    """a8r_append_kv (one token per stream) + a8r_decode_attn in one launch."""
    if want_bookkeeping:
        slots = np.empty((nb, 1), dtype=np.int32)
        ev = np.empty((nb, 1), dtype=np.int64)
        _check(lib().a8r_append_decode_attn(handle, layer, b0, nb, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                            slots.ctypes.data_as(_i32p), ev.ctypes.data_as(_i64p)))
        return slots, ev
    _check(lib().a8r_append_decode_attn(handle, layer, b0, nb, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                        None, None))
    return None, None


def append_chunk_attn(handle: int, layer: int, b0: int, nb: int, n_new: int, k, v, q, out, want_bookkeeping=True):
    """a8r_append_kv (n_new tokens per stream) + a8r_chunk_attn in one launch."""
    if want_bookkeeping:
        slots = np.empty((nb, n_new), dtype=np.int32)
        ev = np.empty((nb, n_new), dtype=np.int64)
        _check(lib().a8r_append_chunk_attn(handle, layer, b0, nb, n_new, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                           slots.ctypes.data_as(_i32p), ev.ctypes.data_as(_i64p)))
        return slots, ev
    _check(lib().a8r_append_chunk_attn(handle, layer, b0, nb, n_new, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                       None, None))
    return None, None


def get_state(handle: int, layer: int, b: int) -> tuple[int, int, int]:
    p, n, s = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().a8r_get_state(handle, layer, b, ctypes.byref(p), ctypes.byref(n), ctypes.byref(s)))
    return p.value, n.value, s.value


def read_ring(handle: int, layer: int, b: int, window: int, n_kv_heads: int, head_dim: int, bf16: bool):
    """Raw ring of one pair in physical slot order: (k, v) host arrays [W, Hkv, D]
    (uint16 bf16 bits or float32)."""
    dt = np.uint16 if bf16 else np.float32
    k = np.empty((window, n_kv_heads, head_dim), dtype=dt)
    v = np.empty((window, n_kv_heads, head_dim), dtype=dt)
    _check(lib().a8r_read_ring(handle, layer, b, k.ctypes.data, v.ctypes.data))
    return k, v


class Cache:
    """Object wrapper over one a8r cache handle."""

    def __init__(self, cfg: Config, stream: int | None = None, workspace=None, ws_bytes: int = 0):
        self.cfg = cfg
        self.handle = cache_create(cfg, stream, workspace, ws_bytes)

    def close(self):
        if getattr(self, "handle", None):
            cache_destroy(self.handle)
            self.handle = None

    def __del__(self, _finalizing=sys.is_finalizing):
        # a cache still open when the interpreter shuts down is left to the
        # process exit: the HIP runtime may already be gone, and destroy
        # synchronizes a stream and frees device memory (the check is bound
        # when the class is made: module globals may be gone by then)
        if not getattr(self, "handle", None):
            return
        if _finalizing():
            self.handle = None
            return
        self.close()

    def set_stream(self, stream):
        set_stream(self.handle, stream)

    def reset(self, b0, next_pos, next_slot=None):
        reset(self.handle, b0, next_pos, next_slot)

    def append_kv(self, layer, b0, nb, n_new, k, v, want_bookkeeping=True):
        return append_kv(self.handle, layer, b0, nb, n_new, k, v, want_bookkeeping)

    def decode_attn(self, layer, b0, nb, q, out):
        decode_attn(self.handle, layer, b0, nb, q, out)

    def chunk_attn(self, layer, b0, nb, n_new, q, out):
        chunk_attn(self.handle, layer, b0, nb, n_new, q, out)

    def chunk_attn_static(self, layer, b0, nb, n_new, q, out):
        chunk_attn_static(self.handle, layer, b0, nb, n_new, q, out)

    def rebuild_window(self, layer, b0, nb, n, hidden_dim, hidden, w_k, w_v):
        rebuild_window(self.handle, layer, b0, nb, n, hidden_dim, hidden, w_k, w_v)

    def append_decode_attn(self, layer, b0, nb, k, v, q, out, want_bookkeeping=True):
        return append_decode_attn(self.handle, layer, b0, nb, k, v, q, out, want_bookkeeping)

    def append_chunk_attn(self, layer, b0, nb, n_new, k, v, q, out, want_bookkeeping=True):
        return append_chunk_attn(self.handle, layer, b0, nb, n_new, k, v, q, out, want_bookkeeping)

    def get_state(self, layer, b):
        return get_state(self.handle, layer, b)

    def append_prefix(self, layer, b0, nb, n_new, k, v):
        _check(lib().a8r_append_prefix(self.handle, layer, b0, nb, n_new, _ptr(k), _ptr(v)))

    def export_prefix(self, layer, b0, nb, n, k_out, v_out):
        _check(lib().a8r_export_prefix(self.handle, layer, b0, nb, n, _ptr(k_out), _ptr(v_out)))

    def import_prefix(self, layer, b0, nb, n_new, k, v):
        _check(lib().a8r_import_prefix(self.handle, layer, b0, nb, n_new, _ptr(k), _ptr(v)))

    def clear_prefix(self, b0, nb):
        _check(lib().a8r_clear_prefix(self.handle, b0, nb))

    def prefix_length(self, layer, b):
        f = ctypes.c_int32()
        _check(lib().a8r_prefix_length(self.handle, layer, b, ctypes.byref(f)))
        return f.value

    def read_ring(self, layer, b):
        c = self.cfg
        return read_ring(self.handle, layer, b, c.window, c.n_kv_heads, c.head_dim, c.dtype == A8R_BF16)


class Ledger:
    """Host-only ring bookkeeping (a8r_ledger_*); no device needed."""

    def __init__(self, n_layers: int, n_streams: int, window: int):
        h = _c_void_p()
        _check(lib().a8r_ledger_create(n_layers, n_streams, window, ctypes.byref(h)))
        self.handle = h.value

    def close(self):
        if getattr(self, "handle", None):
            lib().a8r_ledger_destroy(self.handle)
            self.handle = None

    __del__ = close

    def reset(self, b0, next_pos, next_slot=None):
        pos, pos_p = _i64_array(next_pos)
        slot_p = None
        if next_slot is not None:
            slot, slot_p = _i32_array(next_slot)
        _check(lib().a8r_ledger_reset(self.handle, b0, len(pos), pos_p, slot_p))

    def append(self, layer, b0, nb, n_new):
        slots = np.empty((nb, n_new), dtype=np.int32)
        ev = np.empty((nb, n_new), dtype=np.int64)
        _check(lib().a8r_ledger_append(self.handle, layer, b0, nb, n_new,
                                       slots.ctypes.data_as(_i32p), ev.ctypes.data_as(_i64p)))
        return slots, ev

    def get(self, layer, b):
        p, n, s = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().a8r_ledger_get(self.handle, layer, b, ctypes.byref(p), ctypes.byref(n), ctypes.byref(s)))
        return p.value, n.value, s.value
