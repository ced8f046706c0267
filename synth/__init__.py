"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method (no rotation, no attention, no
ring bookkeeping): it only draws Q/K/V values and start states, and rounds them
to the storage dtype, so that the oracle and the HIP path can be fed the very
same numbers.  Neither side imports the other through it.

Values are N(0, 1) (unit-variance inputs), drawn in blocks of ``BLOCK``
positions from numpy's PCG64 seeded by
``SeedSequence([0xA8, workload_id, layer, stream, epoch, kind, block])`` so any
position range of any (layer, stream) can be regenerated on its own; ``epoch``
counts resets so a stream that restarts at an old position gets fresh values.
For bf16 workloads the float32 draws are rounded to bf16 with
round-to-nearest-even before either side sees them; both sides receive the same
bf16 bits.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 64
KIND_Q, KIND_K, KIND_V = 0, 1, 2
SEED_ROOT = 0xA8


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Values of x after rounding to bf16, as float32."""
    return bf16_to_f32(bf16_bits(x))


def _block(workload_id: int, layer: int, stream: int, epoch: int, kind: int, block: int,
           n_heads: int, head_dim: int) -> np.ndarray:
    ss = np.random.SeedSequence([SEED_ROOT, workload_id, layer, stream, epoch, kind, block])
    rng = np.random.Generator(np.random.PCG64(ss))
    return rng.standard_normal((BLOCK, n_heads, head_dim), dtype=np.float32)


def draw(workload_id: int, layer: int, stream: int, kind: int, pos0: int, count: int,
         n_heads: int, head_dim: int, bf16: bool, epoch: int = 0) -> np.ndarray:
    """Values for absolute positions [pos0, pos0 + count): float32 [count, H, D].

    For bf16 workloads the returned float32 values are exactly representable in
    bf16 (already rounded).
    """
    if count <= 0:
        return np.zeros((0, n_heads, head_dim), dtype=np.float32)
    b_first, b_last = pos0 // BLOCK, (pos0 + count - 1) // BLOCK
    parts = [_block(workload_id, layer, stream, epoch, kind, b, n_heads, head_dim)
             for b in range(b_first, b_last + 1)]
    arr = np.concatenate(parts, axis=0)
    off = pos0 - b_first * BLOCK
    out = arr[off:off + count]
    return round_bf16(out) if bf16 else np.ascontiguousarray(out)


def to_storage(x: np.ndarray, bf16: bool) -> np.ndarray:
    """Host array in the library's element format: uint16 bf16 bits or float32."""
    return bf16_bits(x) if bf16 else np.ascontiguousarray(x, dtype=np.float32)


def from_storage(x: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_to_f32(x) if bf16 else np.asarray(x, dtype=np.float32)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload shape (a decoder attention stack fed N(0,1) Q/K/V)."""
    workload_id: int
    name: str
    n_layers: int
    n_streams: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    bf16: bool
    steps: int
    chunk: int = 1
    rope_theta: float = 1.0e6
    notes: str = field(default="", compare=False)

    @property
    def element_bytes(self) -> int:
        return 2 if self.bf16 else 4


# The five workloads: a tiny fp32 MHA check, the 0.1B-model decoder shape, the
# 3B-class decoder single-stream and batched, and the 80 ms chunked clock.
WORKLOADS = {
    "tiny_mha_fp32": Workload(0, "tiny_mha_fp32", 1, 1, 8, 8, 64, 64, False, 256,
                              notes="1 layer MHA 8 heads D=64 fp32 W=64, 256 decode steps"),
    "audio8_0p1b": Workload(1, "audio8_0p1b", 8, 1, 8, 8, 64, 1024, True, 8192,
                            notes="8 layers, 8/8 heads, D=64, bf16, W=1024, 8192 steps"),
    "qwen3b_single": Workload(2, "qwen3b_single", 36, 1, 16, 2, 128, 4096, True, 100_000,
                              notes="36 layers, 16/2 heads, D=128, bf16, W=4096, 1e5 steps"),
    "qwen3b_batch64": Workload(3, "qwen3b_batch64", 36, 64, 16, 2, 128, 4096, True, 1000,
                               notes="36 layers, 64 streams, 16/2 heads, D=128, bf16, W=4096"),
    "qwen3b_chunk8": Workload(4, "qwen3b_chunk8", 36, 16, 16, 2, 128, 8192, True, 2000, chunk=8,
                              notes="36 layers, 16 streams, W=8192, 8 positions per clock"),
    # the same stream at 120 ms and 160 ms clocks (12 and 16 new positions per call)
    "qwen3b_chunk12": Workload(5, "qwen3b_chunk12", 36, 16, 16, 2, 128, 8192, True, 1334, chunk=12,
                               notes="36 layers, 16 streams, W=8192, 12 positions per clock"),
    "qwen3b_chunk16": Workload(6, "qwen3b_chunk16", 36, 16, 16, 2, 128, 8192, True, 1000, chunk=16,
                               notes="36 layers, 16 streams, W=8192, 16 positions per clock"),
}


def start_states(workload: Workload) -> tuple[np.ndarray, np.ndarray]:
    """Per-stream (absolute start position P0, ring offset R0), seeded.

    The batched workload draws P0 ~ U[0, 1e6) and R0 ~ U[0, W); the chunked ones
    start every stream just below 2**24 (P0 ~ U[2**24 - W, 2**24)) with R0 = P0
    mod W; the others start at P0 = 0, R0 = 0.
    """
    ss = np.random.SeedSequence([SEED_ROOT, workload.workload_id, 0xFFFFFFFF])
    rng = np.random.Generator(np.random.PCG64(ss))
    n = workload.n_streams
    if workload.name == "qwen3b_batch64":
        p0 = rng.integers(0, 1_000_000, size=n, dtype=np.int64)
        r0 = rng.integers(0, workload.window, size=n, dtype=np.int64)
    elif workload.name.startswith("qwen3b_chunk"):
        p0 = rng.integers(2**24 - workload.window, 2**24, size=n, dtype=np.int64)
        r0 = p0 % workload.window
    else:
        p0 = np.zeros(n, dtype=np.int64)
        r0 = np.zeros(n, dtype=np.int64)
    return p0, r0
