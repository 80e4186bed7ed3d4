"""Seeded synthetic inputs for the row-typed Q_q projection.

This module only draws numbers and encodes them; it holds none of the
projection's arithmetic.  Both the GPU path's callers (tests, bench) and the
fp64 oracle's callers take their inputs from here, so the two sides see the
same bits.

Recipe (all inputs synthetic; the paper's kernel study also used synthetic
BF16 tensors at public model shapes, section 7.1 "Kernel Scaling on
Transformer Shapes"):

* X ~ N(0, 1), W ~ N(0, 1/K) (std K^-1/2), dY ~ N(0, 1), drawn in float64 by
  numpy's PCG64 generator, then rounded float64 -> float32 (round to nearest
  even) and, for bf16 operands, float32 -> bf16 (round to nearest even).
* Seeds: 1000*c + {1: X, 2: W, 3: dY, 4: positions} for workload c; per-expert
  weights of a batched workload use 1000*c + 100 + e, positions 1000*c + 200 + e.
* Positions: cyclic 0..M-1 (optionally restarting every `seq_len`, optionally
  with an offset), or absolute positions drawn uniformly from {0..P-1}.

Every array comes back twice: the storage bits the device consumes
(float32 or uint16 bf16 patterns) and the exact float64 value of those bits.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f64_from_bf16_bits",
    "Operand",
    "normal_operand",
    "cyclic_positions",
    "random_positions",
    "seed_for",
]


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # u + 0x7FFF + lsb cannot wrap for a non-NaN float32 (largest: -inf + 0x7FFF)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f64_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


class Operand:
    """A synthetic operand: `bits` is what goes to the device, `f64` its exact value."""

    __slots__ = ("bits", "dtype", "_f64")

    def __init__(self, bits: np.ndarray, dtype: str):
        self.bits = bits
        self.dtype = dtype
        self._f64 = None

    @property
    def f64(self) -> np.ndarray:
        """Exact float64 value of the stored bits (computed on first use)."""
        if self._f64 is None:
            if self.dtype == "bf16":
                self._f64 = f64_from_bf16_bits(self.bits)
            else:
                self._f64 = self.bits.astype(np.float64)
        return self._f64

    @property
    def shape(self):
        return self.bits.shape


_CHUNK = 1 << 23  # values drawn per step; the stream is the same as one big draw


def normal_operand(seed: int, shape, std: float, dtype: str) -> Operand:
    """Draw N(0, std^2) in float64, round to float32, then (for bf16) to bf16."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    g = np.random.Generator(np.random.PCG64(seed))
    shape = tuple(int(x) for x in np.atleast_1d(shape)) if not isinstance(shape, int) else (shape,)
    n = int(np.prod(shape, dtype=np.int64))
    bits = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        v = g.standard_normal(size=hi - lo)
        v *= std
        f32 = v.astype(np.float32)
        bits[lo:hi] = bf16_bits_from_f32(f32) if dtype == "bf16" else f32
    return Operand(bits.reshape(shape), dtype)


def cyclic_positions(M: int, seq_len: int | None = None, offset: int = 0) -> np.ndarray:
    """Positions of M token rows laid out as packed sequences of `seq_len` (default: one sequence)."""
    m = np.arange(M, dtype=np.int64)
    if seq_len:
        m = m % seq_len
    return m + offset


def random_positions(seed: int, M: int, P: int = 4096) -> np.ndarray:
    """M absolute positions drawn i.i.d. uniformly from {0, ..., P-1}."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(0, P, size=M, dtype=np.int64)


def seed_for(workload: int, what: str, expert: int | None = None) -> int:
    """Seed layout: 1000*c + {X:1, W:2, dY:3, pos:4}; per-expert W / pos: +100+e / +200+e."""
    base = 1000 * workload
    if expert is not None:
        if what == "W":
            return base + 100 + expert
        if what == "pos":
            return base + 200 + expert
        if what == "X":
            return base + 300 + expert
        raise ValueError(what)
    return base + {"X": 1, "W": 2, "dY": 3, "pos": 4}[what]
