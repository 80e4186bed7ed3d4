"""Shared GPU-test plumbing: seeded inputs to the device, results back to float64."""
from __future__ import annotations

import sys

import numpy as np

import synth


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch


def to_dev(op: synth.Operand):
    torch = torch_cuda()
    if op.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(op.bits).view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(op.bits)).to("cuda")


def to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def tau_dev(tau: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(tau, dtype=np.int32)).to("cuda")


def make_tau(kind: str, M: int, q: int, seed: int = 0, offset: int = 0, bad: int = 0) -> np.ndarray:
    """Types for a test: 'cyclic' ((m + offset) mod q), 'random', or 'absent' (random without type 1);
    `bad` rows get out-of-range types."""
    if kind == "cyclic":
        tau = ((np.arange(M) + offset) % q).astype(np.int32)
    elif kind == "random":
        g = np.random.Generator(np.random.PCG64(seed))
        tau = g.integers(0, q, size=M).astype(np.int32)
    elif kind == "absent":
        g = np.random.Generator(np.random.PCG64(seed))
        tau = g.integers(0, q - 1, size=M).astype(np.int32)
        tau[tau >= 1] += 1
    elif kind == "zeros":
        tau = np.zeros(M, np.int32)
    else:
        raise ValueError(kind)
    if bad:
        g = np.random.Generator(np.random.PCG64(seed + 1))
        idx = g.choice(M, size=min(bad, M), replace=False)
        tau[idx] = np.where(g.random(idx.size) < 0.5, -1, q + 3)
    return tau


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def merge_perm(F: int, q: int) -> np.ndarray:
    """Column map of the merged gate/up layout (include/qalg.h): merged column k holds column
    perm[k] of the concatenation [gate | up] (up columns offset by F)."""
    r = F // q
    perm = np.empty(2 * F, dtype=np.int64)
    for j in range(q):
        for t in range(r // 128):
            c0, base = j * r + 128 * t, j * 2 * r + 256 * t
            perm[base:base + 64] = np.arange(c0, c0 + 64)
            perm[base + 64:base + 128] = F + np.arange(c0, c0 + 64)
            perm[base + 128:base + 192] = np.arange(c0 + 64, c0 + 128)
            perm[base + 192:base + 256] = F + np.arange(c0 + 64, c0 + 128)
    return perm
