"""Seeded input tensors for a workload.

Tensors are float32 normals scaled by the workload's std. Tensor t of the fixed
order Q, K, V, Qb, Kb, Vb, dO, dOb is cut into chunks of 2^22 elements; chunk c
is drawn from its own generator, ``default_rng(SeedSequence([seed, t, c]))``, so
chunks can be drawn in parallel and the values do not depend on the thread count.
bf16 workloads round them to bf16 with round-to-nearest-even and keep the raw
16-bit patterns (``uint16``); the float32 view of those patterns is exact, so
the oracle and the GPU see bit-identical values.

Layouts (row-major, head_dim contiguous):
  q, do   [Nq, Hq, d]     k, v    [N, Hkv, d]
  qb, dob [Rb, Hq, d]     kb, vb  [Rb, Hkv, d]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from typing import Dict

import numpy as np

from .configs import Workload

_CHUNK = 1 << 22  # elements per independently seeded chunk
_ORDER = ["q", "k", "v", "qb", "kb", "vb", "do", "dob"]


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def shapes(w: Workload) -> Dict[str, tuple]:
    hq, hkv, d = w.num_q_heads, w.num_kv_heads, w.head_dim
    return {
        "q": (w.Nq, hq, d), "k": (w.N, hkv, d), "v": (w.N, hkv, d),
        "qb": (w.Rb, hq, d), "kb": (w.Rb, hkv, d), "vb": (w.Rb, hkv, d),
        "do": (w.Nq, hq, d), "dob": (w.Rb, hq, d),
    }


def _draw(seed: int, tidx: int, shape: tuple, std: float, dtype: str, pool) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def one(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, tidx, c]))
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[lo:hi] = bf16_round_bits(x) if dtype == "bf16" else x

    list(pool.map(one, range((n + _CHUNK - 1) // _CHUNK)))
    return out.reshape(shape)


def make_inputs(w: Workload, grads: bool = False, threads: int = 0) -> Dict[str, np.ndarray]:
    """Seeded tensors for ``w``: bf16 bit patterns (uint16) or float32 arrays."""
    sh = shapes(w)
    names = _ORDER if grads else _ORDER[:6]
    threads = threads or min(16, len(os.sched_getaffinity(0)))
    out = {}
    with cf.ThreadPoolExecutor(max_workers=threads) as pool:
        for nm in names:
            std = w.grad_std if nm in ("do", "dob") else w.std
            out[nm] = _draw(w.seed, _ORDER.index(nm), sh[nm], std, w.dtype, pool)
    return out


def to_f32(x: np.ndarray) -> np.ndarray:
    """Exact float32 values of a tensor produced by ``make_inputs``."""
    return bf16_bits_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)
