"""Seeded synthetic inputs for the Muon / SignMuon step.

This module is shared by the CPU oracle, the tests and the benchmark so that
both sides of every parity check see identical inputs.  It draws random
numbers, rounds them to their storage type and describes the workloads; it
holds none of the method's arithmetic (no momentum, normalisation,
Newton-Schulz, sign, vote or update).

Storage conventions
-------------------
* ``"f32"`` arrays are ``numpy.float32``.
* ``"bf16"`` arrays are ``numpy.uint16`` bit patterns (the upper half of the
  IEEE binary32 encoding), produced by round-to-nearest-even from float32.
* A parameter set of several matrices is one flat row-major buffer: matrix j
  occupies ``[offsets[j], offsets[j+1])`` with shape ``shapes[j]``.

Random streams
--------------
Every array is drawn in float64 from ``numpy.random.default_rng`` seeded with
``[cfg, role, worker, step, chunk]``, one stream per chunk of ``CHUNK``
elements of the flat buffer, so chunks can be filled by a thread pool and the
values never depend on the number of threads.  Roles: 0 = W0, 1 = M0,
2 = G, 3 = heavy-column choice.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

CHUNK = 1 << 20

ROLE_W0, ROLE_M0, ROLE_G, ROLE_HEAVY = 0, 1, 2, 3

# Newton-Schulz coefficient sets used by the workloads.
CUBIC = (1.5, -0.5, 0.0)
QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a set of weight matrices and its step settings."""

    cfg: int
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    w_dtype: Optional[str]          # None: no weight update in this workload
    m_dtype: str
    g_dtype: str
    w_dist: Optional[str]
    m0_dist: str                    # "normal" or "zero"
    g_dist: str                     # "normal", "normal_heavy_cols", "student_t3"
    g_scale: float
    w_scale: float
    coeffs: Tuple[float, float, float]
    ns_steps: int
    workers: int
    beta: float = 0.95
    eta: float = 0.02
    precision: str = "bf16"         # NS operand precision: "f32" or "bf16"

    @property
    def offsets(self) -> np.ndarray:
        sizes = [r * c for r, c in self.shapes]
        return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)

    @property
    def numel(self) -> int:
        return int(self.offsets[-1])

    @property
    def alpha(self) -> float:
        return 1.0 - self.beta


def _gpt2_small_shapes() -> Tuple[Tuple[int, int], ...]:
    layer = ((768, 2304), (768, 768), (768, 3072), (3072, 768))
    return tuple(s for _ in range(12) for s in layer)


WORKLOADS = {
    1: Workload(1, "single 256x256 fp32, cubic NS, 3 workers", ((256, 256),),
                "f32", "f32", "f32", "normal", "normal", "normal", 1.0, 1.0,
                CUBIC, 5, 3, precision="f32"),
    2: Workload(2, "GPT-2-small layer set (12 x {QKV, out, up, down}), bf16, 7 workers",
                _gpt2_small_shapes(), "bf16", "bf16", "bf16", "normal", "zero",
                "normal", 0.02, 0.02, QUINTIC, 5, 7),
    3: Workload(3, "128 batched 1024x1024 bf16 momenta, sign+pack only",
                tuple([(1024, 1024)] * 128), None, "bf16", "bf16", None, "zero",
                "normal", 1.0, 1.0, QUINTIC, 5, 1),
    4: Workload(4, "Llama-3-8B MLP 4096x14336 bf16, heavy columns, 7 workers",
                ((4096, 14336),), "bf16", "bf16", "bf16", "normal", "zero",
                "normal_heavy_cols", 1.0, 1.0, QUINTIC, 5, 7),
    5: Workload(5, "dense FFN 7168x18432 bf16, fp32 momentum, Student-t(3), 15 workers",
                ((7168, 18432),), "bf16", "f32", "bf16", "student_t3", "zero",
                "student_t3", 1.0, 1.0, QUINTIC, 5, 15),
}


# Dion workload: the page's d = 768 layer set (GPT-2-small shapes), fp32 state,
# ranks d/4, d/8, d/16.  Roles 0 = W0, 2 = G, 4 = the initial right factor Q0.
ROLE_Q0 = 4


@dataclasses.dataclass(frozen=True)
class DionWorkload:
    cfg: int
    name: str
    shapes: Tuple[Tuple[int, int], ...]
    rank: int
    mu: float = 0.95
    eta: float = 0.02
    g_scale: float = 0.02
    w_scale: float = 0.02

    @property
    def offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([r * c for r, c in self.shapes])]).astype(np.int64)

    @property
    def q_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([c * self.rank for _, c in self.shapes])]).astype(np.int64)

    @property
    def numel(self) -> int:
        return int(self.offsets[-1])


DION_WORKLOADS = {
    r: DionWorkload(100 + r, f"GPT-2-small layer set, fp32, rank {r}", _gpt2_small_shapes(), r)
    for r in (192, 96, 48)
}


def gen_dion(wl: DionWorkload, step: int = 0) -> dict:
    """W0 and G (flat, fp32, N(0, scale^2)) and Q0 (flat, fp32, N(0, 1)): seeded inputs."""
    W0 = store(_draw("normal", wl.numel, [wl.cfg, ROLE_W0, 0, 0]) * wl.w_scale, "f32")
    G = store(_draw("normal", wl.numel, [wl.cfg, ROLE_G, 0, step]) * wl.g_scale, "f32")
    Q0 = store(_draw("normal", int(wl.q_offsets[-1]), [wl.cfg, ROLE_Q0, 0, 0]), "f32")
    return {"W0": W0, "G": G, "Q0": Q0}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to a storage type: float32 first, then bfloat16."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(stored).astype(np.float64)
    raise ValueError(dtype)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(dist: str, n: int, seed: Sequence[int]) -> np.ndarray:
    """Draw ``n`` float64 values of distribution ``dist`` from one chunked stream set."""
    out = np.empty(n, dtype=np.float64)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int) -> None:
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        rng = np.random.default_rng(list(seed) + [c])
        if dist == "normal":
            out[lo:hi] = rng.standard_normal(hi - lo)
        elif dist == "student_t3":
            # Student-t with 3 degrees of freedom has variance 3; scale to 1.
            out[lo:hi] = rng.standard_t(3.0, hi - lo) / np.sqrt(3.0)
        else:
            raise ValueError(dist)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as pool:
            list(pool.map(fill, range(nchunks)))
    return out


def heavy_columns(wl: Workload, j: int = 0) -> np.ndarray:
    """Column indices of matrix ``j`` scaled x10 (1% of its columns, shared by workers)."""
    rows, cols = wl.shapes[j]
    k = int(np.floor(0.01 * cols))
    rng = np.random.default_rng([wl.cfg, ROLE_HEAVY, 0, 0, j])
    return np.sort(rng.choice(cols, size=k, replace=False))


def gen_W0(wl: Workload) -> Optional[np.ndarray]:
    if wl.w_dtype is None:
        return None
    x = _draw(wl.w_dist, wl.numel, [wl.cfg, ROLE_W0, 0, 0]) * wl.w_scale
    return store(x, wl.w_dtype)


def gen_M0(wl: Workload) -> np.ndarray:
    if wl.m0_dist == "zero":
        return store(np.zeros(wl.numel), wl.m_dtype)
    x = _draw(wl.m0_dist, wl.numel, [wl.cfg, ROLE_M0, 0, 0])
    return store(x, wl.m_dtype)


def gen_G(wl: Workload, worker: int, step: int) -> np.ndarray:
    dist = "normal" if wl.g_dist == "normal_heavy_cols" else wl.g_dist
    x = _draw(dist, wl.numel, [wl.cfg, ROLE_G, worker, step]) * wl.g_scale
    if wl.g_dist == "normal_heavy_cols":
        offs = wl.offsets
        for j, (r, c) in enumerate(wl.shapes):
            view = x[offs[j]:offs[j + 1]].reshape(r, c)
            view[:, heavy_columns(wl, j)] *= 10.0
    return store(x, wl.g_dtype)


def small_workload(rows: int, cols: int, *, dtype: str = "bf16", m_dtype: Optional[str] = None,
                   coeffs=QUINTIC, steps: int = 5, workers: int = 3, m0: str = "normal",
                   cfg: int = 100) -> Workload:
    """A one-matrix workload of arbitrary shape for tests (ragged sizes, tails)."""
    return Workload(cfg, f"test {rows}x{cols}", ((rows, cols),), dtype, m_dtype or dtype,
                    dtype, "normal", m0, "normal", 1.0, 1.0, tuple(coeffs), steps, workers,
                    precision="f32" if dtype == "f32" else "bf16")


def random_matrix(shape: Tuple[int, ...], seed: Sequence[int], dist: str = "normal") -> np.ndarray:
    """A float64 array of the given shape from a named seed (test helper)."""
    n = int(np.prod(shape)) if len(shape) else 1
    return _draw(dist, n, list(seed)).reshape(shape)


__all__ = [
    "Workload", "WORKLOADS", "CUBIC", "QUINTIC", "DionWorkload", "DION_WORKLOADS", "gen_dion", "CHUNK", "f32_to_bf16_bits",
    "bf16_bits_to_f32", "store", "to_f64", "gen_W0", "gen_M0", "gen_G", "heavy_columns",
    "small_workload", "random_matrix",
]
