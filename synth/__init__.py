"""Seeded synthetic inputs for the fused softmax cross-entropy path.

This module only draws random numbers: it holds none of the loss or
gradient arithmetic, so the GPU path and the CPU oracle can both consume
its output without sharing any of the method's code.

Workloads (shapes and value distributions of the classifier-head and
LM-head cases the hot path is sized for):

=================  =========  ========  =====  ========================================
name               B          C         dtype  logits
=================  =========  ========  =====  ========================================
tiny               8          10        f32    sigma 1
classifier         1024       1000      f32    sigma 2
skinny             2097152    10        f32    sigma 20 (large-magnitude, short rows)
lmhead50k          4096       50257     f32    sigma 3, one +1e4 spike per row
lmhead128k         8192       128256    bf16   sigma 4 (RNE-rounded from fp32)
=================  =========  ========  =====  ========================================

Targets are int32, uniform in [0, C), independent of the spike column.

Random streams: ``SeedSequence(seed).spawn(3)`` gives, in this order, the
stream for the targets, the stream for the logits and the stream for the
spike columns.  The logits stream is split further into one child per row
block of ``_BLOCK_ELEMS`` elements, so blocks can be drawn in parallel
threads and any block can be re-drawn on its own; the result does not depend
on the number of threads.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_inputs", "make_workload",
           "spike_columns", "bf16_bits_from_f32", "f16_bits_from_f32", "grid_logits",
           "simplex_rows"]

_BLOCK_ELEMS = 1 << 23  # about 8M logits per independently seeded block


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    dtype: str          # "f32" or "bf16"
    sigma: float
    spike: float | None = None   # value written at one uniform column per row

    @property
    def in_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def describe(self) -> dict:
        d = {"workload": self.name, "B": self.B, "C": self.C, "dtype": self.dtype,
             "logits": f"N(0,{self.sigma:g})"}
        if self.spike is not None:
            d["logits"] += f" + one {self.spike:g} per row"
        return d


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny", 8, 10, "f32", 1.0),
        Workload("classifier", 1024, 1000, "f32", 2.0),
        Workload("skinny", 2_097_152, 10, "f32", 20.0),
        Workload("lmhead50k", 4096, 50257, "f32", 3.0, spike=1.0e4),
        Workload("lmhead128k", 8192, 128256, "bf16", 4.0),
    )
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even) and return the
    16-bit patterns as uint16.  Uses torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE binary16 (nearest, ties to even, with
    subnormals) and return the 16-bit patterns as uint16."""
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(x) if dtype == "bf16" else f16_bits_from_f32(x)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_inputs(B: int, C: int, dtype: str = "f32", sigma: float = 1.0,
                spike: float | None = None, seed: int = 0):
    """Draw ``(logits, targets)`` for a ``[B, C]`` problem.

    ``logits`` is float32 ``[B, C]`` for dtype "f32" and the uint16 bit
    pattern of bfloat16 or float16 values ``[B, C]`` for dtype "bf16" or
    "f16" (the float32 draw rounded to nearest even); ``targets`` is int32
    ``[B]`` uniform in ``[0, C)``.
    """
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    ss_t, ss_z, ss_s = np.random.SeedSequence(seed).spawn(3)
    targets = np.random.Generator(np.random.PCG64(ss_t)).integers(
        0, C, size=B, dtype=np.int32) if C > 0 else np.zeros(B, np.int32)

    n = B * C
    nblocks = max(1, -(-n // _BLOCK_ELEMS))
    children = ss_z.spawn(nblocks)
    flat32 = np.empty(n, dtype=np.float32)
    out = flat32 if dtype == "f32" else np.empty(n, dtype=np.uint16)

    def fill(i: int) -> None:
        lo = i * _BLOCK_ELEMS
        hi = min(n, lo + _BLOCK_ELEMS)
        if hi <= lo:
            return
        g = np.random.Generator(np.random.PCG64(children[i]))
        seg = flat32[lo:hi]
        g.standard_normal(out=seg, dtype=np.float32)
        seg *= np.float32(sigma)
        if spike is not None:
            pass  # spikes are placed after all blocks are drawn
        if dtype != "f32" and spike is None:
            out[lo:hi] = _to_bits(seg, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblocks)))

    if spike is not None:
        cols = np.random.Generator(np.random.PCG64(ss_s)).integers(
            0, C, size=B, dtype=np.int64)
        flat32.reshape(B, C)[np.arange(B), cols] = np.float32(spike)
        if dtype != "f32":
            out[:] = _to_bits(flat32, dtype)
    logits = out.reshape(B, C)
    return logits, targets


def make_workload(name: str, seed: int = 0):
    w = WORKLOADS[name]
    return make_inputs(w.B, w.C, w.dtype, w.sigma, w.spike, seed)


def spike_columns(B: int, C: int, seed: int = 0) -> np.ndarray:
    """The column of each row that ``make_inputs(..., spike=v)`` overwrote."""
    _, _, ss_s = np.random.SeedSequence(seed).spawn(3)
    return np.random.Generator(np.random.PCG64(ss_s)).integers(0, C, size=B, dtype=np.int64)


def grid_logits(B: int, C: int, step: float, lim: float, seed: int = 0) -> np.ndarray:
    """float32 logits on the grid ``step * k`` with ``|value| <= lim``: every
    sum and difference of two such values (and of a small integer shift) is
    exact in fp32, which makes shift-invariance checks bit-exact."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    k = g.integers(-int(lim / step), int(lim / step) + 1, size=(B, C))
    return (k * step).astype(np.float32)


def simplex_rows(B: int, C: int, dtype: str = "f32", seed: int = 0) -> np.ndarray:
    """Rows on the probability simplex, to stand in for a softmax's output:
    one Dirichlet(1, ..., 1) draw per row (independent standard exponentials
    divided by their row sum in float64), then rounded to float32 or to
    bfloat16 (returned as uint16 bit patterns).  Drawn in independently
    seeded row blocks, like ``make_inputs``."""
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rows_per = max(1, _BLOCK_ELEMS // max(C, 1))
    nblocks = max(1, -(-B // rows_per))
    children = np.random.SeedSequence(seed).spawn(nblocks)
    out = np.empty((B, C), dtype=np.float32 if dtype == "f32" else np.uint16)

    def fill(i: int) -> None:
        lo, hi = i * rows_per, min(B, (i + 1) * rows_per)
        if hi <= lo:
            return
        w = np.random.Generator(np.random.PCG64(children[i])).standard_exponential((hi - lo, C))
        y = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
        out[lo:hi] = y if dtype == "f32" else _to_bits(y, dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblocks)))
    return out
