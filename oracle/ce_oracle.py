"""Plain fp64 CPU oracle for fused softmax cross-entropy.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never imports, calls or falls
back to it, and this module imports nothing from the product path.

What it computes
----------------
The definition of the method, written out in float64 on the exact input
values.  The method is stated on two pages:

* rumus project page, milestone M7a "Loss Functions & GPU Optimizers":
  cross-entropy fused on the GPU with the log-sum-exp trick (a max and a
  sum of exponentials reduced per row), the gradient formed during the
  forward pass, and the loss reduced to one scalar for a 4-byte read-back
  (milestone M7b).
* rumus 0.1.1 source view of ``cross_entropy.wgsl``, pass 1 (forward and
  gradient: step 1 row max, step 2 sum of exp(z - max), step 3 per-row loss
  scaled by 1/B, step 4 gradient softmax minus one-hot scaled by 1/B) and
  pass 2 (the per-row losses summed into one scalar).

For each row b of a [B, C] logit matrix z with target class t_b::

    m_b    = max_c z[b, c]
    s_b    = sum_c exp(z[b, c] - m_b)                (1 <= s_b <= C)
    l_b    = (ln s_b + (m_b - z[b, t_b])) / B        per-row loss
    g[b,c] = (exp(z[b, c] - m_b) / s_b - [c == t_b]) / B
    L      = sum_b l_b                               the batch-mean loss

Readings where the pages are silent (each is listed in the design doc):

* targets are int32 class indices (the WGSL page passes them as f32);
* a target outside [0, C) makes that row's loss and its whole gradient row
  NaN (the WGSL page does not guard it);
* bf16 logits are widened exactly (bits << 16 -> fp32 -> fp64); the expected
  bf16 gradient is the fp64 gradient rounded once to bf16, nearest, ties to
  even (the Haelixe page's "BF16 storage, F32 compute" boundary);
* the scalar is the exactly rounded sum (``math.fsum``), so it carries no
  summation-order error of its own.

Pinned by ``tests/test_oracle_pins.py`` (closed forms, special cases,
invariants, finite differences, library cross-checks, planted-mistake
mutants).  The exact fp32/bf16 bits a GPU produces are not unique and are
not pinned; the oracle's own values are.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen_bf16",
    "rne_bf16_bits",
    "ce_rows",
    "ce",
    "reduce_loss",
]


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    A bf16 value is the fp32 value whose upper 16 bits are the pattern and
    whose lower 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to bfloat16 (nearest, ties to even).

    bf16 keeps 8 significant bits and fp32's exponent range.  For a value
    with binary exponent e (x = f * 2**e, 0.5 <= |f| < 1) the spacing of bf16
    values is 2**(e - 8), never finer than the subnormal spacing 2**-133.
    Scaling by a power of two is exact in fp64, and ``np.rint`` rounds half
    to even, so the quotient is rounded exactly once.  Results beyond the
    largest finite bf16 become infinities.  Returns uint16 bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    out[...] = np.where(finite, r, x)
    big = np.abs(out) >= 2.0 ** 128 * (1 - 2.0 ** -9)  # rounds past max bf16
    out = np.where(big & finite, np.copysign(np.inf, out), out)
    with np.errstate(over="ignore"):
        f32 = out.astype(np.float32)
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def ce_rows(z: np.ndarray, t: np.ndarray, B: int):
    """Per-row loss and gradient for a block of rows, in float64.

    ``z`` is [n, C] float64, ``t`` is [n] integer class indices and ``B`` is
    the batch size of the whole problem (the 1/B scale of the batch mean).
    Returns ``(loss_rows [n], grad [n, C])``, both already scaled by 1/B.
    """
    z = np.asarray(z, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    n, C = z.shape
    if C <= 0 or B <= 0:
        raise ValueError("B and C must be positive")
    valid = (t >= 0) & (t < C)
    tc = np.where(valid, t, 0)
    rows = np.arange(n)

    m = z.max(axis=1)                             # row max
    e = np.exp(z - m[:, None])                    # exp(z - m)
    s = e.sum(axis=1)                             # sum of exponentials
    zt = z[rows, tc]                              # target logit
    loss = (np.log(s) + (m - zt)) / B             # (lse - z_t) / B

    grad = e / s[:, None]                         # softmax
    grad[rows, tc] -= 1.0                         # minus one-hot
    grad /= B                                     # batch-mean scale

    loss = np.where(valid, loss, np.nan)
    grad[~valid, :] = np.nan
    return loss, grad


def ce(logits: np.ndarray, targets: np.ndarray, dtype: str = "f32", rows=None,
       block_elems: int = 1 << 22):
    """Oracle for a whole [B, C] problem, or for the rows listed in ``rows``.

    ``logits`` is float32 [B, C] (dtype "f32") or the uint16 bit patterns of
    bfloat16 [B, C] (dtype "bf16").  Rows are processed in blocks of about
    ``block_elems`` elements to bound memory.  Returns fp64
    ``(loss_rows, grad)`` for the selected rows.
    """
    B, C = logits.shape
    idx = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    widen = (lambda a: np.asarray(a, dtype=np.float64)) if dtype == "f32" else widen_bf16
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    loss = np.empty(idx.size, dtype=np.float64)
    grad = np.empty((idx.size, C), dtype=np.float64)
    step = max(1, block_elems // max(C, 1))
    for lo in range(0, idx.size, step):
        sel = idx[lo:lo + step]
        l, g = ce_rows(widen(logits[sel]), targets[sel], B)
        loss[lo:lo + step] = l
        grad[lo:lo + step] = g
    return loss, grad


def reduce_loss(loss_rows) -> float:
    """The batch-mean loss: the exactly rounded sum of the per-row losses
    (which already carry the 1/B scale)."""
    return math.fsum(np.asarray(loss_rows, dtype=np.float64).tolist())
