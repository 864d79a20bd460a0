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
  summation-order error of its own;
* fp16 logits (the pages' F16 data type, rumus project page milestone M11)
  are widened exactly and the expected fp16 gradient is the fp64 gradient
  rounded once to fp16, nearest, ties to even, with fp16's subnormals;
* ``ignore_index`` (not on the pages) follows the common mean-reduction
  convention: a row whose target equals it has loss 0 and a zero gradient
  row, and the other rows are scaled by 1 / (number of rows not ignored)
  instead of 1 / B.

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
    "widen_f16",
    "rne_f16_bits",
    "ce_rows",
    "ce_rows_ignore",
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


def widen_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values: sign,
    5-bit exponent (bias 15) and 10-bit fraction decoded by hand;
    exponent 0 holds the subnormals f * 2^-24, exponent 31 the infinities
    and NaNs."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = np.ldexp(1024.0 + f, np.maximum(e, 1) - 25)      # (1 + f/1024) 2^(e-15)
    val = np.where(e == 0, np.ldexp(f, -24), normal)
    val = np.where(e == 31, np.where(f == 0, np.inf, np.nan), val)
    return sign * val


def rne_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to IEEE binary16 (nearest, ties to even),
    returning uint16 bit patterns.

    binary16 keeps 11 significant bits; for |x| with binary exponent e
    (x = f 2^e, 0.5 <= |f| < 1) the spacing is 2^(e - 11), never finer than
    the subnormal spacing 2^-24.  The quotient by the spacing is an exact
    fp64 scaling and ``np.rint`` rounds half to even.  Results of 65536 or
    more in magnitude (past the largest finite value 65504) become
    infinities.  The rounded value is then encoded by hand."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    q = np.maximum(e - 11, -24)
    r = np.ldexp(np.rint(np.ldexp(xf, -q)), q)
    a = np.abs(r)
    out = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -14
    out = np.where(sub, np.rint(np.ldexp(a, 24)).astype(np.int64), out)
    _, en = np.frexp(np.where(sub | (a == 0), 1.0, a))          # a = fn 2^en, 0.5 <= fn < 1
    frac = np.rint(np.ldexp(np.where(sub, 1.0, a), 11 - en)).astype(np.int64) - 1024
    out = np.where(~sub, ((en - 1 + 15) << 10) | frac, out)
    out = np.where(a >= 65536.0, 0x7C00, out)
    out = np.where(np.isinf(x), 0x7C00, out)
    out = np.where(np.isnan(x), 0x7E00, out)
    neg = np.signbit(np.where(finite, r, x))
    out = np.where(neg, out | 0x8000, out)
    return out.astype(np.uint16)


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


def ce_rows_ignore(z: np.ndarray, t: np.ndarray, ignore_index: int):
    """Per-row loss and gradient of a whole [B, C] problem with rows whose
    target equals ``ignore_index`` left out of the mean: those rows get
    loss 0 and a zero gradient row; every other row is the cross-entropy of
    ``ce_rows`` scaled by 1 / N, N the number of rows not ignored (when
    N = 0 every row is ignored and every output is 0)."""
    z = np.asarray(z, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    ign = t == ignore_index
    N = int((~ign).sum())
    loss = np.zeros(z.shape[0])
    grad = np.zeros(z.shape)
    if N:
        l, g = ce_rows(z[~ign], t[~ign], N)
        loss[~ign] = l
        grad[~ign] = g
    return loss, grad


def ce(logits: np.ndarray, targets: np.ndarray, dtype: str = "f32", rows=None,
       block_elems: int = 1 << 22):
    """Oracle for a whole [B, C] problem, or for the rows listed in ``rows``.

    ``logits`` is float32 [B, C] (dtype "f32") or the uint16 bit patterns of
    bfloat16 or float16 [B, C] (dtype "bf16" or "f16").  Rows are processed
    in blocks of about ``block_elems`` elements to bound memory.  Returns
    fp64 ``(loss_rows, grad)`` for the selected rows.
    """
    B, C = logits.shape
    idx = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    widen = {"f32": lambda a: np.asarray(a, dtype=np.float64), "bf16": widen_bf16,
             "f16": widen_f16}.get(dtype)
    if widen is None:
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
