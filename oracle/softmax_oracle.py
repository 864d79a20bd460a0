"""Plain fp64 CPU oracle for row-wise softmax (forward and backward) and for
cross-entropy over a vocabulary split into column shards.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never imports, calls or falls back to it, and this module imports
nothing from the product path.

Row-wise softmax
----------------
rumus project page, milestone M8c ("BMM, Softmax & SDPA") and the feature
table's Softmax row: a row-wise softmax made stable with the log-sum-exp
trick, with a forward and a backward kernel.  For a row z of C values::

    m   = max_c z_c
    s   = sum_c exp(z_c - m)
    y_c = exp(z_c - m) / s               forward
    lse = m + ln s                       the row's log-sum-exp

The pages give no formula for the backward.  Reading taken: the backward is
the vector-Jacobian product of the forward, written with the forward's
output y (what a backward kernel has at hand) and the upstream gradient dy.
Since dy_j/dz_c = y_j ([j == c] - y_c)::

    dz_c = y_c (dy_c - sum_j dy_j y_j)

Vocabulary shards
-----------------
rumus project page, milestone M24 (3D parallelism): a column-parallel linear
layer splits its weight along the output features, so an LM head split that
way leaves each rank the logits of a contiguous range of classes.  The
pages stop there; the cross-entropy over such shards is derived from the
definition (rumus 0.1.1 ``cross_entropy.wgsl``, pass 1 steps 1-4).  For
shard k holding columns [col0_k, col0_k + C_k) of row b::

    m_k  = max over the shard's columns of z_c
    sx_k = sum over the shard's columns c != t of exp(z_c - m_k)
    zt_k = z_t if the shard holds t, else 0

and the row's values follow from the N shard records in shard order::

    m  = max_k m_k
    sx = sum_k sx_k exp(m_k - m)          (the row's sum without the target)
    zt = sum_k zt_k                       (one shard holds the target)
    S  = sx + exp(zt - m)
    loss = (ln S + m - zt) / B,   grad_c = (exp(z_c - m) / S - [c == t]) / B

which is the single-row cross-entropy of the whole row, because the max and
the sum of exponentials of a union of column sets are the max of the maxes
and the rescaled sum of the sums.

Pinned by ``tests/test_oracle_softmax_pins.py``.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "softmax_rows",
    "softmax_bwd_rows",
    "shard_partials",
    "combine_partials",
]


def softmax_rows(z: np.ndarray):
    """Row-wise softmax of a [n, C] block in float64.

    Returns ``(y [n, C], lse [n])``: the softmax of every row and the row's
    log-sum-exp m + ln s."""
    z = np.asarray(z, dtype=np.float64)
    if z.ndim != 2 or z.shape[1] <= 0:
        raise ValueError("z must be [n, C] with C >= 1")
    m = z.max(axis=1)                             # row max
    e = np.exp(z - m[:, None])                    # exp(z - m)
    s = e.sum(axis=1)                             # sum of exponentials
    y = e / s[:, None]                            # softmax
    lse = m + np.log(s)                           # log-sum-exp
    return y, lse


def softmax_bwd_rows(y: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """Backward of the row-wise softmax in float64: from the forward's output
    y and the upstream gradient dy (both [n, C]), dz = y * (dy - <dy, y>)."""
    y = np.asarray(y, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    if y.shape != dy.shape or y.ndim != 2:
        raise ValueError("y and dy must both be [n, C]")
    dot = (dy * y).sum(axis=1)                    # <dy, y> per row
    return y * (dy - dot[:, None])


def shard_partials(z_shard: np.ndarray, t: np.ndarray, col0: int):
    """One shard's per-row record in float64.

    ``z_shard`` is [n, C_k], the columns [col0, col0 + C_k) of each row;
    ``t`` holds the rows' global target classes.  Returns
    ``(m_k, sx_k, zt_k, owns)``: the shard's max, its sum of exp(z - m_k)
    with the target left out, the target logit where the shard holds it
    (0 elsewhere), and whether it does."""
    z = np.asarray(z_shard, dtype=np.float64)
    t = np.asarray(t, dtype=np.int64)
    n, Ck = z.shape
    if Ck <= 0:
        raise ValueError("a shard holds at least one column")
    local = t - col0
    owns = (local >= 0) & (local < Ck)
    rows = np.arange(n)
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    lc = np.where(owns, local, 0)
    e[rows[owns], lc[owns]] = 0.0                 # the target stays out of the sum
    sx = e.sum(axis=1)
    zt = np.where(owns, z[rows, lc], 0.0)
    return m, sx, zt, owns


def combine_partials(records, t: np.ndarray, C: int, B: int):
    """Combine the shard records (a list, in shard order, of the tuples
    ``shard_partials`` returns) into the rows' (m, S, zt, loss) in float64.

    ``C`` is the whole row's length, for the target's validity; ``B`` the
    batch of the 1/B scale.  A target outside [0, C) gives a NaN loss."""
    t = np.asarray(t, dtype=np.int64)
    m = np.max(np.stack([r[0] for r in records]), axis=0)
    sx = np.zeros_like(m)
    zt = np.zeros_like(m)
    for mk, sxk, ztk, _ in records:               # shard order
        sx = sx + sxk * np.exp(mk - m)
        zt = zt + ztk
    S = sx + np.exp(zt - m)
    valid = (t >= 0) & (t < C)
    loss = np.where(valid, (np.log(S) + (m - zt)) / B, np.nan)
    return m, S, zt, loss
