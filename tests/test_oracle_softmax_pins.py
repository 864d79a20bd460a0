"""Pins for the fp64 oracle of row-wise softmax (forward and backward) and of
cross-entropy over vocabulary shards: facts fixed by the mathematics or by
library routines, not by the oracle's own code.

The real oracle must pass every pin; each planted mistake (a mutant of the
oracle, built in this file on the CPU) must fail at least one.

Definitions pinned here: rumus project page, milestone M8c and the feature
table's Softmax row (row-wise log-sum-exp softmax, forward and backward
kernels); rumus project page, milestone M24 (column-parallel layers, which
leave each rank a contiguous range of classes) with the cross-entropy of
rumus 0.1.1 ``cross_entropy.wgsl`` pass 1 taken over such ranges.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import ce_rows, combine_partials, shard_partials, softmax_bwd_rows, softmax_rows


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# forward pins: f(z) -> (y, lse)
# --------------------------------------------------------------------------

def fpin_uniform(f):
    """Equal logits: y = 1/C and lse = v + ln C."""
    for C in (1, 2, 7, 1000):
        for v in (0.0, -3.5, 1e4, -1e4):
            y, lse = f(np.full((3, C), v))
            np.testing.assert_allclose(y, 1.0 / C, rtol=1e-14, atol=0)
            np.testing.assert_allclose(lse, v + math.log(C), rtol=1e-14, atol=1e-14)


def fpin_worked(f):
    """z = (0, ln 2, ln 3): y = (1/6, 2/6, 3/6), lse = ln 6; z = (ln a_c) in
    general gives y_c = a_c / sum a."""
    y, lse = f(np.array([[0.0, math.log(2.0), math.log(3.0)]]))
    np.testing.assert_allclose(y[0], [1 / 6, 2 / 6, 3 / 6], rtol=1e-14)
    assert math.isclose(lse[0], math.log(6.0), rel_tol=1e-14)
    a = np.arange(1.0, 41.0)
    y, lse = f(np.log(a)[None, :])
    np.testing.assert_allclose(y[0], a / a.sum(), rtol=1e-13)
    assert math.isclose(lse[0], math.log(a.sum()), rel_tol=1e-14)


def fpin_two_class(f):
    """C = 2: y_0 = sigmoid(z_0 - z_1) and lse = max + ln(1 + e^-|d|)."""
    rng = _rng(21)
    z = rng.standard_normal((50, 2)) * 8
    y, lse = f(z)
    for b in range(50):
        d = z[b, 0] - z[b, 1]
        sig = 1.0 / (1.0 + math.exp(-d)) if d >= 0 else math.exp(d) / (1.0 + math.exp(d))
        assert math.isclose(y[b, 0], sig, rel_tol=1e-13, abs_tol=1e-300)
        assert math.isclose(y[b, 1], 1.0 - sig, rel_tol=1e-12, abs_tol=1e-16)
        want = max(z[b]) + math.log1p(math.exp(-abs(d)))
        assert math.isclose(lse[b], want, rel_tol=1e-14, abs_tol=1e-14)


def fpin_shift(f):
    """A constant added to a row leaves y alone and moves lse by it."""
    rng = _rng(22)
    z = rng.standard_normal((6, 29)) * 4
    y0, l0 = f(z)
    for k in (-500.0, 0.25, 77.0):
        y1, l1 = f(z + k)
        np.testing.assert_allclose(y1, y0, rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(l1, l0 + k, rtol=1e-13, atol=1e-11)


def fpin_bounds(f):
    """Rows sum to 1, 0 <= y <= 1, and max <= lse <= max + ln C."""
    rng = _rng(23)
    for C in (1, 3, 500):
        z = rng.standard_normal((40, C)) * 5
        y, lse = f(z)
        assert np.abs(y.sum(axis=1) - 1.0).max() <= 1e-14
        assert (y >= 0).all() and (y <= 1).all()
        m = z.max(axis=1)
        assert (lse >= m - 1e-12).all() and (lse <= m + math.log(C) + 1e-12).all()


def fpin_extreme(f):
    """Rows at +-1e4 and one spike: finite, and a spike of 1e4 over N(0, 3)
    takes all the mass (the others' exp(z - 1e4) vanish)."""
    z = np.array([[1e4] * 5, [-1e4] * 5, [-1e4, 1e4, -1e4, 1e4, 0.0], [0.0, 1.0, 1e4, 2.0, -3.0]])
    y, lse = f(z)
    assert np.isfinite(y).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(y[2], [0, 0.5, 0, 0.5, 0], atol=1e-300)
    assert math.isclose(lse[2], 1e4 + math.log(2.0), rel_tol=1e-15)
    np.testing.assert_array_equal(y[3], [0, 0, 1, 0, 0])
    assert lse[3] == 1e4


def fpin_lse_gradient(f):
    """The gradient of lse is the softmax: central differences of lse
    (step 1e-6) agree with y to 1e-8."""
    rng = _rng(24)
    z = rng.standard_normal((3, 6)) * 2
    y, _ = f(z)
    h = 1e-6
    for b in range(3):
        for c in range(6):
            zp, zm = z.copy(), z.copy()
            zp[b, c] += h
            zm[b, c] -= h
            fd = (f(zp)[1][b] - f(zm)[1][b]) / (2 * h)
            assert abs(fd - y[b, c]) <= 1e-8


def fpin_permutation(f):
    """Permuting the columns permutes y; lse is unchanged."""
    rng = _rng(25)
    z = rng.standard_normal((5, 17)) * 3
    y0, l0 = f(z)
    p = rng.permutation(17)
    y1, l1 = f(z[:, p])
    np.testing.assert_allclose(y1, y0[:, p], rtol=1e-14)
    np.testing.assert_allclose(l1, l0, rtol=1e-15)


def fpin_scipy(f):
    """Library cross-check: scipy.special.softmax and logsumexp."""
    from scipy.special import logsumexp, softmax
    rng = _rng(26)
    for C in (2, 64, 3001):
        z = rng.standard_normal((12, C)) * 4
        y, lse = f(z)
        np.testing.assert_allclose(y, softmax(z, axis=1), rtol=1e-12, atol=1e-300)
        np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-14)


def fpin_torch(f):
    """Library cross-check: torch.softmax and torch.logsumexp in float64 on
    the CPU."""
    import torch
    rng = _rng(27)
    z = rng.standard_normal((9, 333)) * 6
    y, lse = f(z)
    zt = torch.from_numpy(z)
    np.testing.assert_allclose(y, torch.softmax(zt, dim=1).numpy(), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse, torch.logsumexp(zt, dim=1).numpy(), rtol=1e-14)


FWD_PINS = [fpin_uniform, fpin_worked, fpin_two_class, fpin_shift, fpin_bounds, fpin_extreme,
            fpin_lse_gradient, fpin_permutation, fpin_scipy, fpin_torch]


@pytest.mark.parametrize("pin", FWD_PINS, ids=lambda p: p.__name__)
def test_softmax_oracle_meets_pin(pin):
    pin(softmax_rows)


def _fwd_mutant(kind):
    def f(z):
        z = np.asarray(z, dtype=np.float64)
        if kind == "global_max":
            m = np.full(z.shape[0], z.max())
        else:
            m = z.max(axis=1)
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            e = np.exp(z) if kind == "no_max_shift" else np.exp(z - m[:, None])
            s = e.sum(axis=0) if kind == "transposed_norm" else e.sum(axis=1)
            y = e / (s[None, :] if kind == "transposed_norm" else s[:, None])
            if kind == "transposed_norm":
                s = e.sum(axis=1)
            if kind == "no_max_shift":
                lse = np.log(s)
            elif kind == "lse_drops_max":
                lse = np.log(s)
            elif kind == "lse_log2":
                lse = m + np.log2(s)
            else:
                lse = m + np.log(s)
        return y, lse
    f.__name__ = f"fwd_mutant_{kind}"
    return f


FWD_MUTANTS = ["global_max", "no_max_shift", "transposed_norm", "lse_drops_max", "lse_log2"]


def _caught(pins, f):
    hits = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(f)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            hits.append(pin.__name__)
    return hits


@pytest.mark.parametrize("kind", FWD_MUTANTS)
def test_softmax_planted_mistake_is_caught(kind):
    assert _caught(FWD_PINS, _fwd_mutant(kind)), f"no pin catches forward mutant {kind}"


def test_softmax_mutant_scaffold_passes():
    assert _caught(FWD_PINS, _fwd_mutant("none")) == []


# --------------------------------------------------------------------------
# backward pins: g(y, dy) -> dz
# --------------------------------------------------------------------------

def _scipy_softmax(z):
    from scipy.special import softmax
    return softmax(z, axis=1)


def bpin_finite_difference(g):
    """dz is dL/dz for L(z) = sum dy * softmax(z) (softmax from scipy):
    central differences (step 1e-6) agree to 1e-8."""
    rng = _rng(31)
    for n, C in ((1, 1), (2, 3), (3, 8)):
        z = rng.standard_normal((n, C)) * 2
        dy = rng.standard_normal((n, C))
        dz = g(_scipy_softmax(z), dy)
        h = 1e-6
        for b in range(n):
            for c in range(C):
                zp, zm = z.copy(), z.copy()
                zp[b, c] += h
                zm[b, c] -= h
                fd = ((dy * _scipy_softmax(zp)).sum() - (dy * _scipy_softmax(zm)).sum()) / (2 * h)
                assert abs(fd - dz[b, c]) <= 1e-8, (n, C, b, c)


def bpin_jacobian(g):
    """Brute force: dz_c = sum_j dy_j J[j, c] with the Jacobian entries
    J[j, c] = y_j ([j == c] - y_c) summed by explicit loops."""
    rng = _rng(32)
    z = rng.standard_normal((2, 5)) * 3
    y = _scipy_softmax(z)
    dy = rng.standard_normal((2, 5))
    dz = g(y, dy)
    for b in range(2):
        for c in range(5):
            acc = 0.0
            for j in range(5):
                acc += dy[b, j] * y[b, j] * ((1.0 if j == c else 0.0) - y[b, c])
            assert math.isclose(dz[b, c], acc, rel_tol=1e-12, abs_tol=1e-15)


def bpin_invariants(g):
    """sum_c dz_c = 0 (the softmax stays on the simplex); a constant dy gives
    dz = 0; C = 1 gives dz = 0; dz is linear in dy."""
    rng = _rng(33)
    z = rng.standard_normal((8, 40)) * 3
    y = _scipy_softmax(z)
    d1, d2 = rng.standard_normal((2, 8, 40))
    dz = g(y, d1)
    assert np.abs(dz.sum(axis=1)).max() <= 1e-14
    np.testing.assert_allclose(g(y, np.full_like(y, 2.75)), 0.0, atol=1e-15)
    np.testing.assert_array_equal(g(np.ones((4, 1)), rng.standard_normal((4, 1))), 0.0)
    np.testing.assert_allclose(g(y, 3.0 * d1 - 0.5 * d2), 3.0 * dz - 0.5 * g(y, d2),
                               rtol=1e-11, atol=1e-14)


def bpin_onehot_column(g):
    """dy = e_j picks one output: dz = y_j (e_j - y), the closed form of the
    gradient of y_j."""
    rng = _rng(34)
    y = _scipy_softmax(rng.standard_normal((6, 9)) * 2)
    for j in (0, 4, 8):
        dy = np.zeros_like(y)
        dy[:, j] = 1.0
        want = -y * y[:, j:j + 1]
        want[:, j] += y[:, j]
        np.testing.assert_allclose(g(y, dy), want, rtol=1e-13, atol=1e-17)


def bpin_cross_entropy(g):
    """Chain rule through the loss: for loss = -ln y_t / B the upstream
    gradient is dy = -[c == t] / (B y_t), and the softmax backward of it is
    the cross-entropy gradient (softmax - onehot) / B of the pinned CE
    oracle."""
    rng = _rng(35)
    B, C = 16, 70
    z = rng.standard_normal((B, C)) * 3
    t = rng.integers(0, C, B)
    y = _scipy_softmax(z)
    dy = np.zeros_like(y)
    dy[np.arange(B), t] = -1.0 / (B * y[np.arange(B), t])
    _, grad = ce_rows(z, t, B)
    np.testing.assert_allclose(g(y, dy), grad, rtol=1e-11, atol=1e-16)


def bpin_torch(g):
    """Library cross-check: torch autograd through torch.softmax in float64."""
    import torch
    rng = _rng(36)
    z = torch.from_numpy(rng.standard_normal((7, 123)) * 4).requires_grad_(True)
    dy = torch.from_numpy(rng.standard_normal((7, 123)))
    y = torch.softmax(z, dim=1)
    y.backward(dy)
    np.testing.assert_allclose(g(y.detach().numpy(), dy.numpy()), z.grad.numpy(),
                               rtol=1e-11, atol=1e-16)


BWD_PINS = [bpin_finite_difference, bpin_jacobian, bpin_invariants, bpin_onehot_column,
            bpin_cross_entropy, bpin_torch]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_softmax_bwd_oracle_meets_pin(pin):
    pin(softmax_bwd_rows)


def _bwd_mutant(kind):
    def g(y, dy):
        y = np.asarray(y, dtype=np.float64)
        dy = np.asarray(dy, dtype=np.float64)
        if kind == "dot_without_y":
            dot = dy.sum(axis=1)
        elif kind == "transposed_dot":
            dot = (dy * y).sum(axis=0)[np.arange(y.shape[0]) % y.shape[1]]
        else:
            dot = (dy * y).sum(axis=1)
        if kind == "sign":
            return y * (dot[:, None] - dy)
        if kind == "no_y":
            return dy - dot[:, None]
        if kind == "no_dot":
            return y * dy
        if kind == "y_squared":
            return y * y * (dy - dot[:, None])
        return y * (dy - dot[:, None])
    g.__name__ = f"bwd_mutant_{kind}"
    return g


BWD_MUTANTS = ["dot_without_y", "transposed_dot", "sign", "no_y", "no_dot", "y_squared"]


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_softmax_bwd_planted_mistake_is_caught(kind):
    assert _caught(BWD_PINS, _bwd_mutant(kind)), f"no pin catches backward mutant {kind}"


def test_softmax_bwd_mutant_scaffold_passes():
    assert _caught(BWD_PINS, _bwd_mutant("none")) == []


# --------------------------------------------------------------------------
# vocabulary shards: sp(z_shard, t, col0) -> (m, sx, zt, owns);
# cp(records, t, C, B) -> (m, S, zt, loss)
# --------------------------------------------------------------------------

def _splits(C, k, rng):
    cuts = np.sort(rng.choice(np.arange(1, C), size=k - 1, replace=False)) if k > 1 else []
    return [0, *[int(x) for x in cuts], C]


def spin_whole_row(sp, cp):
    """Any split of the row into 1 to 6 shards combines to the row's max, its
    full sum of exponentials and the pinned CE oracle's loss."""
    rng = _rng(41)
    B, C = 12, 97
    z = rng.standard_normal((B, C)) * 4
    z[3, 50] = 1e4
    t = rng.integers(0, C, B)
    t[3] = 50
    l_ref, _ = ce_rows(z, t, B)
    m_ref = z.max(axis=1)
    for k in (1, 2, 3, 6):
        edges = _splits(C, k, rng)
        recs = [sp(z[:, a:b], t, a) for a, b in zip(edges[:-1], edges[1:])]
        assert (np.sum([r[3] for r in recs], axis=0) == 1).all()   # one owner per row
        m, S, zt, loss = cp(recs, t, C, B)
        np.testing.assert_array_equal(m, m_ref)
        np.testing.assert_allclose(S, np.exp(z - m_ref[:, None]).sum(axis=1), rtol=1e-13)
        np.testing.assert_array_equal(zt, z[np.arange(B), t])
        np.testing.assert_allclose(loss, l_ref, rtol=1e-12, atol=1e-15)


def spin_one_shard(sp, cp):
    """One shard: its max is the row max, its sum leaves out exactly the
    target's term, and it holds the target logit."""
    rng = _rng(42)
    z = rng.standard_normal((5, 20)) * 3
    t = rng.integers(0, 20, 5)
    m, sx, zt, owns = sp(z, t, 0)
    assert owns.all()
    np.testing.assert_array_equal(m, z.max(axis=1))
    e = np.exp(z - z.max(axis=1)[:, None])
    np.testing.assert_allclose(sx, e.sum(axis=1) - e[np.arange(5), t], rtol=1e-13)
    np.testing.assert_array_equal(zt, z[np.arange(5), t])


def spin_foreign_shard(sp, cp):
    """A shard without the target: the full sum of its exponentials, zt = 0;
    a one-column shard holding the target: sum 0."""
    rng = _rng(43)
    z = rng.standard_normal((4, 10)) * 3
    t = np.array([0, 25, -1, 9])                  # all outside columns [10, 20)
    m, sx, zt, owns = sp(z, t, 10)
    assert not owns.any() and (zt == 0).all()
    np.testing.assert_allclose(sx, np.exp(z - z.max(axis=1)[:, None]).sum(axis=1), rtol=1e-14)
    m1, sx1, zt1, owns1 = sp(z[:, 3:4], np.array([3, 3, 3, 3]), 3)
    assert owns1.all() and (sx1 == 0).all()
    np.testing.assert_array_equal(zt1, z[:, 3])


def spin_invalid_target(sp, cp):
    """A target outside [0, C) belongs to no shard and gives a NaN loss."""
    rng = _rng(44)
    z = rng.standard_normal((3, 12))
    t = np.array([-1, 12, 5])
    recs = [sp(z[:, :6], t, 0), sp(z[:, 6:], t, 6)]
    _, _, _, loss = cp(recs, t, 12, 3)
    assert np.isnan(loss[0]) and np.isnan(loss[1]) and np.isfinite(loss[2])


def spin_shard_order(sp, cp):
    """The combine is a max and sums: the shards' order changes the result
    by rounding only."""
    rng = _rng(45)
    z = rng.standard_normal((6, 60)) * 5
    t = rng.integers(0, 60, 6)
    recs = [sp(z[:, a:a + 15], t, a) for a in (0, 15, 30, 45)]
    l0 = cp(recs, t, 60, 6)[3]
    l1 = cp(recs[::-1], t, 60, 6)[3]
    np.testing.assert_allclose(l1, l0, rtol=1e-14)


SHARD_PINS = [spin_whole_row, spin_one_shard, spin_foreign_shard, spin_invalid_target,
              spin_shard_order]


@pytest.mark.parametrize("pin", SHARD_PINS, ids=lambda p: p.__name__)
def test_shard_oracle_meets_pin(pin):
    pin(shard_partials, combine_partials)


def _shard_mutants(kind):
    def sp(z_shard, t, col0):
        m, sx, zt, owns = shard_partials(z_shard, t, col0)
        z = np.asarray(z_shard, dtype=np.float64)
        if kind == "target_in_sum":
            sx = np.exp(z - m[:, None]).sum(axis=1)
        if kind == "owner_off_by_one":
            local = np.asarray(t) - col0
            owns = (local >= 0) & (local <= z.shape[1])   # takes the next shard's first column
            lc = np.clip(local, 0, z.shape[1] - 1)
            zt = np.where(owns, z[np.arange(z.shape[0]), lc], 0.0)
        return m, sx, zt, owns

    def cp(records, t, C, B):
        if kind == "no_rescale":
            t = np.asarray(t)
            m = np.max(np.stack([r[0] for r in records]), axis=0)
            sx = np.sum([r[1] for r in records], axis=0)
            zt = np.sum([r[2] for r in records], axis=0)
            S = sx + np.exp(zt - m)
            valid = (t >= 0) & (t < C)
            return m, S, zt, np.where(valid, (np.log(S) + (m - zt)) / B, np.nan)
        if kind == "first_shard_max":
            recs = [(records[0][0], r[1] * np.exp(r[0] - records[0][0]), r[2], r[3])
                    for r in records]
            out = combine_partials(recs, t, C, B)
            return (records[0][0],) + tuple(out[1:])
        return combine_partials(records, t, C, B)
    sp.__name__ = cp.__name__ = f"shard_mutant_{kind}"
    return sp, cp


SHARD_MUTANTS = ["target_in_sum", "owner_off_by_one", "no_rescale", "first_shard_max"]


@pytest.mark.parametrize("kind", SHARD_MUTANTS)
def test_shard_planted_mistake_is_caught(kind):
    sp, cp = _shard_mutants(kind)
    hits = []
    for pin in SHARD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(sp, cp)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            hits.append(pin.__name__)
    assert hits, f"no pin catches shard mutant {kind}"


def test_shard_mutant_scaffold_passes():
    sp, cp = _shard_mutants("none")
    for pin in SHARD_PINS:
        pin(sp, cp)
