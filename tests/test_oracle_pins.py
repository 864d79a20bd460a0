"""Pins for the fp64 oracle: facts fixed by the mathematics, not by the
oracle's own code.

Each ``pin_*`` takes an implementation ``f(z, t, B) -> (loss_rows, grad)``
(float64 in, float64 out, already scaled by 1/B) and raises AssertionError
when the implementation disagrees with the fact it checks.  The real oracle
must pass every pin; each planted mistake (a mutant of the oracle, built in
this file on the CPU) must fail at least one, which shows that a dropped
term, a wrong sign or index or a transposed reduction cannot slip through.

The definition pinned here: rumus project page, milestone M7a (fused
cross-entropy with log-sum-exp; gradient softmax minus one-hot formed in the
forward pass) and rumus 0.1.1 ``cross_entropy.wgsl`` source view, pass 1
steps 1-4 and pass 2.
"""

from __future__ import annotations

import ast
import json
import math
import os

import numpy as np
import pytest

from oracle import ce, ce_rows, reduce_loss, rne_bf16_bits, widen_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_uniform(f):
    """All logits of a row equal: softmax is 1/C, so loss*B = ln C and the
    gradient is (1/C - [c == t]) / B (closed form)."""
    for C in (1, 2, 3, 10, 1000):
        for v in (0.0, 2.5, -1e4, 1e4):
            B = 4
            z = np.full((B, C), v)
            t = np.arange(B) % C
            loss, g = f(z, t, B)
            np.testing.assert_allclose(loss * B, math.log(C), rtol=1e-12, atol=1e-15)
            want = np.full((B, C), 1.0 / C)
            want[np.arange(B), t] -= 1.0
            np.testing.assert_allclose(g, want / B, rtol=0, atol=1e-15)


def pin_one_class(f):
    """C = 1: the softmax is 1, so loss and gradient are exactly 0."""
    z = _rng(1).standard_normal((5, 1)) * 100
    loss, g = f(z, np.zeros(5, np.int64), 5)
    assert np.all(loss == 0.0) and np.all(g == 0.0)


def pin_two_class(f):
    """C = 2 is logistic regression: with d = z_other - z_target,
    loss*B = softplus(d) = ln(1 + e^d) and the gradient of the other class is
    sigmoid(d)/B = -(gradient of the target class)."""
    rng = _rng(2)
    z = rng.standard_normal((64, 2)) * 6
    t = rng.integers(0, 2, 64)
    B = 64
    loss, g = f(z, t, B)
    for b in range(B):
        o = 1 - t[b]
        d = z[b, o] - z[b, t[b]]
        softplus = max(d, 0.0) + math.log1p(math.exp(-abs(d)))
        sig = 1.0 / (1.0 + math.exp(-d)) if d >= 0 else math.exp(d) / (1.0 + math.exp(d))
        # ln(s) with s = 1 + e^d rounded: absolute error ~1e-16 on loss*B
        assert math.isclose(loss[b] * B, softplus, rel_tol=1e-12, abs_tol=1e-14)
        assert math.isclose(g[b, o] * B, sig, rel_tol=1e-12, abs_tol=1e-300)
        # softmax_t - 1 rounds p_t first: absolute error ~1e-16 on g*B
        assert math.isclose(g[b, t[b]] * B, -sig, rel_tol=1e-12, abs_tol=1e-15)


def pin_spike(f):
    """Rows of N(0, 3) with one entry at +1e4: every other exponential
    exp(z - 1e4) is below 1e-4000 and vanishes, so the answer is closed
    form.  Target off the spike: loss*B = 1e4 - z_t, gradient +1/B at the
    spike and -1/B at the target, zero elsewhere.  Target on the spike: loss
    and gradient are zero."""
    rng = _rng(3)
    B, C = 16, 300
    z = rng.standard_normal((B, C)) * 3
    spike = rng.integers(0, C, B)
    z[np.arange(B), spike] = 1e4
    t = rng.integers(0, C, B)
    t[:3] = spike[:3]
    loss, g = f(z, t, B)
    for b in range(B):
        want = np.zeros(C)
        if t[b] == spike[b]:
            assert loss[b] == 0.0
        else:
            assert math.isclose(loss[b] * B, 1e4 - z[b, t[b]], rel_tol=1e-13)
            want[spike[b]] = 1.0 / B
            want[t[b]] = -1.0 / B
        np.testing.assert_allclose(g[b], want, rtol=0, atol=1e-300)


def pin_shift(f):
    """Adding a constant k to a row changes neither loss nor gradient."""
    rng = _rng(4)
    B, C = 8, 37
    z = rng.standard_normal((B, C)) * 5
    t = rng.integers(0, C, B)
    l0, g0 = f(z, t, B)
    for k in (-300.0, -1.0, 0.5, 64.0, 1e3):
        l1, g1 = f(z + k, t, B)
        np.testing.assert_allclose(l1, l0, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(g1, g0, rtol=1e-9, atol=1e-15)


def pin_row_sum(f):
    """Softmax sums to 1 and the one-hot to 1: each gradient row sums to 0."""
    rng = _rng(5)
    for C in (2, 10, 1000):
        B = 32
        z = rng.standard_normal((B, C)) * 4
        t = rng.integers(0, C, B)
        _, g = f(z, t, B)
        assert np.abs(g.sum(axis=1)).max() <= 1e-15


def pin_bounds(f):
    """Sign and range of every entry: the target entry is in [-1/B, 0], the
    others in [0, 1/B]; per row 0 <= loss*B - (max_c z - z_t) <= ln C, so the
    loss is non-negative.  When the target is a row argmax its softmax is at
    least 1/C, so |g_target| <= (1 - 1/C)/B."""
    rng = _rng(6)
    B, C = 64, 50
    z = rng.standard_normal((B, C)) * 3
    t = rng.integers(0, C, B)
    t[:8] = z[:8].argmax(axis=1)
    loss, g = f(z, t, B)
    rows = np.arange(B)
    gt = g[rows, t]
    assert np.all(gt <= 0) and np.all(gt >= -1.0 / B)
    mask = np.ones_like(g, bool)
    mask[rows, t] = False
    assert np.all(g[mask] >= 0) and np.all(g[mask] <= 1.0 / B)
    gap = loss * B - (z.max(axis=1) - z[rows, t])
    assert np.all(gap >= -1e-12) and np.all(gap <= math.log(C) + 1e-12)
    assert np.all(np.abs(gt[:8]) <= (1 - 1.0 / C) / B + 1e-18)


def pin_finite_difference(f):
    """The gradient is dL/dz for L = sum_b loss_b: central differences of L
    (step 1e-6, evaluated in fp64) agree to 1e-8."""
    rng = _rng(7)
    for B, C in ((1, 2), (3, 5), (8, 16)):
        z = rng.standard_normal((B, C)) * 2
        t = rng.integers(0, C, B)
        _, g = f(z, t, B)
        h = 1e-6
        for b in range(B):
            for c in range(C):
                zp = z.copy()
                zp[b, c] += h
                zm = z.copy()
                zm[b, c] -= h
                fd = (math.fsum(f(zp, t, B)[0]) - math.fsum(f(zm, t, B)[0])) / (2 * h)
                assert abs(fd - g[b, c]) <= 1e-8, (B, C, b, c, fd, g[b, c])


def pin_extreme(f):
    """Logits of magnitude 1e4 (all high, all low, mixed signs, one spike):
    every output stays finite and all-equal rows still give ln C."""
    B, C = 4, 7
    z = np.array([[1e4] * C, [-1e4] * C,
                  [1e4 if c % 2 else -1e4 for c in range(C)],
                  [0.0] * (C - 1) + [1e4]])
    t = np.array([0, 3, 2, 6])
    loss, g = f(z, t, B)
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(g))
    assert math.isclose(loss[0] * B, math.log(C), rel_tol=1e-12)
    assert math.isclose(loss[1] * B, math.log(C), rel_tol=1e-12)
    # mixed row: three classes at +1e4 share the mass, target 2 is at -1e4
    assert math.isclose(loss[2] * B, 2e4 + math.log(3), rel_tol=1e-12)


def pin_permutation(f):
    """Permuting the classes (and remapping the target) permutes the
    gradient and leaves the loss unchanged; permuting the rows permutes the
    per-row outputs."""
    rng = _rng(8)
    B, C = 6, 11
    z = rng.standard_normal((B, C)) * 3
    t = rng.integers(0, C, B)
    l0, g0 = f(z, t, B)
    perm = rng.permutation(C)
    inv = np.argsort(perm)
    l1, g1 = f(z[:, perm], inv[t], B)
    np.testing.assert_allclose(l1, l0, rtol=1e-13)
    np.testing.assert_allclose(g1, g0[:, perm], rtol=1e-12, atol=1e-17)
    rp = rng.permutation(B)
    l2, g2 = f(z[rp], t[rp], B)
    np.testing.assert_array_equal(l2, l0[rp])
    np.testing.assert_array_equal(g2, g0[rp])


def pin_batch_independence(f):
    """Row b's outputs times B depend only on row b: adding rows (and
    changing B accordingly) leaves loss*B and grad*B of the old rows alone."""
    rng = _rng(9)
    C = 13
    z = rng.standard_normal((4, C)) * 3
    t = rng.integers(0, C, 4)
    l0, g0 = f(z, t, 4)
    z2 = np.concatenate([z, rng.standard_normal((12, C)) * 3])
    t2 = np.concatenate([t, rng.integers(0, C, 12)])
    l1, g1 = f(z2, t2, 16)
    np.testing.assert_allclose(l1[:4] * 16, l0 * 4, rtol=1e-14)
    np.testing.assert_allclose(g1[:4] * 16, g0 * 4, rtol=1e-13, atol=1e-17)


def pin_scipy(f):
    """Library cross-check: loss = -log_softmax(z)[t] / B and
    grad = (softmax(z) - onehot) / B with scipy.special's routines."""
    from scipy.special import log_softmax, softmax
    rng = _rng(10)
    for C in (3, 100, 5000):
        B = 16
        z = rng.standard_normal((B, C)) * 4
        t = rng.integers(0, C, B)
        loss, g = f(z, t, B)
        ls = log_softmax(z, axis=1)
        np.testing.assert_allclose(loss, -ls[np.arange(B), t] / B, rtol=1e-12)
        want = softmax(z, axis=1)
        want[np.arange(B), t] -= 1.0
        np.testing.assert_allclose(g, want / B, rtol=1e-11, atol=1e-17)


def pin_torch(f):
    """Library cross-check: torch's CPU cross_entropy (mean reduction) in
    float64 and its autograd gradient equal the batch-mean loss and the
    gradient."""
    torch = pytest.importorskip("torch")
    rng = _rng(11)
    for B, C in ((8, 10), (33, 257)):
        z = rng.standard_normal((B, C)) * 3
        t = rng.integers(0, C, B)
        loss, g = f(z, t, B)
        x = torch.tensor(z, dtype=torch.float64, requires_grad=True)
        L = torch.nn.functional.cross_entropy(x, torch.tensor(t, dtype=torch.long))
        L.backward()
        assert math.isclose(math.fsum(loss), L.item(), rel_tol=1e-13)
        np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-11, atol=1e-18)


def _eval_expr(s: str) -> float:
    """Evaluate a closed-form expression: numbers, + - * /, unary minus and
    ln(...).  Nothing else is accepted."""
    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, ast.USub):
            return -ev(n.operand)
        if isinstance(n, ast.BinOp):
            a, b = ev(n.left), ev(n.right)
            ops = {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b}
            if isinstance(n.op, ast.Div):
                return a / b
            return ops[type(n.op)]
        if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id == "ln":
            return math.log(ev(n.args[0]))
        raise ValueError(f"bad expression {s!r}")
    return ev(ast.parse(s, mode="eval"))


def pin_golden(f):
    """Hand-derived cases from tests/golden/closed_forms.json."""
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    for case in cases:
        z = np.array([[_eval_expr(v) for v in row] for row in case["z"]])
        t = np.array(case["t"])
        B = case["B"]
        loss, g = f(z, t, B)
        want_l = np.array([_eval_expr(v) for v in case["loss_rows"]])
        want_g = np.array([[_eval_expr(v) for v in row] for row in case["grad"]])
        np.testing.assert_allclose(loss, want_l, rtol=1e-13, atol=1e-15, err_msg=case["name"])
        np.testing.assert_allclose(g, want_g, rtol=1e-13, atol=1e-15, err_msg=case["name"])
        assert math.isclose(math.fsum(loss), _eval_expr(case["loss"]), rel_tol=1e-13,
                            abs_tol=1e-15), case["name"]


PINS = [pin_uniform, pin_one_class, pin_two_class, pin_spike, pin_shift, pin_row_sum,
        pin_bounds, pin_finite_difference, pin_extreme, pin_permutation,
        pin_batch_independence, pin_scipy, pin_torch, pin_golden]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    pin(ce_rows)


# --------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail some pin
# --------------------------------------------------------------------------

def _mutant(kind):
    def f(z, t, B):
        z = np.asarray(z, dtype=np.float64)
        t = np.asarray(t, dtype=np.int64)
        n, C = z.shape
        rows = np.arange(n)
        m = z.max(axis=1)
        if kind == "no_max_shift":
            with np.errstate(over="ignore", invalid="ignore"):
                e = np.exp(z)
                s = e.sum(axis=1)
                loss = (np.log(s) - z[rows, t]) / B
                g = e / s[:, None]
        else:
            e = np.exp(z - m[:, None])
            s = e.sum(axis=1)
            if kind == "sum_skips_max":
                s = s - 1.0 + 1e-300
            if kind == "transposed_norm":
                s_col = e.sum(axis=0)
                g = e / s_col[None, :]
            else:
                g = e / s[:, None]
            zt = z[(rows + 1) % n, t] if kind == "target_wrong_row" else z[rows, t]
            lse = (np.log2(s) if kind == "log2" else np.log(s))
            if kind == "loss_drops_max":
                loss = (lse - zt) / B
            else:
                loss = (lse + (m - zt)) / B
        if kind == "loss_unscaled":
            loss = loss * B
        oh = (t + 1) % C if kind == "onehot_shift" else t
        sign = -1.0 if kind == "onehot_sign" else 1.0
        g = g.copy()
        g[rows, oh] -= sign * 1.0
        if kind != "grad_unscaled":
            g /= B
        return loss, g
    f.__name__ = f"mutant_{kind}"
    return f


MUTANTS = ["onehot_sign", "grad_unscaled", "loss_unscaled", "onehot_shift", "no_max_shift",
           "loss_drops_max", "transposed_norm", "log2", "target_wrong_row", "sum_skips_max"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    f = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(f)
        except (AssertionError, FloatingPointError, IndexError, ValueError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {kind}"


def test_correct_mutant_baseline_passes():
    """The mutant scaffold with no mistake planted passes every pin, so the
    failures above come from the planted mistakes alone."""
    f = _mutant("none")
    for pin in PINS:
        pin(f)


# --------------------------------------------------------------------------
# the rest of the oracle: invalid targets, the scalar sum, bf16 handling
# --------------------------------------------------------------------------

def test_invalid_target_rows_are_nan():
    z = _rng(12).standard_normal((4, 6))
    t = np.array([0, -1, 6, 5])
    loss, g = ce_rows(z, t, 4)
    assert np.isfinite(loss[[0, 3]]).all() and np.isnan(loss[[1, 2]]).all()
    assert np.isfinite(g[[0, 3]]).all() and np.isnan(g[[1, 2]]).all()


def test_shape_errors():
    with pytest.raises(ValueError):
        ce_rows(np.zeros((2, 0)), np.zeros(2, np.int64), 2)


def test_reduce_is_exactly_rounded():
    # fsum of values whose naive sum loses the small terms
    assert reduce_loss([1e16, 1.0, -1e16]) == 1.0
    rng = _rng(13)
    x = rng.random(10000) * 1e-3
    s = reduce_loss(x)
    assert s == reduce_loss(x[::-1]) == reduce_loss(rng.permutation(x))
    from fractions import Fraction
    exact = sum(Fraction(v) for v in x[:500].tolist())
    assert reduce_loss(x[:500]) == float(exact)


def test_widen_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    w = widen_bf16(bits)
    same = (w == t) | (np.isnan(w) & np.isnan(t))
    assert same.all()


def test_rne_bf16_matches_torch_on_fp32_values():
    """For values that are exactly fp32, a single rounding fp64 -> bf16 equals
    torch's fp32 -> bf16 conversion (round to nearest, ties to even)."""
    torch = pytest.importorskip("torch")
    rng = _rng(14)
    x = np.concatenate([
        (rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000)).astype(np.float32),
        rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        # exact ties: bf16 value plus half a bf16 spacing
        ((rng.integers(0, 1 << 15, 5000, dtype=np.uint32) << 16) | 0x8000).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = rne_bf16_bits(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_rne_bf16_hand_cases():
    one = 0x3F80
    assert rne_bf16_bits(np.array([1.0]))[0] == one
    assert rne_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == one          # tie -> even
    assert rne_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == one + 2  # tie -> even
    assert rne_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 1
    assert rne_bf16_bits(np.array([-0.0]))[0] == 0x8000
    assert rne_bf16_bits(np.array([2.0 ** -133]))[0] == 0x0001           # smallest subnormal
    assert rne_bf16_bits(np.array([2.0 ** -134]))[0] == 0x0000           # tie -> even (zero)


def test_bf16_oracle_widens_exactly():
    """The bf16 entry point equals the f32 entry point on the widened values."""
    rng = _rng(15)
    z = (rng.standard_normal((5, 40)) * 4).astype(np.float32)
    import synth
    bits = synth.bf16_bits_from_f32(z)
    t = rng.integers(0, 40, 5).astype(np.int32)
    l1, g1 = ce(bits, t, "bf16")
    l2, g2 = ce(widen_bf16(bits).astype(np.float32), t, "f32")
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(g1, g2)


def test_row_selection_matches_full():
    import synth
    z, t = synth.make_inputs(50, 33, "f32", 2.0, seed=3)
    lf, gf = ce(z, t, "f32", block_elems=100)
    rows = np.array([49, 0, 17])
    ls, gs = ce(z, t, "f32", rows=rows)
    np.testing.assert_array_equal(ls, lf[rows])
    np.testing.assert_array_equal(gs, gf[rows])


# --------------------------------------------------------------------------
# fp16 conversions and ignore_index
# --------------------------------------------------------------------------

def test_widen_f16_every_pattern():
    """All 65536 binary16 patterns decode to numpy's float16 values."""
    from oracle import widen_f16
    b = np.arange(1 << 16, dtype=np.uint16)
    got, want = widen_f16(b), b.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_rne_f16_hand_cases():
    """Ties to even at 1, in the subnormal range and at the overflow edge."""
    from oracle import rne_f16_bits
    cases = {
        1.0: 0x3C00, 1.0 + 2.0 ** -11: 0x3C00,            # tie: down to even
        1.0 + 3 * 2.0 ** -11: 0x3C02,                       # tie: up to even
        2.0 ** -24: 0x0001, 2.0 ** -25: 0x0000,             # smallest subnormal; tie to 0
        1.5 * 2.0 ** -24: 0x0002, 2.0 ** -14: 0x0400,       # tie up to even; smallest normal
        65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00,  # largest finite; tie to inf
        -2.0: 0xC000, -0.0: 0x8000, float("inf"): 0x7C00, -1e6: 0xFC00,
    }
    x = np.array(list(cases))
    np.testing.assert_array_equal(rne_f16_bits(x), np.array(list(cases.values()), np.uint16))
    assert np.isnan(np.array([0]).astype(np.uint16).view(np.float16)).sum() == 0
    assert rne_f16_bits(np.array([np.nan]))[0] & 0x7C00 == 0x7C00


def test_rne_f16_matches_numpy_and_torch():
    """Random magnitudes from 2^-30 to 2^17: numpy's float64 -> float16
    conversion (one rounding to nearest even) agrees bit for bit, and so
    does torch's float32 -> float16 on float32 inputs (torch's float64 ->
    float16 goes through float32 and rounds twice, so it is not the
    reference for float64 inputs)."""
    import torch
    from oracle import rne_f16_bits
    rng = _rng(60)
    x = rng.standard_normal(300_000) * np.exp2(rng.uniform(-30, 17, 300_000))
    got = rne_f16_bits(x)
    with np.errstate(over="ignore"):
        assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    x32 = x.astype(np.float32)
    tt = torch.from_numpy(x32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rne_f16_bits(x32.astype(np.float64)), tt)


def test_f16_oracle_widens_exactly():
    from oracle import rne_f16_bits, widen_f16
    rng = _rng(61)
    z = rne_f16_bits(rng.standard_normal((6, 300)) * 4)
    t = rng.integers(0, 300, 6)
    l1, g1 = ce(z, t, "f16")
    l2, g2 = ce_rows(widen_f16(z), t, 6)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(g1, g2)


def test_ignore_index_matches_torch():
    """Library cross-check: torch.nn.functional.cross_entropy with
    ignore_index and the mean reduction, in float64 on the CPU, gives the
    sum of the per-row losses and, by autograd, the gradient."""
    import torch
    from oracle import ce_rows_ignore
    rng = _rng(62)
    for B, C, ii in ((16, 9, -100), (40, 300, 7), (5, 2, 0)):
        z = rng.standard_normal((B, C)) * 3
        t = rng.integers(0, C, B)
        t[rng.random(B) < 0.4] = ii
        t[0] = ii
        if (t == ii).all():
            t[1] = (ii + 1) % C
        loss, grad = ce_rows_ignore(z, t, ii)
        zt = torch.from_numpy(z).requires_grad_(True)
        L = torch.nn.functional.cross_entropy(zt, torch.from_numpy(t), ignore_index=ii)
        L.backward()
        assert math.isclose(math.fsum(loss), L.item(), rel_tol=1e-13)
        np.testing.assert_allclose(grad, zt.grad.numpy(), rtol=1e-12, atol=1e-17)


def test_ignore_index_reductions():
    """No row ignored: ce_rows with B; every row ignored: zeros; the logits of
    an ignored row change nothing; each kept row equals ce_rows of the kept
    rows with B = their count."""
    from oracle import ce_rows_ignore
    rng = _rng(63)
    B, C = 12, 20
    z = rng.standard_normal((B, C)) * 2
    t = rng.integers(0, C, B)
    l0, g0 = ce_rows(z, t, B)
    l1, g1 = ce_rows_ignore(z, t, -1)
    np.testing.assert_array_equal(l0, l1)
    np.testing.assert_array_equal(g0, g1)
    l2, g2 = ce_rows_ignore(z, np.full(B, 3), 3)
    assert (l2 == 0).all() and (g2 == 0).all()
    t2 = t.copy()
    t2[[1, 4, 5]] = -100
    l3, g3 = ce_rows_ignore(z, t2, -100)
    z2 = z.copy()
    z2[[1, 4, 5]] = 1e4
    l4, g4 = ce_rows_ignore(z2, t2, -100)
    np.testing.assert_array_equal(l3, l4)
    np.testing.assert_array_equal(g3, g4)
    keep = t2 != -100
    l5, g5 = ce_rows(z[keep], t2[keep], int(keep.sum()))
    np.testing.assert_array_equal(l3[keep], l5)
    np.testing.assert_array_equal(g3[keep], g5)
    assert (l3[~keep] == 0).all() and (g3[~keep] == 0).all()


def test_ignore_index_mutant_scaled_by_batch_is_caught():
    """A planted mistake (kept rows scaled by 1/B instead of 1/N) fails the
    torch cross-check."""
    import torch
    rng = _rng(64)
    B, C = 16, 9
    z = rng.standard_normal((B, C))
    t = rng.integers(0, C, B)
    t[:5] = -100
    keep = t != -100
    l_bad, _ = ce_rows(z[keep], t[keep], B)
    L = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(t),
                                          ignore_index=-100)
    assert not math.isclose(math.fsum(l_bad), L.item(), rel_tol=1e-6)
