"""Row-wise softmax forward and backward on the GPU against the fp64 oracle
(rumus project page, milestone M8c).

Bars (derived from the float32 arithmetic of the kernels):

* forward, y: as the cross-entropy gradient at B = 1: fp32 max |y - y_ora|
  <= 1e-6; bf16 within 1 ulp of the oracle's value rounded once to bf16
  (magnitudes below 2^-126 count as zero).
* forward, lse = ln2 * (round(m log2 e) + log2 S): |lse - lse_ora| <=
  2^-20 (|m| + ln C + 1), the rounding of m log2 e, of S and of the
  logarithm, each a few ulps of float32 of the row's magnitudes.
* backward, dx = y (dy - dot): the float32 dot of C products is off by at
  most g = 2^-24 (16 + C/256) sum |y dy| (its longest chain of dependent
  additions is below 16 + C/256), which reaches dx through the factor y;
  the two roundings of y (dy - dot) add 2^-22 |dx|.  fp32: |dx - dx_ora|
  <= y g + 2^-22 |dx_ora|.  bf16: the same plus one bf16 ulp (2^-7
  |dx_ora|, magnitudes below 2^-126 counting as zero).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import ce_rows, rne_bf16_bits, softmax_bwd_rows, softmax_rows, widen_bf16

from _parity import path_takes, wave_bwd_takes, bf16_order, grad_to_host, widen_rows

pytestmark = pytest.mark.gpu

FWD_SHAPES = [
    (8, 10, "f32", 1.0, None),
    (7, 1, "f32", 3.0, None),
    (300, 2, "bf16", 5.0, None),
    (129, 100, "bf16", 4.0, None),
    (64, 256, "f32", 2.0, None),
    (64, 257, "bf16", 3.0, None),
    (1024, 1000, "f32", 2.0, None),
    (33, 4099, "f32", 3.0, None),
    (17, 12345, "bf16", 4.0, None),
    (40, 50257, "f32", 3.0, 1.0e4),
    (9, 128256, "bf16", 4.0, None),
    (5, 70001, "bf16", 4.0, None),
    (3, 200_000, "bf16", 4.0, None),
    (6, 151936, "f32", 3.0, None),
    (3, 300_000, "bf16", 4.0, None),
    (4, 180_000, "f32", 3.0, None),
]
FWD_IDS = [f"{b}x{c}-{d}{'-spike' if s else ''}" for b, c, d, _, s in FWD_SHAPES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _reset_path():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _legal(path, C, dtype):
    return path_takes(path, C, dtype)


def _dev(a, dtype):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


def check_y(y_host, y_ora, dtype, where):
    if dtype == "f32":
        err = np.abs(y_host.astype(np.float64) - y_ora)
        assert err.max() <= 1e-6, (where, float(err.max()))
        return float(err.max())
    ulp = np.abs(bf16_order(y_host) - bf16_order(rne_bf16_bits(y_ora)))
    assert ulp.max() <= 1, (where, int(ulp.max()))
    return int(ulp.max())


def check_lse(lse_host, z64, lse_ora, where):
    C = z64.shape[1]
    tol = 2.0 ** -20 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0)
    err = np.abs(lse_host.astype(np.float64) - lse_ora)
    assert (err <= tol).all(), (where, float(err.max()), float(tol[np.argmax(err - tol)]))


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype,sigma,spike", FWD_SHAPES, ids=FWD_IDS)
def test_softmax_fwd_matches_oracle(B, C, dtype, sigma, spike, path):
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, _ = synth.make_inputs(B, C, dtype, sigma, spike=spike, seed=B * 7 + C)
    zd = _dev(z, dtype)
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    z64 = widen_rows(z, dtype)
    y_ora, lse_ora = softmax_rows(z64)
    worst = check_y(grad_to_host(y, dtype), y_ora, dtype, f"{B}x{C} {dtype} p{path}")
    check_lse(lse.cpu().numpy(), z64, lse_ora, f"{B}x{C} {dtype} p{path}")
    print(f"[softmax] fwd {B}x{C} {dtype} p{path}: worst {worst}", flush=True)
    # without the log-sum-exp: the same softmax bits
    y2 = ce.softmax_fwd(zd)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y2), _bits(y))


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype", [(64, 200, "bf16"), (33, 4099, "f32"), (9, 50257, "f32"),
                                       (6, 128256, "bf16"), (3, 200_000, "bf16")])
def test_softmax_fwd_in_place(B, C, dtype, path):
    """y == x: the same bits as out of place on the same path (two-part rows
    are refused on forced path 4 and run on path 2 or 3 otherwise)."""
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    z, _ = synth.make_inputs(B, C, dtype, 3.0, seed=C + 1)
    zd = _dev(z, dtype)
    two_part = C // (16 // (4 if dtype == "f32" else 2)) > 10 * 1024
    ce.force_path(path)
    buf = zd.clone()
    lse_in = torch.empty(B, dtype=torch.float32, device=zd.device)
    if path == 4 and two_part:
        with pytest.raises(ce.CEError):
            ce.softmax_fwd_into(buf, buf, lse_in)
        return
    ce.softmax_fwd_into(buf, buf, lse_in)
    if path == 0 and two_part:
        # out of place these rows run as row parts, in place on path 2 or 3
        # with the automatic configuration: both against the oracle
        torch.cuda.synchronize()
        z64 = widen_rows(z, dtype)
        y_ora, lse_ora = softmax_rows(z64)
        check_y(grad_to_host(buf, dtype), y_ora, dtype, f"in place {B}x{C}")
        check_lse(lse_in.cpu().numpy(), z64, lse_ora, f"in place {B}x{C}")
        return
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(buf), _bits(y))
    assert torch.equal(lse_in.view(torch.int32), lse.view(torch.int32))


def test_softmax_fwd_extremes():
    """Rows at +-1e4, a spike and equal values: finite, uniform rows exact."""
    import torch
    ce = _ce()
    C = 1000
    z = np.zeros((6, C), np.float32)
    z[0] = 1e4
    z[1] = -1e4
    z[2, ::2] = 1e4
    z[2, 1::2] = -1e4
    z[3, 17] = 1e4
    z[4] = 3.0
    z[5] = np.linspace(-50, 50, C, dtype=np.float32)
    for path in (0, 2, 3, 4):
        ce.force_path(path)
        y, lse = ce.softmax_fwd(_dev(z, "f32"), with_lse=True)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        assert np.isfinite(yh).all() and np.isfinite(lse.cpu().numpy()).all()
        y_ora, lse_ora = softmax_rows(z.astype(np.float64))
        check_y(yh, y_ora, "f32", f"extremes p{path}")
        check_lse(lse.cpu().numpy(), z.astype(np.float64), lse_ora, f"extremes p{path}")
        assert (yh[3, 17] == 1.0) and (np.delete(yh[3], 17) == 0).all()


def test_softmax_fwd_full_lmhead128k_sampled():
    """The 8192 x 128256 bf16 workload in the benchmark's launch
    configuration: 48 sampled rows against the oracle, and every row's sum
    within 2^-7 of 1 (bf16 rounding of 128256 values, each off by at most
    half an ulp)."""
    import torch
    ce = _ce()
    w = synth.workload("lmhead128k")
    z, _ = synth.make_workload("lmhead128k")
    zd = _dev(z, "bf16")
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(5)).choice(w.B, 48, replace=False)
    rows[:2] = [0, w.B - 1]
    z64 = widen_bf16(z[rows])
    y_ora, lse_ora = softmax_rows(z64)
    check_y(grad_to_host(y[torch.from_numpy(rows).cuda()], "bf16"), y_ora, "bf16", "lmhead128k")
    check_lse(lse.cpu().numpy()[rows], z64, lse_ora, "lmhead128k")
    s = y.float().sum(dim=1).cpu().numpy()
    assert np.abs(s - 1.0).max() <= 2.0 ** -7


# --------------------------------------------------------------- backward

BWD_SHAPES = [
    (8, 10, "f32"),
    (7, 1, "f32"),
    (300, 3, "bf16"),
    (129, 100, "bf16"),
    (64, 256, "f32"),
    (64, 257, "bf16"),
    (1024, 1000, "f32"),
    (33, 4099, "f32"),
    (17, 12345, "bf16"),
    (20, 50257, "f32"),
    (9, 128256, "bf16"),
    (3, 200_000, "bf16"),
    (5, 128256, "f32"),
    (2, 262_144, "bf16"),
    # path 5: attention-shaped rows, 8- and 4-byte vectors, 8 KB rows
    (77, 2048, "bf16"),
    (45, 300, "bf16"),
    (31, 1002, "bf16"),
    (19, 2047, "f32"),
    (11, 4096, "bf16"),
]
BWD_IDS = [f"{b}x{c}-{d}" for b, c, d in BWD_SHAPES]


def _bwd_legal(path, C, dtype, in_place=False):
    es = 4 if dtype == "f32" else 2
    if path == 1:
        return C <= 256
    if path == 2:
        return (C * es + 15) // 16 + 1 <= 8192
    if path == 4:
        return not in_place and 128 <= C // (16 // es) <= 32768
    if path == 5:
        return wave_bwd_takes(C, es)
    return path in (0, 3)


def check_dx(dx_host, y64, dy64, dtype, where):
    dx_ora = softmax_bwd_rows(y64, dy64)
    C = y64.shape[1]
    g = 2.0 ** -24 * (16 + C / 256) * np.abs(y64 * dy64).sum(axis=1, keepdims=True)
    tol = np.abs(y64) * g + 2.0 ** -22 * np.abs(dx_ora)
    if dtype == "f32":
        got = dx_host.astype(np.float64)
    else:
        got = widen_bf16(dx_host)
        tol = tol + 2.0 ** -7 * np.abs(dx_ora)
        tiny = (np.abs(dx_ora) < 2.0 ** -126) & (np.abs(got) < 2.0 ** -126)
        tol = np.where(tiny, np.inf, tol)
    err = np.abs(got - dx_ora)
    assert np.isfinite(got).all(), where
    bad = err > tol
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: dx error {err[r, c]:.3g} > {tol[r, c]:.3g} at row {r} "
                             f"col {c}: gpu {got[r, c]!r} oracle {dx_ora[r, c]!r}")
    return float((err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype", BWD_SHAPES, ids=BWD_IDS)
def test_softmax_bwd_matches_oracle(B, C, dtype, path):
    import torch
    ce = _ce()
    if not _bwd_legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    y = synth.simplex_rows(B, C, dtype, seed=B + 3 * C)
    dy, _ = synth.make_inputs(B, C, dtype, 1.0, seed=B + 5 * C)
    dx = ce.softmax_bwd(_dev(y, dtype), _dev(dy, dtype))
    torch.cuda.synchronize()
    r = check_dx(grad_to_host(dx, dtype), widen_rows(y, dtype), widen_rows(dy, dtype), dtype,
                 f"{B}x{C} {dtype} p{path}")
    print(f"[softmax] bwd {B}x{C} {dtype} p{path}: worst error / bar {r:.3g}", flush=True)


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype", [(64, 200, "f32"), (40, 50257, "f32"), (9, 128256, "bf16")])
def test_softmax_bwd_chain_to_cross_entropy(B, C, dtype, path):
    """The softmax of logits (from the oracle; a quarter of the rows with a
    +1e4 spike, half of those on the target) and the upstream gradient of
    the loss -ln y_t / B: the backward gives the cross-entropy gradient
    (softmax - onehot) / B of the CE oracle, to the backward's bar."""
    import torch
    ce = _ce()
    if not _bwd_legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, "f32", 3.0, seed=C)
    cols = synth.spike_columns(B, C, seed=C)
    q = max(1, B // 4)
    z[np.arange(q), cols[:q]] = 1.0e4
    t[: q // 2 + 1] = cols[: q // 2 + 1].astype(np.int32)
    y_ora, _ = softmax_rows(z.astype(np.float64))
    yq = y_ora.astype(np.float32) if dtype == "f32" else rne_bf16_bits(y_ora)
    y64 = widen_rows(yq, dtype)
    rows = np.arange(B)
    dy64 = np.zeros_like(y64)
    keep = y64[rows, t] > 0
    dy64[rows[keep], t[keep]] = -1.0 / (B * y64[rows[keep], t[keep]])
    dyq = dy64.astype(np.float32) if dtype == "f32" else rne_bf16_bits(dy64)
    dx = ce.softmax_bwd(_dev(yq, dtype), _dev(dyq, dtype))
    torch.cuda.synchronize()
    check_dx(grad_to_host(dx, dtype), y64, widen_rows(dyq, dtype), dtype, f"chain {B}x{C} p{path}")
    if dtype == "f32":
        # and against the CE oracle directly, where the rounding of y is
        # below the bar
        _, g = ce_rows(z.astype(np.float64), t, B)
        got = dx.cpu().numpy().astype(np.float64)
        assert np.abs(got[keep] - g[keep]).max() <= 1e-6


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype", [(64, 200, "bf16"), (33, 4099, "f32"), (9, 128256, "bf16")])
def test_softmax_bwd_in_place(B, C, dtype, path):
    """dx == dy and dx == y give the bits of the out-of-place call on the
    same path; forced row parts refuse to run in place, and automatic
    selection runs long rows in place on path 3."""
    import torch
    ce = _ce()
    if path == 4 and _bwd_legal(4, C, dtype):
        ce.force_path(4)
        y = _dev(synth.simplex_rows(B, C, dtype, seed=C), dtype)
        a = _dev(synth.make_inputs(B, C, dtype, 1.0, seed=C + 1)[0], dtype)
        with pytest.raises(ce.CEError):
            ce.softmax_bwd_into(y, a, a)
        return
    if not _bwd_legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    yh = synth.simplex_rows(B, C, dtype, seed=C)
    dyh = synth.make_inputs(B, C, dtype, 1.0, seed=C + 1)[0]
    y, dy = _dev(yh, dtype), _dev(dyh, dtype)
    ref = ce.softmax_bwd(y, dy)
    a = dy.clone()
    ce.softmax_bwd_into(y, a, a)
    b = y.clone()
    ce.softmax_bwd_into(b, dy, b)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(b))
    if path == 0 and _bwd_legal(4, C, dtype) and not _bwd_legal(2, C, dtype):
        # out of place these rows run as row parts, in place on path 3: both
        # against the oracle
        check_dx(grad_to_host(a, dtype), widen_rows(yh, dtype), widen_rows(dyh, dtype), dtype,
                 f"in place {B}x{C}")
        return
    assert torch.equal(_bits(a), _bits(ref))


def test_softmax_bwd_full_lmhead128k_sampled():
    """8192 x 128256 bf16, the benchmark's launch configuration: 32 sampled
    rows against the oracle."""
    import torch
    ce = _ce()
    B, C = 8192, 128256
    y = synth.simplex_rows(B, C, "bf16", seed=11)
    dy, _ = synth.make_inputs(B, C, "bf16", 1.0, seed=12)
    dx = ce.softmax_bwd(_dev(y, "bf16"), _dev(dy, "bf16"))
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(6)).choice(B, 32, replace=False)
    rows[:2] = [0, B - 1]
    check_dx(grad_to_host(dx[torch.from_numpy(rows).cuda()], "bf16"), widen_bf16(y[rows]),
             widen_bf16(dy[rows]), "bf16", "lmhead128k bwd")


@pytest.mark.parametrize("B,C,dtype", [(16, 300, "f32"), (8, 50257, "f32"), (4, 128256, "bf16")])
def test_softmax_autograd(B, C, dtype):
    """ce.softmax as a torch autograd function: forward and backward against
    the oracle."""
    import torch
    ce = _ce()
    z, _ = synth.make_inputs(B, C, dtype, 3.0, seed=C + 2)
    dy, _ = synth.make_inputs(B, C, dtype, 1.0, seed=C + 3)
    x = _dev(z, dtype).requires_grad_(True)
    y = ce.softmax(x)
    y.backward(_dev(dy, dtype))
    torch.cuda.synchronize()
    y_host = grad_to_host(y.detach(), dtype)
    y_ora, _ = softmax_rows(widen_rows(z, dtype))
    check_y(y_host, y_ora, dtype, "autograd fwd")
    check_dx(grad_to_host(x.grad, dtype), widen_rows(y_host, dtype), widen_rows(dy, dtype), dtype,
             "autograd bwd")


@pytest.mark.parametrize("B,C,dtype", [(16, 128256, "bf16"), (9, 50257, "f32"), (5, 99999, "f16"),
                                       (33, 70001, "bf16"), (5, 128256, "f32"), (3, 200_000, "bf16"),
                                       (2, 262_144, "f16")])
def test_softmax_bwd_parts_fallback_is_bitwise(B, C, dtype):
    """Row parts of the backward with no polls: every part recomputes the
    other parts' partial dots; the bits equal those of the exchange, and the
    device counter sees every missing partial (four parts up to a body of
    16384 vectors, eight beyond)."""
    import torch
    ce = _ce()
    if dtype == "f16":
        y = _dev(synth.simplex_rows(B, C, "f16", seed=C), "f16")
        dy = _dev(synth.make_inputs(B, C, "f16", 1.0, seed=C + 1)[0], "f16")
    else:
        y = _dev(synth.simplex_rows(B, C, dtype, seed=C), dtype)
        dy = _dev(synth.make_inputs(B, C, dtype, 1.0, seed=C + 1)[0], dtype)
    ce.force_path(4)
    prev = ce.part_polls(64)
    counter = torch.zeros(1, dtype=torch.int32, device=y.device)
    ce.part_counter(counter)
    try:
        dx1 = ce.softmax_bwd(y, dy)
        torch.cuda.synchronize()
        ce.part_polls(0)
        counter.zero_()
        dx2 = ce.softmax_bwd(y, dy)
        torch.cuda.synchronize()
        n = int(counter.item())
    finally:
        ce.part_counter(None)
        ce.part_polls(prev)
    P = 4 if C // (4 if dtype == "f32" else 8) <= 16384 else 8
    assert n == B * P * (P - 1)
    assert torch.equal(_bits(dx1), _bits(dx2))
