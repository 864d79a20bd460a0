"""The backward of the fused loss: the gradient formed in the forward times
the upstream gradient of the loss, a device scalar.

* ce_fwd_grad_scaled folds a known scale into the forward pass: its
  gradient is compared with the fp64 oracle's gradient times the scale, to
  the parity bars (fp32: absolute error 1e-6 times max(1, |s|); bf16: 1 ulp
  of the nearest-even rounding of the oracle's value times s).
* ce_scale_grad scales a stored gradient in place.  One fp32 multiply and
  one rounding: fp32 results equal the fp32 product; bf16 results are
  within 1 ulp of the nearest-even rounding of the exact product of the
  stored value and s (they equal it unless a double rounding lands on a
  tie), and equal the fused result exactly when s is a power of two and
  the values are not subnormal.
* cross_entropy_loss is a torch.autograd.Function over the two."""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import ce_rows, rne_bf16_bits, widen_bf16

from _parity import path_takes, BF16_MAX_ULP, F32_GRAD_ATOL, bf16_order, grad_to_host, to_device, widen_rows

pytestmark = pytest.mark.gpu

SHAPES = [
    (16, 10, "f32", 20.0),
    (64, 1000, "f32", 2.0),
    (9, 50257, "f32", 3.0),
    (6, 128256, "bf16", 4.0),
    (33, 4099, "bf16", 4.0),
    (5, 70001, "bf16", 4.0),
]
IDS = [f"{b}x{c}-{d}" for b, c, d, _ in SHAPES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _reset_path():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _scalar(x, device):
    import torch
    return torch.tensor([x], dtype=torch.float32, device=device)


def _check_scaled(g_host, z, t, dtype, s, where):
    B = z.shape[0]
    _, g64 = ce_rows(widen_rows(z, dtype), t, B)
    want = g64 * s
    if dtype == "f32":
        err = np.abs(g_host.astype(np.float64) - want)
        assert err.max() <= F32_GRAD_ATOL * max(1.0, abs(s)), (where, err.max())
        return float(err.max())
    ulp = np.abs(bf16_order(g_host) - bf16_order(rne_bf16_bits(want)))
    slack = np.abs(widen_bf16(g_host) - want) <= 2.0 ** -50 / B * max(1.0, abs(s))
    bad = (ulp > BF16_MAX_ULP) & ~slack
    assert not bad.any(), (where, int(ulp.max()))
    return int(ulp.max())


@pytest.mark.parametrize("s", [0.5, 3.0, -1.25, 0.0])
@pytest.mark.parametrize("path", [0, 2, 3, 4, 5], ids=["auto", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_fused_scale_matches_oracle(B, C, dtype, sigma, path, s):
    import torch
    ce = _ce()
    if path == 4 and not path_takes(4, C, dtype):
        pytest.skip("row too long for the row parts")
    if path == 2 and (C * (4 if dtype == "f32" else 2) + 15) // 16 + 1 > 16384:
        pytest.skip("row too long for the resident path")
    if path == 5 and not path_takes(5, C, dtype):
        pytest.skip("rows that path 5 does not take")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C + 7)
    zd, td = to_device(z, t, dtype)
    g = torch.empty_like(zd)
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    ce.fwd_grad_scaled_into(zd, td, g, lr, _scalar(s, zd.device))
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    assert torch.equal(lr.view(torch.int32), l0.view(torch.int32))   # the loss is not scaled
    worst = _check_scaled(grad_to_host(g, dtype), z, t, dtype, s, f"{B}x{C} {dtype} p{path} s={s}")
    print(f"[scale] fused {B}x{C} {dtype} p{path} s={s}: worst {worst}", flush=True)


@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_fused_scale_one_is_unscaled(B, C, dtype, sigma):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C + 8)
    zd, td = to_device(z, t, dtype)
    g = torch.empty_like(zd)
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    ce.fwd_grad_scaled_into(zd, td, g, lr, _scalar(1.0, zd.device))
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(g.view(view), g0.view(view))


@pytest.mark.parametrize("s", [1.0, 0.25, 3.0, -0.7])
@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_scale_grad_in_place(B, C, dtype, sigma, s):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C + 9)
    zd, td = to_device(z, t, dtype)
    g, _ = ce.fwd_grad(zd, td)
    before = grad_to_host(g, dtype).copy()
    ce.scale_grad_(g, _scalar(s, zd.device))
    torch.cuda.synchronize()
    after = grad_to_host(g, dtype)
    if dtype == "f32":
        want = (before.astype(np.float32) * np.float32(s)).astype(np.float32)
        assert np.array_equal(after.view(np.uint32), want.view(np.uint32))
    else:
        exact = widen_bf16(before) * s
        ulp = np.abs(bf16_order(after) - bf16_order(rne_bf16_bits(exact)))
        assert ulp.max() <= 1, int(ulp.max())
        if s in (1.0, 0.25):
            assert np.array_equal(after, rne_bf16_bits(exact))
    if s == 1.0:
        assert np.array_equal(after.view(np.uint8), before.view(np.uint8))
    if math.log2(abs(s)).is_integer():
        # a power-of-two scale commutes with rounding above the subnormal
        # range: the fused result is the same bits there
        gs = torch.empty_like(zd)
        lr = torch.empty(B, dtype=torch.float32, device=zd.device)
        ce.fwd_grad_scaled_into(zd, td, gs, lr, _scalar(s, zd.device))
        torch.cuda.synchronize()
        a = g.float().abs().cpu().numpy()
        b = gs.float().abs().cpu().numpy()
        normal = (a >= 2.0 ** -126) | (b >= 2.0 ** -126)
        view = torch.int16 if dtype == "bf16" else torch.int32
        ga = g.view(view).cpu().numpy()
        gb = gs.view(view).cpu().numpy()
        assert np.array_equal(ga[normal], gb[normal])
        assert (a[~normal] < 2.0 ** -126).all() and (b[~normal] < 2.0 ** -126).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset,n", [(0, 1), (1, 7), (3, 70001), (0, 9 * 8192 * 8 + 5), (5, 131072)])
def test_scale_grad_edges_and_guard_bands(dtype, offset, n):
    """Any element alignment and length: every element scaled, none outside."""
    import torch
    ce = _ce()
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    gen = torch.Generator().manual_seed(n + offset)
    base = torch.randn(offset + n + 64, generator=gen).to(tdt).cuda()
    ref = base.clone()
    ce.scale_grad_(base[offset:offset + n], _scalar(-2.0, base.device))
    torch.cuda.synchronize()
    assert torch.equal(base[:offset], ref[:offset])
    assert torch.equal(base[offset + n:], ref[offset + n:])
    assert torch.equal(base[offset:offset + n], ref[offset:offset + n] * -2)


@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_autograd_function(B, C, dtype, sigma):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C + 10)
    zd, td = to_device(z, t, dtype)
    # upstream gradient 1: the stored gradient itself, bitwise
    x = zd.clone().requires_grad_(True)
    loss = ce.cross_entropy_loss(x, td)
    loss.backward()
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(x.grad.view(view), g0.view(view))
    assert abs(loss.item() - ce.reduce_loss(l0).item()) == 0.0
    # upstream gradient 4 (a power of two: exact) through an ordinary torch op
    y = zd.clone().requires_grad_(True)
    (ce.cross_entropy_loss(y, td) * 4.0).backward()
    torch.cuda.synchronize()
    _check_scaled(grad_to_host(y.grad, dtype), z, t, dtype, 4.0, f"autograd {B}x{C} {dtype}")
    # upstream gradient 2.5: one more rounding of the stored gradient
    w = zd.clone().requires_grad_(True)
    (ce.cross_entropy_loss(w, td) * 2.5).backward()
    torch.cuda.synchronize()
    stored = grad_to_host(g0, dtype)
    got = grad_to_host(w.grad, dtype)
    if dtype == "f32":
        want = (stored * np.float32(2.5)).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    else:
        ulp = np.abs(bf16_order(got) - bf16_order(rne_bf16_bits(widen_bf16(stored) * 2.5)))
        assert ulp.max() <= 1


def test_autograd_backward_once():
    import torch
    ce = _ce()
    z, t = synth.make_inputs(8, 100, "f32", 2.0, seed=1)
    zd, td = to_device(z, t, "f32")
    x = zd.clone().requires_grad_(True)
    loss = ce.cross_entropy_loss(x, td)
    loss.backward(retain_graph=True)
    with pytest.raises(RuntimeError, match="once per forward"):
        loss.backward()
