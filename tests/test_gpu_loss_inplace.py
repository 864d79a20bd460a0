"""Loss-only forward (ce_fwd_loss) and the gradient in place of the logits
(ce_fwd_grad with grad_out == logits), against the fp64 oracle on the same
seeded inputs, to the parity bars of the full path."""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import ce_rows, reduce_loss

from _parity import path_takes, compare_block, compare_scalar, grad_to_host, to_device, widen_rows

pytestmark = pytest.mark.gpu

SHAPES = [
    (8, 10, "f32", 1.0),
    (300, 7, "f32", 20.0),
    (129, 100, "bf16", 4.0),
    (64, 257, "bf16", 3.0),
    (1024, 1000, "f32", 2.0),
    (33, 4099, "f32", 3.0),
    (17, 12345, "bf16", 4.0),
    (9, 50257, "f32", 3.0),
    (6, 128256, "bf16", 4.0),
    (300, 70001, "bf16", 4.0),
    (3, 200_000, "bf16", 4.0),
]
IDS = [f"{b}x{c}-{d}" for b, c, d, _ in SHAPES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


@pytest.fixture(autouse=True)
def _reset_path():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _legal(path, C, dtype):
    return path_takes(path, C, dtype)


def _multi_part(C, dtype):
    """Rows that path 4 cuts into several parts (an aligned body of 10241
    to 65536 16-byte vectors)."""
    nb = C // (4 if dtype == "f32" else 8)
    return 10 * 1024 < nb <= 64 * 1024


def _check_losses(lr_gpu, z, t, dtype, where, B=None):
    """Per-row losses against the oracle; B is the batch of the call (the
    1/B scale), which may be more than the rows compared."""
    C = z.shape[1]
    B = z.shape[0] if B is None else B
    l_ora, _ = ce_rows(widen_rows(z, dtype), t, B)
    tol = 1e-5 * (np.abs(widen_rows(z, dtype).max(axis=1)) + math.log(C) + 1.0) / B
    err = np.abs(lr_gpu.astype(np.float64) - l_ora)
    assert (err <= tol).all(), (where, float(err.max()))
    return l_ora


@pytest.mark.parametrize("path", [0, 1, 2, 3, 5], ids=["auto", "short", "resident", "long", "wave"])
@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_loss_only_matches_oracle(B, C, dtype, sigma, path):
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B * 3 + C)
    zd, td = to_device(z, t, dtype)
    lr = ce.fwd_loss(zd, td)
    loss = ce.reduce_loss(lr)
    torch.cuda.synchronize()
    l_ora = _check_losses(lr.cpu().numpy(), z, t, dtype, f"{B}x{C} {dtype} p{path}")
    compare_scalar(float(loss.item()), reduce_loss(l_ora), dtype, f"loss-only {B}x{C}")
    # where the loss alone runs the kernel configuration of the full call,
    # the same bits (path 2 picks wider workgroups for the loss alone
    # between 1024 and 4096 vectors, and no LDS prefetch above 8192; path 5
    # runs one kernel for both)
    nv = (C * (4 if dtype == "f32" else 2) + 15) // 16 + 1
    if path in (1, 3, 5) or (path == 2 and (nv <= 1024 or 4096 < nv <= 8192)):
        _, lr_full = ce.fwd_grad(zd, td)
        torch.cuda.synchronize()
        assert torch.equal(lr.view(torch.int32), lr_full.view(torch.int32))


def test_loss_only_refuses_forced_parts():
    ce = _ce()
    z, t = synth.make_inputs(4, 50257, "f32", 3.0, seed=1)
    zd, td = to_device(z, t, "f32")
    ce.force_path(4)
    with pytest.raises(ce.CEError):
        ce.fwd_loss(zd, td)


def test_loss_only_invalid_targets_and_spikes():
    import torch
    ce = _ce()
    B, C = 40, 50257
    z, t = synth.make_inputs(B, C, "f32", 3.0, spike=1e4, seed=11)
    t[:5] = synth.spike_columns(B, C, seed=11)[:5].astype(np.int32)
    t[7] = -1
    t[8] = C
    zd, td = to_device(z, t, "f32")
    lr = ce.fwd_loss(zd, td).cpu().numpy()
    assert np.isnan(lr[7]) and np.isnan(lr[8])
    keep = [i for i in range(B) if i not in (7, 8)]
    _check_losses(lr[keep], z[keep], t[keep], "f32", "spikes", B=B)


@pytest.mark.parametrize("path", [0, 1, 2, 3, 4, 5], ids=["auto", "short", "resident", "long", "parts", "wave"])
@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_in_place_matches_oracle(B, C, dtype, sigma, path):
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B * 5 + C)
    zd, td = to_device(z, t, dtype)
    buf = zd.clone()
    if path == 4 and _multi_part(C, dtype):
        # without the in-place workspace (ce_fwd_grad), forcing path 4 in
        # place is refused
        with pytest.raises(ce.CEError):
            ce.fwd_grad_into(buf, td, buf, torch.empty(B, dtype=torch.float32, device=zd.device))
    lr = ce.fwd_grad_inplace_(buf, td)
    torch.cuda.synchronize()
    g = grad_to_host(buf, dtype)
    worst, l_ora = compare_block(g, lr.cpu().numpy(), z, t, B, dtype, where=f"in place {B}x{C} p{path}")
    print(f"[in-place] {B}x{C} {dtype} p{path}: {worst}", flush=True)
    if path in (0, 4) and _multi_part(C, dtype):
        # the in-place part kernel: the same bits when (nearly) every part
        # but one defers its gradient to a partner
        prev = ce.part_polls(0)
        buf2 = zd.clone()
        lr2 = ce.fwd_grad_inplace_(buf2, td)
        ce.part_polls(prev)
        torch.cuda.synchronize()
        assert torch.equal(_bits(buf2), _bits(buf)) and torch.equal(_bits(lr2), _bits(lr))
        return
    # the same kernel out of place: the same bits
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(buf.view(view), g0.view(view))
    assert torch.equal(lr.view(torch.int32), l0.view(torch.int32))


def test_in_place_autograd_style_loop():
    """Several in-place calls in a row on fresh logits (ce_fwd_grad, no
    workspace, so two-part rows run on path 2): each matches the
    out-of-place result of its kernel."""
    import torch
    ce = _ce()
    for seed in range(3):
        z, t = synth.make_inputs(16, 128256, "bf16", 4.0, seed=100 + seed)
        zd, td = to_device(z, t, "bf16")
        buf = zd.clone()
        ce.fwd_grad_into(buf, td, buf, torch.empty(16, dtype=torch.float32, device=zd.device))
        ce.force_path(2)
        g0, _ = ce.fwd_grad(zd, td)
        ce.force_path(0)
        torch.cuda.synchronize()
        assert torch.equal(buf.view(torch.int16), g0.view(torch.int16))
