"""The LDS-staged kernel (contiguous rows of more than 64 bytes whose length
in bytes 16 does not divide: on path 1 up to 256 elements, odd lengths or
100 or 250 bf16 elements or 50 or 130 fp32 elements; on path 2 16-bit rows
of odd length up to 1024 elements) on the GPU against the fp64 oracle.

A chunk of rows is moved between HBM and LDS with whole 16-byte vectors and
each row is reduced by a segment of 8 or 16 lanes reading its elements from
LDS.  The kernel is persistent and keeps the loads of two chunks in flight
in two register sets, so the large cases give every workgroup several
chunks (more rows than the resident grid holds), both register sets and a
ragged last chunk; the small ones a single partial chunk.  The loss alone
and the gradient in place run the same arithmetic: the same bits.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import rne_bf16_bits, softmax_rows

from _parity import bf16_order, full_parity, grad_to_host, to_device, widen_rows

pytestmark = pytest.mark.gpu

# (B, C, dtype): every configuration (2 lanes per row with 16 to 32
# elements each, 4 lanes with 10 to 24, 8 lanes with 10 to 16, 16 lanes
# with 10 to 16), odd and
# even lengths, full chunks with a ragged last one, and single partial
# chunks
CASES = [
    (400_001, 17, "bf16"),      # 2 lanes x 16 (16-bit rows from 33 bytes)
    (300_001, 31, "bf16"),      # 2 lanes x 16
    (200_001, 25, "f16"),       # 2 lanes x 16
    (3, 19, "bf16"),            # one partial chunk
    (300_001, 33, "bf16"),      # 2 lanes x 20
    (200_003, 81, "bf16"),      # 4 lanes x 24
    (250_001, 45, "bf16"),      # 2 lanes x 24
    (200_001, 49, "bf16"),      # 2 lanes x 28
    (200_001, 63, "bf16"),      # 2 lanes x 32
    (100_001, 255, "bf16"),     # 16 lanes x 16
    (150_001, 129, "bf16"),     # 16 lanes x 10
    (150_001, 71, "bf16"),      # 4 lanes x 20
    (200_001, 100, "bf16"),     # 8 lanes x 14; 200-byte rows (8-byte vectors on the short kernel)
    (120_001, 250, "bf16"),
    (250_001, 17, "f32"),       # 2 lanes x 16
    (200_001, 31, "f32"),       # 2 lanes x 16
    (150_001, 39, "f32"),       # 4 lanes x 10
    (150_001, 47, "f32"),       # 4 lanes x 12
    (100_003, 101, "f32"),      # 8 lanes x 14
    (60_001, 255, "f32"),       # 16 lanes x 16
    (100_000, 50, "f32"),       # 4 lanes x 16; 200-byte rows
    (90_001, 130, "f32"),       # 16 lanes x 10
    (150_001, 75, "bf16"),      # 4 lanes x 20
    (100_001, 127, "bf16"),     # 8 lanes x 16
    (80_001, 191, "bf16"),      # 16 lanes x 12
    (70_001, 223, "bf16"),      # 16 lanes x 14
    (100_001, 63, "f32"),       # 4 lanes x 16
    (100_001, 77, "f32"),       # 8 lanes x 10
    (60_001, 93, "f32"),        # 8 lanes x 12
    (50_001, 119, "f32"),       # 8 lanes x 16
    (40_001, 171, "f32"),       # 16 lanes x 12
    (40_001, 213, "f32"),       # 16 lanes x 14
    (60_001, 77, "f16"),
    (5, 33, "bf16"),            # one partial chunk
    (37, 101, "f32"),
    (1, 255, "bf16"),
]
IDS = [f"{b}x{c}-{d}" for b, c, d in CASES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _auto():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("B,C,dtype", CASES, ids=IDS)
def test_staged_matches_oracle(B, C, dtype):
    import torch
    ce = _ce()
    es = 4 if dtype == "f32" else 2
    assert (C * es) % 16 != 0 and C * es > (32 if es == 2 else 64)
    assert ce.select_path(C, 0 if dtype == "f32" else 1) == 1
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + 7 * C)
    # targets on the first and last element of some rows
    t[: min(B, 3)] = 0
    t[-min(B, 3):] = C - 1
    worst = full_parity(z, t, dtype, where=f"staged {B}x{C} {dtype}")
    print(f"[staged] {B}x{C} {dtype}: {worst}", flush=True)
    # the loss alone and the gradient in place: the bits of the full call
    zd, td = to_device(z, t, dtype)
    g_full, l_full = ce.fwd_grad(zd, td)
    l_only = ce.fwd_loss(zd, td)
    buf = zd.clone()
    l_in = ce.fwd_grad_inplace_(buf, td)
    torch.cuda.synchronize()
    assert torch.equal(_bits(l_only), _bits(l_full))
    assert torch.equal(_bits(l_in), _bits(l_full))
    assert torch.equal(_bits(buf), _bits(g_full))


# 16-bit rows of odd length from 257 to 1024 elements run the same kernel
# on path 2, 32 lanes per row (10 to 32 elements each)
LONG_CASES = [
    (40_001, 257, "bf16"),      # 32 lanes x 10
    (30_001, 383, "bf16"),      # x 12
    (20_001, 511, "bf16"),      # x 16
    (20_001, 601, "bf16"),      # x 20
    (15_001, 767, "bf16"),      # x 24
    (10_001, 1001, "bf16"),     # x 32
    (9_001, 1023, "f16"),
    (3, 999, "bf16"),           # one partial chunk
]
LONG_IDS = [f"{b}x{c}-{d}" for b, c, d in LONG_CASES]


@pytest.mark.parametrize("B,C,dtype", LONG_CASES, ids=LONG_IDS)
def test_staged_long_rows_match_oracle(B, C, dtype):
    import torch
    ce = _ce()
    assert ce.select_path(C, 1) == 2
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=B + 3 * C)
    t[: min(B, 2)] = 0
    t[-min(B, 2):] = C - 1
    worst = full_parity(z, t, dtype, where=f"staged long {B}x{C} {dtype}")
    print(f"[staged] {B}x{C} {dtype}: {worst}", flush=True)
    zd, td = to_device(z, t, dtype)
    g_full, l_full = ce.fwd_grad(zd, td)
    l_only = ce.fwd_loss(zd, td)
    buf = zd.clone()
    l_in = ce.fwd_grad_inplace_(buf, td)
    torch.cuda.synchronize()
    assert torch.equal(_bits(l_only), _bits(l_full))
    assert torch.equal(_bits(l_in), _bits(l_full))
    assert torch.equal(_bits(buf), _bits(g_full))


@pytest.mark.parametrize("B,C,dtype", [(200_003, 81, "bf16"), (100_003, 101, "f32"),
                                       (77, 255, "bf16"), (20_001, 701, "bf16")])
def test_staged_softmax_matches_oracle(B, C, dtype):
    import torch
    ce = _ce()
    z, _ = synth.make_inputs(B, C, dtype, 3.0, seed=C + 5)
    zd, _ = to_device(z, np.zeros(B, np.int32), dtype)
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    yh, lh = grad_to_host(y, dtype), lse.cpu().numpy()
    step = 1 << 16
    for lo in range(0, B, step):
        z64 = widen_rows(z[lo:lo + step], dtype)
        y_ora, lse_ora = softmax_rows(z64)
        if dtype == "f32":
            assert np.abs(yh[lo:lo + step].astype(np.float64) - y_ora).max() <= 1e-6
        else:
            assert np.abs(bf16_order(yh[lo:lo + step]) - bf16_order(rne_bf16_bits(y_ora))).max() <= 1
        tol = 2.0 ** -20 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0)
        assert (np.abs(lh[lo:lo + step] - lse_ora) <= tol).all()


@pytest.mark.parametrize("B,C,dtype", [(100_001, 99, "bf16"), (50_001, 63, "f32")])
def test_staged_ignore_index(B, C, dtype):
    """A quarter of the rows ignored: their loss and gradient are zero, the
    others match the oracle with the mean over the rows kept."""
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + C)
    rng = np.random.Generator(np.random.PCG64(C))
    ign = rng.random(B) < 0.25
    t[ign] = -100
    zd, td = to_device(z, t, dtype)
    g, lr = ce.fwd_grad_ex(zd, td, ignore_index=-100)
    torch.cuda.synchronize()
    gh, lh = grad_to_host(g, dtype), lr.cpu().numpy()
    assert (lh[ign] == 0).all()
    assert (gh[ign].view(np.uint32 if dtype == "f32" else np.uint16) == 0).all()
    from _parity import compare_block
    N = int((~ign).sum())
    compare_block(gh[~ign], lh[~ign], z[~ign], t[~ign], N, dtype, where=f"staged ignore {B}x{C}")


# The softmax backward of such rows: y, dy and dx staged through LDS (8, 16
# or 32 lanes per row), on path 1 and, for 16-bit rows of 257 to 512
# elements, on path 2
BWD_CASES = [
    (200_001, 33, "bf16"),      # 8 lanes
    (100_003, 81, "bf16"),      # 8 lanes
    (60_001, 255, "bf16"),      # 16 lanes
    (30_001, 301, "bf16"),      # 32 lanes, path 2
    (20_001, 511, "bf16"),      # 32 lanes, path 2
    (200_001, 17, "f32"),       # 8 lanes
    (100_001, 101, "f32"),      # 16 lanes
    (40_001, 255, "f32"),       # 32 lanes
    (7, 99, "bf16"),            # one partial chunk
]
BWD_IDS = [f"{b}x{c}-{d}" for b, c, d in BWD_CASES]


@pytest.mark.parametrize("B,C,dtype", BWD_CASES, ids=BWD_IDS)
def test_staged_softmax_bwd_matches_oracle(B, C, dtype):
    import torch
    from test_gpu_softmax import check_dx, _dev
    ce = _ce()
    y = synth.simplex_rows(B, C, dtype, seed=B + C)
    dy, _ = synth.make_inputs(B, C, dtype, 1.0, seed=B + 2 * C)
    yd, dyd = _dev(y, dtype), _dev(dy, dtype)
    dx = ce.softmax_bwd(yd, dyd)
    torch.cuda.synchronize()
    r = check_dx(grad_to_host(dx, dtype), widen_rows(y, dtype), widen_rows(dy, dtype), dtype,
                 f"staged bwd {B}x{C} {dtype}")
    print(f"[staged] bwd {B}x{C} {dtype}: worst error / bar {r:.3g}", flush=True)
    # in place of dy and of y: the same bits
    a = dyd.clone()
    ce.softmax_bwd_into(yd, a, a)
    b = yd.clone()
    ce.softmax_bwd_into(b, dyd, b)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a), _bits(dx))
    assert torch.equal(_bits(b), _bits(dx))
