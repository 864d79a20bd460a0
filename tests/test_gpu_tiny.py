"""Path 1's tiny-row kernel (rows of at most 64 bytes, one row per lane
from LDS) on the GPU against the fp64 oracle, in every layout it has.

Rows of a multiple of 16 bytes sit in LDS at a padded, odd stride of
32-bit words; other rows keep the packed layout.  16-bit rows of at most 8
elements take four rows per lane, other rows of at most 32 bytes two.  Each
wave owns one chunk of 64 x R rows in its own LDS slot (four waves per
workgroup), and the last, partial chunk moves element by element: the
large cases have thousands of chunks and a ragged last one, the small ones
put the call's end at every position of a chunk, a wave and a workgroup.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import rne_bf16_bits, softmax_rows

from _parity import bf16_order, full_parity, grad_to_host, to_device, widen_rows

pytestmark = pytest.mark.gpu

# (B, C, dtype): padded rows (16, 32, 48, 64 bytes), packed rows with two
# or four rows per thread and with one
CASES = [
    (1_500_001, 16, "f32"),     # 64 B, padded, one row per thread
    (1_200_001, 8, "f32"),      # 32 B, padded, two rows per thread
    (2_000_003, 2, "f32"),      # 8 B, packed, two rows per lane
    (700_001, 6, "f32"),        # 24 B, packed, two rows per thread
    (1_000_003, 32, "bf16"),    # 64 B, padded
    (999_999, 24, "bf16"),      # 48 B, padded
    (1_500_007, 12, "bf16"),    # 24 B, packed, two rows per thread
    (3_000_001, 4, "bf16"),     # 8 B, packed, four rows per lane
    (1_100_000, 9, "bf16"),     # 18 B, packed (rows not whole words), two per thread
    (257, 16, "f32"),           # one partial chunk, padded
    (1000, 4, "f32"),           # partial chunk, 16 B padded rows, two per thread
    (3, 32, "bf16"),
    # the end of the call at the edges of a chunk (64 x R rows), of a wave's
    # slot and of a workgroup's four waves
    (63, 10, "f32"), (64, 10, "f32"), (65, 10, "f32"), (255, 10, "f32"), (256, 10, "f32"),
    (257, 10, "f32"), (129, 6, "f32"), (511, 8, "bf16"), (513, 8, "bf16"), (1, 3, "f16"),
    (4 * 64 * 3 + 64 + 17, 12, "bf16"), (1023, 7, "f16"), (640, 16, "bf16"),
]
IDS = [f"{b}x{c}-{d}" for b, c, d in CASES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.mark.parametrize("B,C,dtype", CASES, ids=IDS)
def test_tiny_matches_oracle(B, C, dtype):
    import torch
    ce = _ce()
    assert ce.select_path(C, 0 if dtype == "f32" else 1) == 1
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + C)
    worst = full_parity(z, t, dtype, where=f"tiny {B}x{C} {dtype}")
    print(f"[tiny] {B}x{C} {dtype}: {worst}", flush=True)
    # the loss alone runs the same kernel without the gradient: the same bits
    zd, td = to_device(z, t, dtype)
    _, l_full = ce.fwd_grad(zd, td)
    l_only = ce.fwd_loss(zd, td)
    torch.cuda.synchronize()
    assert torch.equal(l_only.view(torch.int32), l_full.view(torch.int32))


@pytest.mark.parametrize("B,C,dtype", [(1_200_001, 8, "f32"), (1_000_003, 32, "bf16"),
                                       (2_000_003, 2, "f32"), (1_500_007, 12, "bf16")])
def test_tiny_softmax_matches_oracle(B, C, dtype):
    import torch
    ce = _ce()
    z, _ = synth.make_inputs(B, C, dtype, 3.0, seed=C + 3)
    zd, _ = to_device(z, np.zeros(B, np.int32), dtype)
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    yh, lh = grad_to_host(y, dtype), lse.cpu().numpy()
    step = 1 << 18
    for lo in range(0, B, step):
        z64 = widen_rows(z[lo:lo + step], dtype)
        y_ora, lse_ora = softmax_rows(z64)
        if dtype == "f32":
            assert np.abs(yh[lo:lo + step].astype(np.float64) - y_ora).max() <= 1e-6
        else:
            assert np.abs(bf16_order(yh[lo:lo + step]) - bf16_order(rne_bf16_bits(y_ora))).max() <= 1
        tol = 2.0 ** -20 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0)
        assert (np.abs(lh[lo:lo + step] - lse_ora) <= tol).all()
