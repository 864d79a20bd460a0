"""ce_reduce_loss_noalloc: the batch sum with no workspace argument, its
first level's partial sums in the library's per-GPU scratch array.  Called
through the C ABI and compared with ce_reduce_loss (workspace passed in)
bit for bit, on two calls in a row (the second smaller), with the scratch
holding the first call's partials when the second runs; both against the
exactly rounded sum of the same float32 values."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

from oracle import reduce_loss

pytestmark = pytest.mark.gpu


def _rows(B, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.random(B, dtype=np.float32) * 3.0 / B).astype(np.float32)


def _noalloc(xd, out):
    import torch
    import softmax_cross_entropy_ce_amd as ce
    st = ce.lib().ce_reduce_loss_noalloc(ctypes.c_void_p(xd.data_ptr()), xd.shape[0],
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, ce.status_string(st)


@pytest.mark.parametrize("sizes", [(2_097_152, 100_003), (3_000_001, 16_385), (65_536, 7)])
def test_noalloc_matches_workspace_reduce(sizes):
    import torch
    import softmax_cross_entropy_ce_amd as ce
    for i, B in enumerate(sizes):
        x = _rows(B, seed=B + i)
        xd = torch.from_numpy(x).cuda()
        got = torch.full((1,), float("nan"), dtype=torch.float32, device=xd.device)
        _noalloc(xd, got)
        want = ce.reduce_loss(xd)
        torch.cuda.synchronize()
        print(f"[noalloc] call {i} B={B}: {got.item()!r} vs {want.item()!r}", flush=True)
        assert got.view(torch.int32).item() == want.view(torch.int32).item(), (i, B)
        exact = reduce_loss(x.astype(np.float64))
        assert abs(got.item() - exact) <= 2e-6 * abs(exact), (i, B)


def test_noalloc_rejects_out_of_range_sizes():
    import torch
    import softmax_cross_entropy_ce_amd as ce
    L = ce.lib()
    xd = torch.ones(8, dtype=torch.float32, device="cuda:0")
    out = torch.empty(1, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for B in (0, -3, (1 << 31), (1 << 40)):
        st = L.ce_reduce_loss_noalloc(ctypes.c_void_p(xd.data_ptr()), B,
                                      ctypes.c_void_p(out.data_ptr()), stream)
        assert st == -2, (B, st)   # CE_ERR_SHAPE, before any launch
    assert L.ce_reduce_loss_noalloc(None, 8, ctypes.c_void_p(out.data_ptr()), stream) == -1
