"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs, element by element, on every kernel path."""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import ce_rows, reduce_loss

from _parity import (path_takes, compare_block, compare_scalar, full_parity, grad_to_host, run_gpu,
                     to_device, widen_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset_path():
    import softmax_cross_entropy_ce_amd as ce
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _force(path):
    import softmax_cross_entropy_ce_amd as ce
    ce.force_path(path)


def _log(name, worst):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3g}" for k, v in worst.items()), flush=True)


# (B, C, dtype, sigma) — several tiles and a ragged tail on every path;
# odd C makes fp32 rows 4-byte aligned and bf16 rows 2-byte aligned.
SMALL = [
    (8, 10, "f32", 1.0),
    (37, 1, "f32", 3.0),
    (5, 3, "bf16", 2.0),
    (300, 7, "f32", 20.0),
    (513, 16, "bf16", 4.0),
    (70, 33, "f32", 5.0),
    (129, 100, "bf16", 4.0),
    (257, 256, "f32", 2.0),
    (64, 257, "bf16", 3.0),
    (1024, 1000, "f32", 2.0),
    (33, 4099, "f32", 3.0),
    (17, 12345, "bf16", 4.0),
    (9, 50257, "f32", 3.0),
    (6, 128256, "bf16", 4.0),
    # rows on the LDS-prefetch kernel: partial prefetched slot with 2-byte
    # aligned rows, partial register slot, the largest resident rows, one
    # row, and more rows than the persistent grid holds
    (300, 70001, "bf16", 4.0),
    (257, 40000, "f32", 3.0),
    (3, 65531, "f32", 3.0),
    (5, 131064, "bf16", 4.0),
    (1, 128256, "bf16", 4.0),
    # row parts (path 4): the one-part configurations at their capacity,
    # two parts with 2-byte aligned bf16 rows, and two parts filling every
    # register and LDS slot
    (21, 32767, "bf16", 4.0),
    (13, 81919, "bf16", 4.0),
    (7, 99999, "bf16", 4.0),
    (11, 196607, "bf16", 4.0),
    (4, 98303, "f32", 3.0),
]

PATHS = [0, 1, 2, 3, 4, 5]
PATH_IDS = ["auto", "short", "resident", "long", "parts", "wave"]


def _legal(path, C, dtype):
    return path_takes(path, C, dtype)


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("B,C,dtype,sigma", SMALL, ids=[f"{b}x{c}-{d}" for b, c, d, _ in SMALL])
def test_parity_small(path, B, C, dtype, sigma):
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B * 1000 + C)
    _force(path)
    _log(f"{B}x{C} {dtype} path={path}", full_parity(z, t, dtype, where=f"{B}x{C} {dtype} p{path}"))


@pytest.mark.parametrize("path", [0, 2, 3, 4], ids=["auto", "resident", "long", "parts"])
def test_parity_spike_rows(path):
    """Rows with one +1e4 entry (the LM-head stability case) on a ragged
    shape, including rows whose target is the spike."""
    B, C = 40, 50257
    z, t = synth.make_inputs(B, C, "f32", 3.0, spike=1e4, seed=11)
    spikes = synth.spike_columns(B, C, seed=11)
    t[:5] = spikes[:5].astype(np.int32)
    _force(path)
    _log(f"spike path={path}", full_parity(z, t, "f32", where=f"spike p{path}"))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_parity_edge_values(path, dtype):
    """Uniform rows (loss ln C), rows of +-1e4, rows where the target holds
    nearly all the mass, and invalid targets (NaN rows)."""
    C = 200
    rng = np.random.Generator(np.random.PCG64(5))
    z = (rng.standard_normal((12, C)) * 3).astype(np.float32)
    t = rng.integers(0, C, 12).astype(np.int32)
    z[0] = 0.0
    z[1] = 1e4
    z[2] = -1e4
    z[3, ::2] = 1e4
    z[3, 1::2] = -1e4
    z[4, t[4]] = z[4].max() + 30.0       # target dominates: softmax_t ~ 1 - 1e-11
    z[5, t[5]] = z[5].max() + 12.0
    t[6] = -1                            # invalid targets
    t[7] = C
    z[8] = np.float32(2.5)
    if dtype == "bf16":
        z = synth.bf16_bits_from_f32(z)
    _force(path)
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    _log(f"edges {dtype} path={path}", full_parity(z, t, dtype, where=f"edges {dtype} p{path}"))


def test_parity_tiny_workload():
    z, t = synth.make_workload("tiny")
    _log("tiny", full_parity(z, t, "f32", where="tiny"))


def test_parity_classifier_workload():
    z, t = synth.make_workload("classifier")
    _log("classifier", full_parity(z, t, "f32", where="classifier"))


def test_parity_skinny_workload():
    """2,097,152 rows of 10 classes, sigma 20: every row compared, and the
    2M-term loss reduction."""
    z, t = synth.make_workload("skinny")
    _log("skinny", full_parity(z, t, "f32", block_elems=1 << 22, where="skinny"))


def test_parity_lmhead50k_workload():
    """4096 x 50257 fp32 with a +1e4 spike per row: every row compared."""
    z, t = synth.make_workload("lmhead50k")
    _log("lmhead50k", full_parity(z, t, "f32", block_elems=1 << 24, where="lmhead50k"))


def test_parity_lmhead128k_workload():
    """8192 x 128256 bf16 at full size in the launch configuration the
    benchmark times: every row's gradient compared with the oracle element
    by element (1 bf16 ulp from RNE of the fp64 value) and every per-row
    loss, in blocks of 64 rows on a pool of threads, and the scalar against
    the oracle's sum over all rows."""
    from concurrent.futures import ThreadPoolExecutor
    z, t = synth.make_workload("lmhead128k")
    B, C = z.shape
    z_dev, t_dev = to_device(z, t, "bf16")
    grad, loss_rows, loss = run_gpu(z_dev, t_dev)
    g_all = grad_to_host(grad, "bf16")
    lr = loss_rows.cpu().numpy()
    del grad, z_dev
    step = 64

    def block(lo):
        hi = min(B, lo + step)
        return compare_block(g_all[lo:hi], lr[lo:hi], z[lo:hi], t[lo:hi], B, "bf16",
                             where=f"lmhead128k rows {lo}:{hi}")

    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(block, range(0, B, step)))
    worst: dict = {}
    for res, _ in parts:
        for k, v in res.items():
            worst[k] = max(worst.get(k, 0), v)
    ora = np.concatenate([p[1] for p in parts])
    worst["loss_rel"] = compare_scalar(float(loss.item()), reduce_loss(ora), "bf16", "lmhead128k")
    worst["rows_compared"] = B
    _log("lmhead128k all rows", worst)


@pytest.mark.parametrize("B,C,dtype", [(8, 10, "f32"), (1024, 1000, "f32"), (37, 3000, "bf16"),
                                       (64, 128256, "bf16"), (20000, 10, "f32"), (9, 50257, "f16")],
                         ids=["8x10-f32", "1024x1000-f32", "37x3000-bf16", "64x128256-bf16",
                              "20000x10-f32", "9x50257-f16"])
def test_fwd_grad_loss_one_call(B, C, dtype):
    """ce_fwd_grad_loss (the whole step in one call): the gradient, the
    per-row losses and the batch loss bitwise those of ce_fwd_grad followed
    by ce_reduce_loss, and the batch loss against the oracle's sum; past
    16384 rows the reduction's workspace is required."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + C)
    zd, td = to_device(z, t, dtype)
    g0, l0 = ce.fwd_grad(zd, td)
    s0 = torch.empty((), dtype=torch.float32, device=zd.device)
    ce.reduce_loss_into(l0, s0)
    g1 = torch.empty_like(zd)
    l1 = torch.empty(B, dtype=torch.float32, device=zd.device)
    s1 = torch.full((), float("nan"), dtype=torch.float32, device=zd.device)
    ce.fwd_grad_loss_into(zd, td, g1, l1, s1)
    torch.cuda.synchronize()
    view = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(g1.view(view), g0.view(view))
    assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
    assert torch.equal(s1.view(torch.int32), s0.view(torch.int32))
    l_ora, _ = ce_rows(widen_rows(z, dtype), t, B)
    want = reduce_loss(l_ora)
    assert abs(float(s1.item()) - want) <= 1e-5 * abs(want) + 1e-6
    if ce.reduce_workspace_bytes(B) > 0:
        lib = ce.lib()
        st = lib.ce_fwd_grad_loss(zd.data_ptr(), td.data_ptr(), B, C, ce._dtype_code(zd),
                                  g1.data_ptr(), l1.data_ptr(), s1.data_ptr(), None, 0,
                                  ce._stream_ptr(zd.device))
        assert st == -4  # CE_ERR_WORKSPACE, nothing launched
