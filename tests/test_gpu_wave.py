"""Path 5 (whole rows in one wavefront's registers, several rows per wave)
on the GPU against the fp64 oracle, at the edges of its configurations.

The kernel's configuration follows from the row's bytes and the widest
vector (16, 8 or 4 bytes) that every row start and row length allows: 16
to 256 bytes of a row per lane, 8 rows per wave at 16 bytes down to one at
128 and 256.  The cases put rows just below and above each of those sizes,
with every vector width and dtype, row counts that leave the last wave and
workgroup partly empty, targets on a lane's first and last element and on
the last vector of a row, arrays whose base sits off a 16-byte boundary, and
each operation the path runs (the fused loss, the loss alone, in place, the
softmax and the shard records).  Where automatic selection picks path 5
(rows of up to 8 KB of 16-bit or 4 KB of fp32 elements) it gives the forced
path's bits.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import rne_bf16_bits, rne_f16_bits, softmax_rows

from _parity import (bf16_order, compare_block, f16_order, full_parity, grad_to_host, to_device,
                     wave_takes, wave_vector_bytes, widen_rows)

pytestmark = pytest.mark.gpu


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _reset_path():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _es(dtype):
    return 4 if dtype == "f32" else 2


def _auto(C, dtype):
    """The path automatic selection takes for contiguous rows (whatever path
    is forced at the moment)."""
    ce = _ce()
    prev = ce.force_path(0)
    try:
        return ce.select_path(C, {"f32": 0, "bf16": 1, "f16": 2}[dtype])
    finally:
        ce.force_path(prev)


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


# (B, C, dtype): row bytes around 1, 2, 4, 8 and 16 KB with 16-, 8- and
# 4-byte vectors; B leaves the last wave (up to 8 rows) and workgroup
# (4 waves) partly empty.
CASES = [
    (67, 258, "bf16"),      # 516 B, 4-byte vectors, 8 rows per wave
    (131, 300, "bf16"),     # 600 B, 8-byte vectors
    (45, 512, "bf16"),      # 1 KB exactly, 16-byte vectors
    (37, 514, "f16"),       # just over 1 KB: 32 bytes per lane, 4 rows per wave
    (29, 257, "f32"),       # 1028 B, 4-byte vectors
    (61, 1000, "bf16"),     # 2000 B
    (41, 1002, "bf16"),     # 2004 B, 4-byte vectors
    (50, 1000, "f32"),      # 4000 B, 16-byte vectors
    (23, 1023, "f32"),      # 4092 B, 4-byte vectors
    (33, 2048, "bf16"),     # 4 KB exactly
    (19, 2047, "f32"),      # 8188 B, 4-byte vectors (their largest)
    (25, 4096, "bf16"),     # 8 KB exactly
    (17, 2050, "f32"),      # 8200 B, 8-byte vectors: 256 bytes per lane
    (11, 6000, "bf16"),     # 12000 B
    (13, 4096, "f32"),      # 16 KB exactly
    (9, 8192, "f16"),       # 16 KB exactly
    (7, 4094, "f32"),       # 16376 B, 8-byte vectors
    (1, 3000, "bf16"),      # a single row
]
IDS = [f"{b}x{c}-{d}" for b, c, d in CASES]


def _targets_on_edges(t, C, dtype, vb):
    """Targets on the first and last elements of a row, on the last element
    of lane 63's first vector, and on the first element of the second slot
    of lane 0, where the row has them."""
    vw = vb // _es(dtype)
    picks = [0, C - 1, 64 * vw - 1, 64 * vw]
    for i, c in enumerate(picks):
        if i < len(t) and c < C:
            t[i] = c
    return t


@pytest.mark.parametrize("B,C,dtype", CASES, ids=IDS)
def test_wave_matches_oracle(B, C, dtype):
    import torch
    ce = _ce()
    es = _es(dtype)
    assert wave_takes(C, es)
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=B * 31 + C)
    t = _targets_on_edges(t, C, dtype, wave_vector_bytes(es, (C,)))
    ce.force_path(5)
    worst = full_parity(z, t, dtype, where=f"wave {B}x{C} {dtype}")
    print(f"[wave] {B}x{C} {dtype}: {worst}", flush=True)
    # where automatic selection takes path 5 (rows of up to 8 KB of 16-bit
    # or 4 KB of fp32 elements): the same kernel, the same bits
    if _auto(C, dtype) != 5:
        return
    zd, td = to_device(z, t, dtype)
    g5, l5 = ce.fwd_grad(zd, td)
    ce.force_path(0)
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g0), _bits(g5)) and torch.equal(_bits(l0), _bits(l5))


@pytest.mark.parametrize("B,C,dtype", CASES, ids=IDS)
def test_wave_loss_only_and_in_place(B, C, dtype):
    """The loss alone and the gradient in place: the bits of the fused call."""
    import torch
    ce = _ce()
    ce.force_path(5)
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + 7 * C)
    zd, td = to_device(z, t, dtype)
    g, lr = ce.fwd_grad(zd, td)
    lo = ce.fwd_loss(zd, td)
    buf = zd.clone()
    li = ce.fwd_grad_inplace_(buf, td)
    torch.cuda.synchronize()
    assert torch.equal(_bits(lo), _bits(lr))
    assert torch.equal(_bits(buf), _bits(g)) and torch.equal(_bits(li), _bits(lr))


@pytest.mark.parametrize("B,C,dtype", CASES, ids=IDS)
def test_wave_softmax_fwd(B, C, dtype):
    import torch
    ce = _ce()
    ce.force_path(5)
    z, _ = synth.make_inputs(B, C, dtype, 3.0, seed=C + 11)
    zd, _ = to_device(z, np.zeros(B, np.int32), dtype)
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    z64 = widen_rows(z, dtype)
    y_ora, lse_ora = softmax_rows(z64)
    yh = grad_to_host(y, dtype)
    if dtype == "f32":
        assert np.abs(yh.astype(np.float64) - y_ora).max() <= 1e-6
    elif dtype == "bf16":
        assert np.abs(bf16_order(yh) - bf16_order(rne_bf16_bits(y_ora))).max() <= 1
    else:
        assert np.abs(f16_order(yh) - f16_order(rne_f16_bits(y_ora))).max() <= 1
    tol = 2.0 ** -20 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0)
    assert (np.abs(lse.cpu().numpy() - lse_ora) <= tol).all()
    if _auto(C, dtype) != 5:
        return
    ce.force_path(0)
    y0 = ce.softmax_fwd(zd)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y0), _bits(y))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wave_shards(dtype):
    """Three shards whose widths fall on path 5 with different vector
    widths: records on path 5, gradient against the whole-row oracle."""
    import torch
    ce = _ce()
    B = 37
    edges = [0, 1000, 3002, 5000] if dtype == "bf16" else [0, 1000, 2047, 3000]
    C = edges[-1]
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=C + 2)
    t[0], t[1], t[2] = edges[1] - 1, edges[1], C - 1
    zd, td = to_device(z, t, dtype)
    ce.force_path(5)
    shards = [zd[:, a:b].contiguous() for a, b in zip(edges[:-1], edges[1:])]
    for s in shards:
        assert wave_takes(s.shape[1], _es(dtype))
    recs = torch.stack([ce.shard_stats(s, td, a) for s, a in zip(shards, edges[:-1])])
    out = [ce.shard_grad(s, td, a, C, recs, with_loss=True) for s, a in zip(shards, edges[:-1])]
    torch.cuda.synchronize()
    grad = torch.cat([g for g, _ in out], dim=1)
    compare_block(grad_to_host(grad, dtype), out[0][1].cpu().numpy(), z, t, B, dtype,
                  where=f"wave shards {dtype}")


@pytest.mark.parametrize("off", [1, 2, 3, 4, 6])
@pytest.mark.parametrize("B,C,dtype", [(40, 1000, "bf16"), (24, 3000, "f32"), (9, 8192, "bf16")])
def test_wave_offset_bases(B, C, dtype, off):
    """Arrays that start off elements past a 16-byte boundary: path 5 with
    the narrower vectors they allow, or the automatic fallback to path 2
    where it has none (forced path 5 then refuses the call)."""
    import torch
    ce = _ce()
    es = _es(dtype)
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=off * 100 + C)
    zd, td = to_device(z, t, dtype)
    flat = torch.empty(off + B * C + 16, dtype=zd.dtype, device=zd.device)
    zv = flat[off:off + B * C].view(B, C)
    zv.copy_(zd)
    gflat = torch.empty_like(flat)
    gv = gflat[off:off + B * C].view(B, C)
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    takes = wave_takes(C, es, (C,), (zv.data_ptr(), gv.data_ptr()))
    ce.force_path(5)
    if not takes:
        with pytest.raises(ce.CEError):
            ce.fwd_grad_into(zv, td, gv, lr)
        ce.force_path(0)
    ce.fwd_grad_into(zv, td, gv, lr)
    torch.cuda.synchronize()
    compare_block(grad_to_host(gv, dtype), lr.cpu().numpy(), z, t, B, dtype,
                  where=f"wave offset {off} {B}x{C} {dtype}")


def test_wave_ignore_index_and_stride():
    """ignore_index and a padded row stride on path 5: ignored rows exactly
    zero, the others against the oracle's mean over the rows kept."""
    import torch
    ce = _ce()
    B, C, dtype, ii = 70, 1000, "bf16", -100
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=5)
    t[::3] = ii
    zd, td = to_device(z, t, dtype)
    wide = torch.zeros((B, C + 8), dtype=zd.dtype, device=zd.device)
    view = wide[:, :C]
    view.copy_(zd)
    assert wave_takes(C, 2, (C, C + 8), (view.data_ptr(),))
    ce.force_path(5)
    g, lr = ce.fwd_grad_ex(view, td, ignore_index=ii)
    torch.cuda.synchronize()
    gh, lh = grad_to_host(g, dtype), lr.cpu().numpy()
    ign = t == ii
    assert (lh[ign] == 0).all() and (gh[ign] == 0).all()
    compare_block(gh[~ign], lh[~ign], z[~ign], t[~ign], int((~ign).sum()), dtype,
                  where="wave ignore")


@pytest.mark.parametrize("B,C,dtype", [(77, 2048, "bf16"), (19, 2047, "f32"), (45, 300, "bf16"),
                                       (11, 4096, "bf16")])
def test_wave_softmax_bwd_auto_is_path5(B, C, dtype):
    """Automatic selection runs the softmax backward of these rows on path 5:
    the forced path's bits, in place too."""
    import torch
    ce = _ce()
    y = synth.simplex_rows(B, C, dtype, seed=C)
    dy, _ = synth.make_inputs(B, C, dtype, 1.0, seed=C + 1)
    yd, _ = to_device(y, np.zeros(B, np.int32), dtype)
    dyd, _ = to_device(dy, np.zeros(B, np.int32), dtype)
    dx0 = ce.softmax_bwd(yd, dyd)
    ce.force_path(5)
    dx5 = ce.softmax_bwd(yd, dyd)
    buf = dyd.clone()
    ce.softmax_bwd_into(yd, buf, buf)
    torch.cuda.synchronize()
    assert torch.equal(_bits(dx0), _bits(dx5)) and torch.equal(_bits(buf), _bits(dx5))
