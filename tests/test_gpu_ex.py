"""fp16 logits, row-strided logits and gradients, and ignore_index, on the
GPU against the fp64 oracle.

* fp16 (the pages' F16 data type): every path of the fused loss, the
  softmax forward and backward, the shard records and gradient, and the
  backward scale, to the fp16 bars of ``_parity`` (1 fp16 ulp of the
  oracle's value rounded once, subnormals included).
* Row strides (ce_fwd_grad_ex): rows of logits and gradient inside wider
  buffers; every path against the oracle, the padding between rows left
  untouched, in place and loss only.
* ignore_index (ce_fwd_grad_ex): rows whose target equals it get loss 0 and
  a zero gradient row exactly; the other rows match the oracle's
  cross-entropy with the mean over the rows kept.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import ce_rows, ce_rows_ignore, reduce_loss, rne_f16_bits, softmax_bwd_rows, softmax_rows

from _parity import (path_takes, wave_bwd_takes, wave_takes, compare_block, compare_scalar, f16_order, full_parity, grad_to_host,
                     to_device, widen_rows)

pytestmark = pytest.mark.gpu

PATHS = [0, 1, 2, 3, 4, 5]
PATH_IDS = ["auto", "short", "resident", "long", "parts", "wave"]


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


def _legal(path, C, dtype):
    return path_takes(path, C, dtype)


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


# ------------------------------------------------------------------- fp16

F16_SHAPES = [
    (8, 10, 1.0, None),
    (300, 7, 20.0, None),
    (129, 100, 4.0, None),
    (64, 257, 3.0, None),
    (1024, 1000, 2.0, None),
    (33, 4099, 3.0, None),
    (17, 12345, 4.0, None),
    (40, 50257, 3.0, 1.0e4),
    (9, 128256, 4.0, None),
    (5, 70001, 4.0, None),
    (3, 200_000, 4.0, None),
]
F16_IDS = [f"{b}x{c}{'-spike' if s else ''}" for b, c, _, s in F16_SHAPES]


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("B,C,sigma,spike", F16_SHAPES, ids=F16_IDS)
def test_f16_fused_loss_matches_oracle(B, C, sigma, spike, path):
    ce = _ce()
    if not _legal(path, C, "f16"):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, "f16", sigma, spike=spike, seed=B + C + 16)
    if spike is not None:
        t[: B // 4] = synth.spike_columns(B, C, seed=B + C + 16)[: B // 4].astype(np.int32)
    worst = full_parity(z, t, "f16", where=f"f16 {B}x{C} p{path}")
    print(f"[f16] {B}x{C} p{path}: {worst}", flush=True)


@pytest.mark.parametrize("B,C", [(64, 200), (33, 4099), (9, 128256)])
def test_f16_loss_only_in_place_and_scale(B, C):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, "f16", 4.0, seed=C)
    zd, td = to_device(z, t, "f16")
    g0, l0 = ce.fwd_grad(zd, td)
    lr = ce.fwd_loss(zd, td)
    buf = zd.clone()
    lb = ce.fwd_grad_inplace_(buf, td)
    torch.cuda.synchronize()
    compare_block(grad_to_host(buf, "f16"), lb.cpu().numpy(), z, t, B, "f16", where="f16 in place")
    l_ora, _ = ce_rows(widen_rows(z, "f16"), t, B)
    tol = 1e-5 * (np.abs(widen_rows(z, "f16").max(axis=1)) + math.log(C) + 1.0) / B
    assert (np.abs(lr.cpu().numpy() - l_ora) <= tol).all()
    # the backward scale by -3: one float32 product rounded once, within 1
    # ulp of the exact product of the stored value
    g = g0.clone()
    ce.scale_grad_(g, torch.tensor([-3.0], device=zd.device))
    torch.cuda.synchronize()
    want = rne_f16_bits(widen_rows(grad_to_host(g0, "f16"), "f16") * -3.0)
    assert np.abs(f16_order(grad_to_host(g, "f16")) - f16_order(want)).max() <= 1


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("B,C", [(64, 200), (33, 4099), (9, 128256)])
def test_f16_softmax(B, C, path):
    """Softmax forward (1 fp16 ulp) and backward (the backward's bar with an
    fp16 ulp, 2^-10 relative or 2^-24 absolute below 2^-14)."""
    import torch
    ce = _ce()
    if not _legal(path, C, "f16"):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, _ = synth.make_inputs(B, C, "f16", 3.0, seed=C + 4)
    zd, _ = to_device(z, np.zeros(B, np.int32), "f16")
    y, lse = ce.softmax_fwd(zd, with_lse=True)
    torch.cuda.synchronize()
    z64 = widen_rows(z, "f16")
    y_ora, lse_ora = softmax_rows(z64)
    yh = grad_to_host(y, "f16")
    assert np.abs(f16_order(yh) - f16_order(rne_f16_bits(y_ora))).max() <= 1
    tol = 2.0 ** -20 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0)
    assert (np.abs(lse.cpu().numpy() - lse_ora) <= tol).all()
    if path == 4 or (path == 5 and not wave_bwd_takes(C, 2)) or \
            (path == 2 and (C * 2 + 15) // 16 + 1 > 8192):
        return  # no backward for these rows on the forced path
    dy, _ = synth.make_inputs(B, C, "f16", 1.0, seed=C + 5)
    dyd, _ = to_device(dy, np.zeros(B, np.int32), "f16")
    dx = ce.softmax_bwd(y, dyd)
    torch.cuda.synchronize()
    y64, dy64 = widen_rows(yh, "f16"), widen_rows(dy, "f16")
    dx_ora = softmax_bwd_rows(y64, dy64)
    gdot = 2.0 ** -24 * (16 + C / 256) * np.abs(y64 * dy64).sum(axis=1, keepdims=True)
    bar = np.abs(y64) * gdot + 2.0 ** -22 * np.abs(dx_ora) + np.maximum(2.0 ** -10 * np.abs(dx_ora),
                                                                         2.0 ** -24)
    err = np.abs(widen_rows(grad_to_host(dx, "f16"), "f16") - dx_ora)
    assert (err <= bar).all(), float((err / bar).max())


def test_f16_shards():
    B, C = 33, 12345
    edges = [0, 5000, 12345]
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, "f16", 4.0, seed=21)
    zd, td = to_device(z, t, "f16")
    shards = [zd[:, a:b].contiguous() for a, b in zip(edges[:-1], edges[1:])]
    recs = torch.stack([ce.shard_stats(s, td, a) for s, a in zip(shards, edges[:-1])])
    out = [ce.shard_grad(s, td, a, C, recs, with_loss=True) for s, a in zip(shards, edges[:-1])]
    torch.cuda.synchronize()
    grad = torch.cat([g for g, _ in out], dim=1)
    compare_block(grad_to_host(grad, "f16"), out[0][1].cpu().numpy(), z, t, B, "f16",
                  where="f16 shards")


def test_f16_full_lmhead128k_sampled():
    """8192 x 128256 fp16, N(0, 4): 48 sampled rows and the scalar loss
    against the oracle."""
    import torch
    ce = _ce()
    B, C = 8192, 128256
    z, t = synth.make_inputs(B, C, "f16", 4.0, seed=0)
    zd, td = to_device(z, t, "f16")
    g, lr = ce.fwd_grad(zd, td)
    loss = ce.reduce_loss(lr)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(9)).choice(B, 48, replace=False)
    rows[:2] = [0, B - 1]
    compare_block(grad_to_host(g[torch.from_numpy(rows).cuda()], "f16"), lr.cpu().numpy()[rows],
                  z[rows], t[rows], B, "f16", where="f16 lmhead128k")
    # the scalar: the oracle's per-row losses of every row, in blocks
    l_all = np.concatenate([ce_rows(widen_rows(z[i:i + 512], "f16"), t[i:i + 512], B)[0]
                            for i in range(0, B, 512)])
    compare_scalar(float(loss.item()), reduce_loss(l_all), "f16", "f16 lmhead128k")


# ------------------------------------------------------------ row strides

# (B, C, dtype, padding of the logits rows, padding of the gradient rows):
# most strides leave rows at every offset modulo 16 bytes; the last case's
# strides differ by 12 bytes, which the call refuses.
STRIDE_CASES = [
    (8, 10, "f32", 6, 2),
    (300, 100, "bf16", 8, 24),
    (64, 257, "f16", 5, 13),
    (129, 1000, "f32", 24, 0),
    (33, 4099, "bf16", 3, 11),
    (9, 50257, "f32", 2, 6),
    (6, 128256, "bf16", 256, 128),
    (6, 128256, "bf16", 3, 11),
    (3, 200_000, "f16", 1, 9),
    (8, 10, "f32", 6, 3),
]
STRIDE_IDS = [f"{b}x{c}-{d}-pad{p}-{q}" for b, c, d, p, q in STRIDE_CASES]


def _wide(z, dtype, pad, fill=None):
    """The rows of z inside a [B, C + pad] buffer (padding = fill, or a
    sentinel pattern), returned as (buffer, [B, C] view)."""
    import torch
    B, C = z.shape
    zd, _ = to_device(z, np.zeros(B, np.int32), dtype)
    buf = torch.empty((B, C + pad), dtype=zd.dtype, device=zd.device)
    _bits(buf).fill_(0x7BAD if zd.element_size() == 2 else 0x7BADBEEF)
    view = buf[:, :C]
    view.copy_(zd)
    return buf, view


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("B,C,dtype,padz,padg", STRIDE_CASES, ids=STRIDE_IDS)
def test_row_stride_matches_oracle(B, C, dtype, padz, padg, path):
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B * 11 + C)
    _, td = to_device(z, t, dtype)
    zbuf, zv = _wide(z, dtype, padz)
    gbuf, gv = _wide(np.zeros_like(z), dtype, padg)
    if path == 5 and not wave_takes(C, _es(dtype), (C, C + padz, C + padg),
                                    (zv.data_ptr(), gv.data_ptr())):
        pytest.skip("rows that path 5 does not take at these strides")
    zsnap = zbuf.clone()
    gsnap = gbuf.clone()
    lr = torch.empty(B, dtype=torch.float32, device=zv.device)
    es = _es(dtype)
    if ((padg - padz) * es) % 16:
        with pytest.raises(ce.CEError):
            ce.fwd_grad_ex_into(zv, td, gv, lr)
        return
    ce.fwd_grad_ex_into(zv, td, gv, lr)
    torch.cuda.synchronize()
    assert torch.equal(_bits(zbuf), _bits(zsnap))                 # logits untouched
    assert torch.equal(_bits(gbuf[:, C:]), _bits(gsnap[:, C:]))   # grad padding untouched
    worst, l_ora = compare_block(grad_to_host(gv, dtype), lr.cpu().numpy(), z, t, B, dtype,
                                 where=f"stride {B}x{C} p{path}")
    print(f"[stride] {B}x{C} {dtype} ld {C + padz}/{C + padg} p{path}: {worst}", flush=True)
    # loss only (refused on forced path 4), and in place over the strided
    # logits
    lr2 = torch.empty_like(lr)
    if path != 4:
        ce.fwd_grad_ex_into(zv, td, None, lr2)
        torch.cuda.synchronize()
        tol = 1e-5 * (np.abs(widen_rows(z, dtype).max(axis=1)) + math.log(C) + 1.0) / B
        assert (np.abs(lr2.cpu().numpy() - l_ora) <= tol).all()
    # rows of several parts in place run as parts with the in-place
    # workspace (the binding passes one)
    ce.fwd_grad_ex_into(zv, td, zv, lr2)
    torch.cuda.synchronize()
    compare_block(grad_to_host(zv, dtype), lr2.cpu().numpy(), z, t, B, dtype,
                  where=f"stride in place {B}x{C} p{path}")
    assert torch.equal(_bits(zbuf[:, C:]), _bits(zsnap[:, C:]))


def test_row_stride_aligned_equals_contiguous():
    """Strides that keep every row's alignment: the bits of the contiguous
    call on the same path."""
    import torch
    ce = _ce()
    for B, C, dtype, pad in ((40, 1000, "f32", 24), (9, 128256, "bf16", 64), (64, 304, "f16", 8)):
        z, t = synth.make_inputs(B, C, dtype, 3.0, seed=C)
        zd, td = to_device(z, t, dtype)
        g0, l0 = ce.fwd_grad(zd, td)
        wide = torch.zeros((B, C + pad), dtype=zd.dtype, device=zd.device)
        # rows of C elements at a stride of C + pad: the first row of the
        # view starts at the buffer, each later row pad elements further
        view = wide[:, :C]
        view.copy_(zd)
        if (C * _es(dtype)) % 16 == 0 and (pad * _es(dtype)) % 16 == 0:
            g1, l1 = ce.fwd_grad_ex(view, td)
            torch.cuda.synchronize()
            assert torch.equal(_bits(g1), _bits(g0)) and torch.equal(_bits(l1), _bits(l0))


# ----------------------------------------------------------- ignore_index

IGN_CASES = [
    (8, 10, "f32", -100),
    (300, 7, "bf16", 3),
    (129, 100, "f16", -1),
    (1024, 1000, "f32", -100),
    (33, 4099, "bf16", -100),
    (40, 50257, "f32", -100),
    (16, 128256, "bf16", -100),
    (3, 200_000, "bf16", -100),
    # the kept-row count over several workgroups (one atomic each), and
    # over more rounds than workgroups
    (40_000, 10, "f32", -100),
    (4_200_001, 3, "bf16", 0),
]
IGN_IDS = [f"{b}x{c}-{d}-ign{i}" for b, c, d, i in IGN_CASES]


def check_ignore(g_host, l_host, z, t, ii, dtype, where):
    ign = t == ii
    N = int((~ign).sum())
    assert (l_host[ign] == 0).all(), where
    gi = g_host[ign]
    assert (gi.view(np.uint32 if dtype == "f32" else np.uint16) == 0).all(), where
    if N:
        res, l_ora = compare_block(g_host[~ign], l_host[~ign], z[~ign], t[~ign], N, dtype,
                                   where=where)
        return res
    return {}


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
@pytest.mark.parametrize("B,C,dtype,ii", IGN_CASES, ids=IGN_IDS)
def test_ignore_index_matches_oracle(B, C, dtype, ii, path):
    import torch
    ce = _ce()
    if not _legal(path, C, dtype):
        pytest.skip("the forced path does not take this row length")
    if B > 1_000_000 and path != 0:
        pytest.skip("millions of rows: the automatic path only (the count is path-independent)")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + 13 * C)
    rng = np.random.Generator(np.random.PCG64(B + C))
    t[rng.random(B) < 0.3] = ii
    t[0] = ii
    zd, td = to_device(z, t, dtype)
    g, lr = ce.fwd_grad_ex(zd, td, ignore_index=ii)
    loss = ce.reduce_loss(lr)
    torch.cuda.synchronize()
    gh, lh = grad_to_host(g, dtype), lr.cpu().numpy()
    worst = check_ignore(gh, lh, z, t, ii, dtype, f"ignore {B}x{C} p{path}")
    l_ora, _ = ce_rows_ignore(widen_rows(z, dtype), t, ii)
    compare_scalar(float(loss.item()), reduce_loss(l_ora), dtype, f"ignore {B}x{C}")
    print(f"[ignore] {B}x{C} {dtype} p{path}: {worst}", flush=True)
    # the losses alone (no row parts there)
    if path != 4:
        _, lr2 = ce.fwd_grad_ex(zd, td, ignore_index=ii, with_grad=False)
        torch.cuda.synchronize()
        l2 = lr2.cpu().numpy()
        ign = t == ii
        assert (l2[ign] == 0).all()
        tol = 1e-5 * (np.abs(widen_rows(z, dtype).max(axis=1)) + math.log(C) + 1.0) / (~ign).sum()
        assert (np.abs(l2 - l_ora) <= tol).all()


def test_ignore_index_edges():
    """Every row ignored: all outputs 0 (no NaN); no row ignored: the bits of
    ce_fwd_grad; with a device grad scale and in place."""
    import torch
    ce = _ce()
    B, C = 64, 3000
    z, t = synth.make_inputs(B, C, "bf16", 4.0, seed=5)
    zd, td = to_device(z, t, "bf16")
    g, lr = ce.fwd_grad_ex(zd, torch.full_like(td, 7), ignore_index=7)
    torch.cuda.synchronize()
    assert (lr == 0).all() and (_bits(g) == 0).all()
    g0, l0 = ce.fwd_grad(zd, td)
    g1, l1 = ce.fwd_grad_ex(zd, td, ignore_index=-100)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g0), _bits(g1)) and torch.equal(_bits(l0), _bits(l1))
    t2 = t.copy()
    t2[::3] = -100
    td2 = torch.from_numpy(t2).cuda()
    sc = torch.tensor([2.0], device=zd.device)
    gs, ls = ce.fwd_grad_ex(zd, td2, ignore_index=-100, grad_scale=sc)
    ga, la = ce.fwd_grad_ex(zd, td2, ignore_index=-100)
    buf = zd.clone()
    lb = torch.empty_like(la)
    ce.fwd_grad_ex_into(buf, td2, buf, lb, ignore_index=-100)
    torch.cuda.synchronize()
    assert torch.equal(_bits(ls), _bits(la))
    assert torch.equal(_bits(gs), _bits((ga.float() * 2).to(torch.bfloat16)))
    check_ignore(grad_to_host(buf, "bf16"), lb.cpu().numpy(), z, t2, -100, "bf16", "in place")


def test_ignore_index_autograd():
    import torch
    ce = _ce()
    B, C = 48, 50257
    z, t = synth.make_inputs(B, C, "f32", 3.0, seed=6)
    t[::4] = -100
    zd, td = to_device(z, t, "f32")
    x = zd.clone().requires_grad_(True)
    loss = ce.cross_entropy_loss(x, td, ignore_index=-100)
    loss.backward()
    torch.cuda.synchronize()
    l_ora, g_ora = ce_rows_ignore(z.astype(np.float64), t, -100)
    assert math.isclose(loss.item(), reduce_loss(l_ora), rel_tol=1e-5)
    assert np.abs(x.grad.cpu().numpy() - g_ora).max() <= 1e-6


def test_ignore_index_full_lmhead128k_sampled():
    """The 8192 x 128256 bf16 workload with a quarter of the rows ignored:
    48 sampled rows and the scalar loss against the oracle."""
    import torch
    ce = _ce()
    w = synth.workload("lmhead128k")
    z, t = synth.make_workload("lmhead128k")
    t[np.random.Generator(np.random.PCG64(10)).random(w.B) < 0.25] = -100
    zd, td = to_device(z, t, "bf16")
    g, lr = ce.fwd_grad_ex(zd, td, ignore_index=-100)
    loss = ce.reduce_loss(lr)
    torch.cuda.synchronize()
    rows = np.random.Generator(np.random.PCG64(11)).choice(w.B, 48, replace=False)
    ign = t == -100
    N = int((~ign).sum())
    sel = rows[~ign[rows]]
    compare_block(grad_to_host(g[torch.from_numpy(sel).cuda()], "bf16"), lr.cpu().numpy()[sel],
                  z[sel], t[sel], N, "bf16", where="ignore lmhead128k")
    lh = lr.cpu().numpy()
    assert (lh[ign] == 0).all()
    l_kept = np.concatenate([ce_rows(widen_rows(z[i:i + 512][~ign[i:i + 512]], "bf16"),
                                     t[i:i + 512][~ign[i:i + 512]], N)[0]
                             for i in range(0, w.B, 512)])
    compare_scalar(float(loss.item()), reduce_loss(l_kept), "bf16", "ignore lmhead128k")


def test_binding_allocates_outputs_congruent_to_inputs():
    """Views whose base is not on a 16-byte boundary: the binding's
    allocating calls give outputs at the same offset modulo 16, so the
    library accepts them, and the results match the aligned copies'."""
    import torch
    ce = _ce()
    for dtype, off in (("f32", 1), ("bf16", 3), ("f16", 5)):
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
        z, t = synth.make_inputs(12, 300, dtype, 3.0, seed=off)
        za, td = to_device(z, t, dtype)
        flat = torch.empty(off + za.numel() + 16, dtype=tdt, device=za.device)
        zm = flat[off:off + za.numel()].view(za.shape)
        zm.copy_(za)
        g, lr = ce.fwd_grad(zm, td)
        assert g.data_ptr() % 16 == zm.data_ptr() % 16
        y = ce.softmax_fwd(zm)
        dx = ce.softmax_bwd(y, torch.ones_like(za))       # dy aligned, y not
        torch.cuda.synchronize()
        compare_block(grad_to_host(g, dtype), lr.cpu().numpy(), z, t, 12, dtype, where=f"offset {dtype}")
        assert float(dx.float().abs().max().item()) <= 2.0 ** -6   # dy constant: dx = 0 up to rounding
