"""Cross-entropy over a vocabulary split into column shards, on the GPU,
against the fp64 oracle: every shard's record (ce_shard_stats) against the
oracle's shard record, and the gradients and losses that ce_shard_grad
writes from the gathered records against the cross-entropy oracle of the
whole, unsplit row (rumus project page, milestone M24 column-parallel
layers; the cross-entropy of rumus 0.1.1 cross_entropy.wgsl pass 1).

Bars: the records are compared through quantities that do not depend on
the reference point a kernel picks: c ln2 against the shard max m_k
(|c ln2 - m_k| <= 2^-22 |m_k| + 2^-126), the log of the shard's sum
without the target, ln sx + c ln2 against ln sx_k + m_k (within 2^-20
(|m_k| + ln C_k + 1)), zt and own exactly.  The gradient and the per-row
loss are held to the fused path's bars (fp32 gradient 1e-6 absolute, bf16
1 ulp; per-row loss 1e-5 (|max z| + ln C + 1) / B; scalar loss 1e-5 or
2e-3 relative).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import reduce_loss, shard_partials

from _parity import wave_takes, compare_block, compare_scalar, grad_to_host, to_device, widen_rows

pytestmark = pytest.mark.gpu

# (B, C, dtype, sigma, spike, shard edges as fractions of C)
CASES = [
    (8, 10, "f32", 1.0, None, [0, 3, 10]),
    (300, 7, "f32", 20.0, None, [0, 1, 2, 7]),
    (129, 1000, "bf16", 4.0, None, [0, 250, 500, 750, 1000]),
    (64, 4099, "f32", 3.0, None, [0, 1, 4098, 4099]),
    (40, 50257, "f32", 3.0, 1.0e4, [0, 25000, 50257]),
    (16, 128256, "bf16", 4.0, None, [i * 16032 for i in range(9)]),
    (9, 99999, "bf16", 4.0, None, [0, 33333, 33334, 99999]),
    (5, 200_000, "bf16", 4.0, None, [0, 200_000]),
]
IDS = [f"{b}x{c}-{d}-{len(e) - 1}shards" for b, c, d, _, _, e in CASES]


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _reset_path():
    ce = _ce()
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _shards(zd, edges):
    return [zd[:, a:b].contiguous() for a, b in zip(edges[:-1], edges[1:])]


def check_records(rec, z_shard, t, col0, dtype, where):
    z64 = widen_rows(z_shard, dtype)
    m, sx, zt, own = shard_partials(z64, t, col0)
    c, s, zt_g, own_g = (rec[:, i].astype(np.float64) for i in range(4))
    ln2 = math.log(2.0)
    assert np.array_equal(own_g, own.astype(np.float64)), where
    assert np.array_equal(zt_g, zt), where
    assert (np.abs(c * ln2 - m) <= 2.0 ** -22 * np.abs(m) + 2.0 ** -126).all(), where
    Ck = z64.shape[1]
    tol = 2.0 ** -20 * (np.abs(m) + math.log(Ck) + 1.0)
    pos = sx > 0
    assert np.array_equal(s > 0, pos), where
    with np.errstate(divide="ignore"):
        err = np.abs((np.log(s[pos]) + c[pos] * ln2) - (np.log(sx[pos]) + m[pos]))
    assert (err <= tol[pos]).all(), (where, float(err.max()))


def run_sharded(zd, td, edges, dtype, loss_from=0, grad_scale=None, in_place=False):
    import torch
    ce = _ce()
    C = edges[-1]
    shards = _shards(zd, edges)
    recs = torch.stack([ce.shard_stats(s, td, a) for s, a in zip(shards, edges[:-1])])
    grads, loss_rows = [], None
    for k, (s, a) in enumerate(zip(shards, edges[:-1])):
        lr = torch.empty(s.shape[0], dtype=torch.float32, device=s.device) if k == loss_from else None
        g = s if in_place else torch.empty_like(s)
        ce.shard_grad_into(s, td, a, C, recs, g, lr, grad_scale)
        grads.append(g)
        if lr is not None:
            loss_rows = lr
    torch.cuda.synchronize()
    return recs, torch.cat(grads, dim=1), loss_rows


@pytest.mark.parametrize("path", [0, 1, 2, 3, 5], ids=["auto", "short", "resident", "long", "wave"])
@pytest.mark.parametrize("B,C,dtype,sigma,spike,edges", CASES, ids=IDS)
def test_sharded_matches_whole_row_oracle(B, C, dtype, sigma, spike, edges, path):
    import torch
    ce = _ce()
    widths = np.diff(edges)
    if path == 1 and widths.max() > 256:
        pytest.skip("a shard longer than the short path takes")
    es = 4 if dtype == "f32" else 2
    if path == 2 and (int(widths.max()) * es + 15) // 16 + 1 > 16384:
        pytest.skip("a shard longer than the resident path takes")
    if path == 5 and not all(wave_takes(int(w), es) for w in widths):
        pytest.skip("a shard that path 5 does not take")
    ce.force_path(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, spike=spike, seed=B + C + len(edges))
    if spike is not None:
        t[: B // 4] = synth.spike_columns(B, C, seed=B + C + len(edges))[: B // 4].astype(np.int32)
    t[-1] = edges[1] - 1 if len(edges) > 2 else C - 1       # a shard's last column
    if B > 2:
        t[-2] = edges[-2]                                   # the last shard's first column
    zd, td = to_device(z, t, dtype)
    recs, grad, loss_rows = run_sharded(zd, td, edges, dtype, loss_from=len(edges) - 2)
    rh = recs.cpu().numpy()
    for k, (a, b) in enumerate(zip(edges[:-1], edges[1:])):
        check_records(rh[k], z[:, a:b], t, a, dtype, f"{B}x{C} shard {k} p{path}")
    worst, l_ora = compare_block(grad_to_host(grad, dtype), loss_rows.cpu().numpy(), z, t, B, dtype,
                                 where=f"sharded {B}x{C} p{path}")
    loss = ce.reduce_loss(loss_rows)
    compare_scalar(float(loss.item()), reduce_loss(l_ora), dtype, f"sharded {B}x{C}")
    print(f"[shard] {B}x{C} {dtype} {len(edges) - 1} shards p{path}: {worst}", flush=True)


def test_every_shard_writes_the_same_losses():
    import torch
    B, C, dtype = 33, 12345, "bf16"
    edges = [0, 4000, 8000, 12345]
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=3)
    zd, td = to_device(z, t, dtype)
    out = [run_sharded(zd, td, edges, dtype, loss_from=k)[2] for k in range(3)]
    for lr in out[1:]:
        assert torch.equal(lr.view(torch.int32), out[0].view(torch.int32))


def test_invalid_targets_and_missing_owner():
    """Targets outside [0, C_total) give NaN rows; so do records that name no
    owner (the owning shard's records left out of the gather)."""
    import torch
    ce = _ce()
    B, C, dtype = 12, 3000, "f32"
    edges = [0, 1000, 2000, 3000]
    z, t = synth.make_inputs(B, C, dtype, 2.0, seed=9)
    t[0], t[1], t[2] = -1, C, 2**31 - 1
    t[3] = 1500
    zd, td = to_device(z, t, dtype)
    recs, grad, loss_rows = run_sharded(zd, td, edges, dtype)
    lr = loss_rows.cpu().numpy()
    g = grad.cpu().numpy()
    assert np.isnan(lr[:3]).all() and np.isnan(g[:3]).all()
    compare_block(g[3:], lr[3:], z[3:], t[3:], B, dtype, where="valid rows")
    # shard 1's records dropped: row 3 (target 1500) has no owner
    shards = _shards(zd, edges)
    part = recs[[0, 2]].contiguous()
    g0 = torch.empty_like(shards[0])
    lr0 = torch.empty(B, dtype=torch.float32, device=zd.device)
    ce.shard_grad_into(shards[0], td, 0, C, part, g0, lr0)
    torch.cuda.synchronize()
    assert math.isnan(float(lr0[3].item())) and torch.isnan(g0[3]).all()


@pytest.mark.parametrize("s", [0.5, -3.0])
def test_grad_scale_and_in_place(s):
    """A device grad_scale multiplies the gradient (not the loss), and the
    gradient written over the shard itself has the bits of the separate
    output."""
    import torch
    B, C, dtype = 24, 50000, "bf16"
    edges = [0, 20000, 50000]
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=4)
    zd, td = to_device(z, t, dtype)
    _, g1, l1 = run_sharded(zd, td, edges, dtype)
    sc = torch.tensor([s], dtype=torch.float32, device=zd.device)
    _, g2, l2 = run_sharded(zd, td, edges, dtype, grad_scale=sc)
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    want = (g1.float() * s).to(torch.bfloat16)
    d = (g2.view(torch.int16).int() - want.view(torch.int16).int()).abs()
    assert int(d.max().item()) <= 1
    _, g3, l3 = run_sharded(zd, td, edges, dtype, in_place=True)
    assert torch.equal(g3.view(torch.int16), g1.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l1.view(torch.int32))


def test_lmhead128k_eight_shards_sampled():
    """The 8192 x 128256 bf16 workload in eight shards of 16032 columns (the
    shape the benchmark times): every row's records and 48 sampled rows of
    gradient and loss against the oracle."""
    import torch
    w = synth.workload("lmhead128k")
    z, t = synth.make_workload("lmhead128k")
    zd, td = to_device(z, t, "bf16")
    edges = [i * 16032 for i in range(9)]
    recs, grad, loss_rows = run_sharded(zd, td, edges, "bf16")
    rows = np.random.Generator(np.random.PCG64(8)).choice(w.B, 48, replace=False)
    rows[:2] = [0, w.B - 1]
    rh = recs.cpu().numpy()
    for k in (0, 7):
        a, b = edges[k], edges[k + 1]
        check_records(rh[k][rows], z[rows, a:b], t[rows], a, "bf16", f"lmhead128k shard {k}")
    gsel = grad[torch.from_numpy(rows).cuda()]
    compare_block(grad_to_host(gsel, "bf16"), loss_rows.cpu().numpy()[rows], z[rows], t[rows],
                  w.B, "bf16", where="lmhead128k 8 shards")
