"""The gradient in place of rows that path 4 cuts into two, four or eight
parts, on the in-place variant of the part kernel (ce_fwd_grad_ex with the
in-place workspace): every row against the oracle; bitwise the same
whether each part writes its own gradient or defers it to a partner (no
polls makes nearly every part but one defer, and the device counter sees
the deferrals); the workspace's row words zero again after every call;
with ignore_index and a gradient scale; captured in a HIP graph; on two
streams at once; the 8192 x 128256 bf16 workload at full size and large
batches of four- and eight-part rows.  Without the workspace such rows still run off path 4
(and forcing path 4 is refused)."""

from __future__ import annotations

import numpy as np
import pytest

import synth
from _parity import compare_block, grad_to_host, to_device
from test_gpu_ex import check_ignore

pytestmark = pytest.mark.gpu


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


@pytest.fixture(autouse=True)
def _reset_hooks():
    ce = _ce()
    prev_path, prev_polls = ce.force_path(0), ce.part_polls(64)
    ce.part_polls(prev_polls)
    yield
    ce.force_path(prev_path)
    ce.part_polls(prev_polls)
    ce.part_counter(None)


def _workspace(B, device="cuda:0"):
    import torch
    return torch.zeros(_ce().fwd_inplace_workspace_bytes(B), dtype=torch.uint8, device=device)


def _words_zero(ws) -> bool:
    return bool((ws[256:] == 0).all().item())


def _in_place(zd, td, ws, **kw):
    """ce_fwd_grad_ex in place on a copy of zd; returns (gradient, losses)."""
    import torch
    ce = _ce()
    buf = zd.clone()
    lr = torch.empty(zd.shape[0], dtype=torch.float32, device=zd.device)
    ce.fwd_grad_ex_into(buf, td, buf, lr, workspace=ws, **kw)
    return buf, lr


# (B, C, dtype): two parts of register slots (bf16 and fp16 C up to 131072,
# fp32 up to 65536) and of register and LDS slots beyond, four parts (bf16
# and fp16 C up to 393216, fp32 up to 196608, with 2 LDS slots past 262144
# and 131072 and 4 past 327680 and 163840), eight parts (bf16 up to 524288,
# fp32 up to 262144); the smallest and largest rows of each, one row,
# ragged batches
SHAPES = [
    (1, 128256, "bf16"), (37, 128256, "bf16"), (6, 150000, "bf16"), (300, 81930, "bf16"),
    (5, 196608, "bf16"), (17, 100000, "f16"), (9, 50257, "f32"), (33, 70000, "f32"),
    (4, 98304, "f32"), (64, 40964, "f32"),
    (3, 196616, "bf16"), (20, 262144, "bf16"), (7, 300000, "bf16"), (18, 256000, "f16"),
    (2, 393216, "bf16"), (5, 393224, "bf16"), (16, 500000, "bf16"), (1, 524288, "bf16"),
    (13, 128256, "f32"), (3, 98308, "f32"), (6, 200003, "f32"), (17, 262144, "f32"),
    (9, 151936, "f32"), (5, 163844, "f32"), (4, 196608, "f32"), (3, 196612, "f32"),
]


def _parts(C, dtype):
    """Parts per row of an aligned body (as path 4 cuts it in place)."""
    nb = C // (4 if dtype == "f32" else 8)
    if nb <= 10 * 1024:
        return 1
    if nb <= 24 * 1024:
        return 2
    return 4 if nb <= 48 * 1024 else 8


@pytest.mark.parametrize("B,C,dtype", SHAPES, ids=[f"{b}x{c}-{d}" for b, c, d in SHAPES])
def test_in_place_parts_match_oracle_and_defer_bitwise(B, C, dtype):
    import torch
    ce = _ce()
    assert ce.select_path(C, {"f32": 0, "bf16": 1, "f16": 2}[dtype]) == 4
    assert _parts(C, dtype) > 1
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=B * 11 + C)
    # targets on the row's first and last element and around the middle and
    # a quarter (where parts meet)
    for i, col in enumerate((0, C - 1, C // 2 - 1, C // 2, C // 2 + 1, C // 4, C // 4 - 1)):
        if i < B:
            t[i] = col
    zd, td = to_device(z, t, dtype)
    ws = _workspace(B)
    g, lr = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    assert _words_zero(ws)
    worst, _ = compare_block(grad_to_host(g, dtype), lr.cpu().numpy(), z, t, B, dtype,
                             where=f"in-place parts {B}x{C} {dtype}")
    print(f"[in-place parts] {B}x{C} {dtype}: {worst}", flush=True)
    # (nearly) every part but one defers: a partner writes its gradient, with
    # the same bits
    counter = torch.zeros(1, dtype=torch.int32, device=zd.device)
    ce.part_counter(counter)
    ce.part_polls(0)
    g2, lr2 = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    ce.part_counter(None)
    assert torch.equal(_bits(g2), _bits(g)) and torch.equal(_bits(lr2), _bits(lr))
    assert _words_zero(ws)
    print(f"[in-place parts] {B}x{C} {dtype}: {int(counter.item())} of {B} rows deferred",
          flush=True)
    # (with no polls a part defers unless its partners published before it
    # looked: in batches of a few rows that can happen to every row)
    if B >= 16:
        assert int(counter.item()) >= 1


def test_in_place_parts_ignore_index_and_scale():
    """A third of the rows ignored and a device gradient scale of 0.5, in
    place on rows of two and of eight parts: against the oracle, and
    bitwise with deferrals."""
    ce = _ce()
    polls = ce.part_polls(0)
    for C in (128256, 500000):
        ce.part_polls(polls)
        _ignore_and_scale(C)


def _ignore_and_scale(C):
    import torch
    ce = _ce()
    B, dtype = 48, "bf16"
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=3)
    t[::3] = -100
    zd, td = to_device(z, t, dtype)
    ws = _workspace(B)
    g, lr = _in_place(zd, td, ws, ignore_index=-100)
    torch.cuda.synchronize()
    check_ignore(grad_to_host(g, dtype), lr.cpu().numpy(), z, t, -100, dtype, "in-place parts")
    half = torch.tensor([0.5], dtype=torch.float32, device=zd.device)
    gs, ls = _in_place(zd, td, ws, ignore_index=-100, grad_scale=half)
    torch.cuda.synchronize()
    assert torch.equal(_bits(ls), _bits(lr))
    assert torch.equal(_bits(gs), _bits((g.float() * 0.5).to(torch.bfloat16)))
    ce.part_polls(0)
    g2, _ = _in_place(zd, td, ws, ignore_index=-100)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g2), _bits(g)) and _words_zero(ws)


def test_in_place_parts_workspace_reuse_and_smaller_batch():
    """One workspace (zero-filled once) over calls of different B and
    parts per row: each call's result is its own (the same bits as on a
    fresh workspace) and the words are zero after each."""
    import torch
    ws = _workspace(512)
    for B, C, seed in ((512, 50257, 1), (7, 50257, 2), (512, 150000, 3), (100, 50257, 4),
                       (64, 200003, 5), (300, 128256, 6)):
        z, t = synth.make_inputs(B, C, "f32", 3.0, seed=seed)
        zd, td = to_device(z, t, "f32")
        g, lr = _in_place(zd, td, ws)
        g0, l0 = _in_place(zd, td, _workspace(B))
        torch.cuda.synchronize()
        assert torch.equal(_bits(g), _bits(g0)) and torch.equal(_bits(lr), _bits(l0))
        assert _words_zero(ws)


def test_in_place_parts_graph_replays():
    """Captured once; before each replay new logits are copied into the
    captured buffer (the call overwrites them with the gradient): each
    replay equals the eager call on those logits."""
    import torch
    ce = _ce()
    B, C, dtype = 40, 128256, "bf16"
    inputs = [to_device(*synth.make_inputs(B, C, dtype, 4.0, seed=30 + k), dtype) for k in range(3)]
    buf = inputs[0][0].clone()
    td = inputs[0][1].clone()
    lr = torch.empty(B, dtype=torch.float32, device=buf.device)
    ws = _workspace(B)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ce.fwd_grad_ex_into(buf, td, buf, lr, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ce.fwd_grad_ex_into(buf, td, buf, lr, workspace=ws)
    for rep in range(6):
        zk, tk = inputs[rep % 3]
        buf.copy_(zk)
        td.copy_(tk)
        lr.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        g0, l0 = _in_place(zk, tk, _workspace(B))
        torch.cuda.synchronize()
        assert torch.equal(_bits(buf), _bits(g0)) and torch.equal(_bits(lr), _bits(l0)), rep
        assert _words_zero(ws)


def test_plain_in_place_keeps_off_parts():
    """ce_fwd_grad in place (no workspace): two-part rows run on path 2 and
    forcing path 4 is refused; ce_fwd_grad_ex with a workspace too small
    does the same."""
    import torch
    ce = _ce()
    B, C = 8, 128256
    z, t = synth.make_inputs(B, C, "bf16", 4.0, seed=8)
    zd, td = to_device(z, t, "bf16")
    buf = zd.clone()
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    ce.force_path(4)
    with pytest.raises(ce.CEError):
        ce.fwd_grad_into(buf, td, buf, lr)
    small = torch.zeros(ce.fwd_inplace_workspace_bytes(B) - 16, dtype=torch.uint8, device=zd.device)
    with pytest.raises(ce.CEError):
        ce.fwd_grad_ex_into(buf, td, buf, lr, workspace=small)
    ce.force_path(0)
    ce.fwd_grad_into(buf, td, buf, lr)
    ce.force_path(2)
    g0, l0 = ce.fwd_grad(zd, td)
    torch.cuda.synchronize()
    assert torch.equal(_bits(buf), _bits(g0)) and torch.equal(_bits(lr), _bits(l0))


def test_in_place_parts_lmhead128k_full():
    """8192 x 128256 bf16 in place: 64 sampled rows against the oracle, the
    whole gradient bitwise equal with every first part deferring, and the
    words zero after both calls."""
    import torch
    ce = _ce()
    w = synth.workload("lmhead128k")
    z, t = synth.make_workload("lmhead128k")
    zd, td = to_device(z, t, "bf16")
    ws = _workspace(w.B)
    g, lr = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    assert _words_zero(ws)
    rows = np.sort(np.random.Generator(np.random.PCG64(12)).choice(w.B, 64, replace=False))
    gh = grad_to_host(g[torch.from_numpy(rows).cuda()], "bf16")
    compare_block(gh, lr.cpu().numpy()[rows], z[rows], t[rows], w.B, "bf16", where="lmhead128k in place")
    ce.part_polls(0)
    g2, lr2 = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g2), _bits(g)) and torch.equal(_bits(lr2), _bits(lr))
    assert _words_zero(ws)


@pytest.mark.parametrize("B,C,dtype", [(1024, 256000, "bf16"), (512, 500000, "bf16"),
                                       (512, 262144, "f32"), (1024, 151936, "f32")],
                         ids=["1024x256000-bf16", "512x500000-bf16", "512x262144-f32",
                              "1024x151936-f32"])
def test_in_place_parts_large_batches(B, C, dtype):
    """Large batches of four- and eight-part rows in place: 32 sampled rows
    against the oracle, the whole gradient bitwise equal with (nearly)
    every part but one deferring, and the words zero after both calls."""
    import torch
    ce = _ce()
    assert _parts(C, dtype) in (4, 8)
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=B + C)
    zd, td = to_device(z, t, dtype)
    ws = _workspace(B)
    g, lr = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    assert _words_zero(ws)
    rows = np.sort(np.random.Generator(np.random.PCG64(C)).choice(B, 32, replace=False))
    gh = grad_to_host(g[torch.from_numpy(rows).cuda()], dtype)
    compare_block(gh, lr.cpu().numpy()[rows], z[rows], t[rows], B, dtype,
                  where=f"in place {B}x{C} {dtype}")
    ce.part_polls(0)
    g2, lr2 = _in_place(zd, td, ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(g2), _bits(g)) and torch.equal(_bits(lr2), _bits(lr))
    assert _words_zero(ws)


def test_in_place_parts_two_streams_at_once():
    """In place on two streams at once, each call with the binding's
    workspace for its own stream (rows of two, four and eight parts),
    three calls a stream queued together: every result has the bits of the
    call made alone."""
    import torch
    ce = _ce()
    for B, C, dtype in ((48, 128256, "bf16"), (24, 300000, "bf16"), (12, 200003, "f32")):
        z, t = synth.make_inputs(B, C, dtype, 4.0, seed=C)
        zd, td = to_device(z, t, dtype)
        g0, l0 = _in_place(zd, td, _workspace(B))
        torch.cuda.synchronize()
        outs = []
        streams = (torch.cuda.Stream(), torch.cuda.Stream())
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for s in streams:
            with torch.cuda.stream(s):
                buf = torch.empty_like(zd)
                lr = torch.empty(B, dtype=torch.float32, device=zd.device)
                for _ in range(3):
                    buf.copy_(zd)
                    ce.fwd_grad_ex_into(buf, td, buf, lr)
                outs.append((buf, lr))
        torch.cuda.synchronize()
        for buf, lr in outs:
            assert torch.equal(_bits(buf), _bits(g0)) and torch.equal(_bits(lr), _bits(l0)), (B, C)
