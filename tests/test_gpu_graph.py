"""The path under HIP graph capture (torch.cuda.CUDAGraph): a step of
ce_fwd_grad + ce_reduce_loss (and the other entry points) captured once
and replayed several times, with the program's own eager work and
synchronisations between replays; every replay must equal the eager
result bit for bit.  No entry point records a memset: workspaces and
counters are cleared by kernels."""

from __future__ import annotations

import numpy as np
import pytest

import synth

from _parity import to_device

pytestmark = pytest.mark.gpu


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


@pytest.mark.parametrize("B,C,dtype", [(8, 10, "f32"), (1024, 1000, "f32"), (65536, 10, "f32"),
                                       (64, 50257, "f32"), (32, 128256, "bf16"), (40, 3000, "f16")])
def test_step_replays_equal_eager(B, C, dtype):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, 3.0, seed=B + C)
    zd, td = to_device(z, t, dtype)
    grad = ce._empty_congruent(zd)
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    loss = torch.empty((), dtype=torch.float32, device=zd.device)
    need = ce.reduce_workspace_bytes(B)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=zd.device)
    # eager reference
    ce.fwd_grad_into(zd, td, grad, lr)
    ce.reduce_loss_into(lr, loss, ws)
    torch.cuda.synchronize()
    g0, l0, s0 = grad.clone(), lr.clone(), loss.clone()
    # capture (on a side stream, as torch requires), after a warm-up there
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ce.fwd_grad_into(zd, td, grad, lr)
        ce.reduce_loss_into(lr, loss, ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ce.fwd_grad_into(zd, td, grad, lr)
        ce.reduce_loss_into(lr, loss, ws)
    for rep in range(4):
        grad.fill_(0)
        lr.fill_(float("nan"))
        loss.fill_(-1.0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(grad), _bits(g0)), rep
        assert torch.equal(_bits(lr), _bits(l0)), rep
        assert torch.equal(_bits(loss), _bits(s0)), rep
        # eager work between replays
        ce.fwd_loss_into(zd, td, lr)
        torch.cuda.synchronize()


def test_ignore_index_and_softmax_replay():
    """ce_fwd_grad_ex with ignore_index (its count cleared by a kernel) and
    the softmax forward and backward, captured together."""
    import torch
    ce = _ce()
    B, C = 256, 5000
    z, t = synth.make_inputs(B, C, "bf16", 3.0, seed=3)
    t[::4] = -100
    zd, td = to_device(z, t, "bf16")
    g = ce._empty_congruent(zd)
    lr = torch.empty(B, dtype=torch.float32, device=zd.device)
    ws = torch.empty(4, dtype=torch.uint8, device=zd.device)
    y = ce._empty_congruent(zd)
    dx = ce._empty_congruent(zd)

    def run():
        ce.fwd_grad_ex_into(zd, td, g, lr, ignore_index=-100, workspace=ws)
        ce.softmax_fwd_into(zd, y)
        ce.softmax_bwd_into(y, zd, dx)

    run()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (g, lr, y, dx)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(4):
        for x in (g, lr, y, dx):
            x.fill_(0)
        ws.fill_(7)            # a stale count must not survive into a replay
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((g, lr, y, dx), ref):
            assert torch.equal(_bits(a), _bits(b)), rep
