"""Row parts (path 4): the trade of max/sum-exp pairs between the
workgroups of a row.

A part that does not receive its partner's pair in time recomputes it with
the same code.  These tests force that (zero polls) and check that the
outputs are bitwise those of the exchange, that the device counter sees
every part of every row of two, four or eight parts recompute every other
part's pair, that mailbox-like bit patterns
left in grad_out on entry change nothing, that the forced fallback matches
the oracle, and that calls on two streams at once do not disturb each
other."""

from __future__ import annotations

import numpy as np
import pytest

import synth

from _parity import full_parity, to_device

pytestmark = pytest.mark.gpu

# (B, C, dtype, sigma): two parts per row (aligned, 2-byte aligned, 4-byte
# aligned fp32, every slot filled), four parts per row (registers only,
# fp32 register slots at their largest, 2-byte aligned with LDS slots, every
# slot filled; 2 LDS slots: fp32 just past the register slots, a
# 151936-wide fp32 row, both types at their largest, bf16 just past them),
# eight parts per row (fp32 just past four parts, a 256000-wide fp32 row,
# both types at their largest, 2-byte aligned bf16) and one one-part shape
# as a control.
SHAPES = [
    (64, 128256, "bf16", 4.0),
    (9, 99999, "bf16", 4.0),
    (33, 50257, "f32", 3.0),
    (5, 196607, "bf16", 4.0),
    (11, 256000, "bf16", 4.0),
    (6, 131071, "f32", 3.0),
    (5, 300001, "bf16", 4.0),
    (3, 393216, "bf16", 4.0),
    (7, 131077, "f32", 3.0),
    (13, 151936, "f32", 3.0),
    (4, 163840, "f32", 3.0),
    (6, 262152, "bf16", 4.0),
    (3, 327680, "bf16", 4.0),
    (5, 327688, "bf16", 4.0),
    (5, 163844, "f32", 3.0),
    (9, 256000, "f32", 3.0),
    (3, 262144, "f32", 3.0),
    (3, 524288, "bf16", 4.0),
    (4, 400001, "bf16", 4.0),
    (40, 40000, "f32", 3.0),
]
IDS = [f"{b}x{c}-{d}" for b, c, d, _ in SHAPES]

MAIL_TAG = 0x7FA57FA5
MAIL_EMPTY = 0x7FA17FA1


def _ce():
    import softmax_cross_entropy_ce_amd as ce
    return ce


@pytest.fixture(autouse=True)
def _reset_hooks():
    ce = _ce()
    prev_path = ce.force_path(4)
    prev_polls = ce.part_polls(64)
    yield
    ce.part_counter(None)
    ce.part_polls(prev_polls)
    ce.force_path(prev_path)


def _parts(C, dtype):
    """Parts per row: one up to an aligned body of 10240 vectors, two up to
    24576, four up to 49152 (16-bit) or 40960 (fp32), then eight."""
    nb = C // (4 if dtype == "f32" else 8)
    if nb <= 10 * 1024:
        return 1
    if nb <= 24 * 1024:
        return 2
    return 4 if nb <= (40 if dtype == "f32" else 48) * 1024 else 8


def _bits(x):
    import torch
    return x.view(torch.int16 if x.element_size() == 2 else torch.int32)


def _run(z_dev, t_dev):
    import torch
    grad, loss_rows = _ce().fwd_grad(z_dev, t_dev)
    torch.cuda.synchronize()
    return grad, loss_rows


@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES, ids=IDS)
def test_fallback_is_bitwise_and_counted(B, C, dtype, sigma):
    import torch
    ce = _ce()
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C)
    z_dev, t_dev = to_device(z, t, dtype)
    counter = torch.zeros(1, dtype=torch.int32, device=z_dev.device)
    ce.part_counter(counter)
    g1, l1 = _run(z_dev, t_dev)
    n_default = int(counter.item())
    ce.part_polls(0)
    counter.zero_()
    g2, l2 = _run(z_dev, t_dev)
    n_forced = int(counter.item())
    print(f"[parts] {B}x{C} {dtype}: recomputed pairs {n_default} (64 polls), "
          f"{n_forced} (0 polls)", flush=True)
    P = _parts(C, dtype)
    assert n_forced == B * P * (P - 1)      # every part recomputes every other part's pair
    assert torch.equal(_bits(g1), _bits(g2))
    assert torch.equal(_bits(l1), _bits(l2))


@pytest.mark.parametrize("pattern", [MAIL_TAG, MAIL_EMPTY, 0], ids=["tag", "empty", "zero"])
def test_stale_grad_content_is_ignored(pattern):
    """grad_out filled with the mailbox tag (or the empty tag) before the
    call: the clear step makes the parts ignore it."""
    import torch
    ce = _ce()
    B, C, dtype = 24, 99999, "bf16"
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=77)
    z_dev, t_dev = to_device(z, t, dtype)
    g_ref, l_ref = _run(z_dev, t_dev)
    words = torch.full((B * C // 2,), pattern - (1 << 32) if pattern >= 1 << 31 else pattern,
                       dtype=torch.int32, device=z_dev.device)
    grad = torch.empty_like(z_dev)
    grad.view(-1)[: 2 * words.numel()].view(torch.int32).copy_(words)
    loss_rows = torch.full((B,), float("nan"), dtype=torch.float32, device=z_dev.device)
    ce.fwd_grad_into(z_dev, t_dev, grad, loss_rows)
    torch.cuda.synchronize()
    assert torch.equal(_bits(grad), _bits(g_ref))
    assert torch.equal(_bits(loss_rows), _bits(l_ref))


@pytest.mark.parametrize("B,C,dtype,sigma", SHAPES[:-1], ids=IDS[:-1])
def test_forced_fallback_matches_oracle(B, C, dtype, sigma):
    _ce().part_polls(0)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=3 * B + C)
    full_parity(z, t, dtype, where=f"{B}x{C} {dtype} fallback")


def test_spike_rows_forced_fallback():
    """+1e4 spikes, some on the target, with every pair recomputed."""
    _ce().part_polls(0)
    B, C = 33, 50257
    z, t = synth.make_inputs(B, C, "f32", 3.0, spike=1e4, seed=12)
    t[:6] = synth.spike_columns(B, C, seed=12)[:6].astype(np.int32)
    full_parity(z, t, "f32", where="spike fallback")


def test_two_streams_at_once():
    """Two calls on two streams with their own outputs, queued together:
    each matches a call made alone."""
    import torch
    ce = _ce()
    B, C, dtype = 48, 128256, "bf16"
    z, t = synth.make_inputs(B, C, dtype, 4.0, seed=5)
    z_dev, t_dev = to_device(z, t, dtype)
    g_ref, l_ref = _run(z_dev, t_dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    torch.cuda.synchronize()
    for s in (s1, s2):
        g = torch.empty_like(z_dev)
        lr = torch.empty(B, dtype=torch.float32, device=z_dev.device)
        with torch.cuda.stream(s):
            for _ in range(3):
                ce.fwd_grad_into(z_dev, t_dev, g, lr)
        outs.append((g, lr))
    torch.cuda.synchronize()
    for g, lr in outs:
        assert torch.equal(_bits(g), _bits(g_ref))
        assert torch.equal(_bits(lr), _bits(l_ref))


@pytest.mark.parametrize("B,C,dtype,sigma", [(1040, 256000, "f32", 3.0), (1024, 524288, "bf16", 4.0)],
                         ids=["1040x256000-f32", "1024x524288-bf16"])
def test_eight_parts_full_grid_sampled(B, C, dtype, sigma):
    """Eight parts per row on a grid of about 1 GB of logits, so that parts
    of one row may not all be resident at once (the bounded polls, then the
    recompute): 34 sampled rows, the first and last among them, against the
    oracle element by element, the device counter's recomputed pairs
    reported, and the whole gradient and every per-row loss bitwise equal to
    a run in which every pair is recomputed (zero polls)."""
    import torch
    from _parity import compare_block, grad_to_host
    ce = _ce()
    ce.force_path(0)
    assert _parts(C, dtype) == 8
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=B + C)
    z_dev, t_dev = to_device(z, t, dtype)
    counter = torch.zeros(1, dtype=torch.int32, device=z_dev.device)
    ce.part_counter(counter)
    grad, loss_rows = _run(z_dev, t_dev)
    n = int(counter.item())
    rng = np.random.Generator(np.random.PCG64(B))
    rows = np.unique(np.concatenate([[0, B - 1], rng.choice(B, 32, replace=False)]))
    idx = torch.from_numpy(rows).to(grad.device)
    g = grad_to_host(grad.index_select(0, idx), dtype)
    worst, _ = compare_block(g, loss_rows.cpu().numpy()[rows], z[rows], t[rows], B, dtype,
                             where=f"eight parts {B}x{C} {dtype}")
    print(f"[parts] {B}x{C} {dtype}: {worst}, recomputed pairs {n}", flush=True)
    ce.part_counter(None)
    ce.part_polls(0)
    grad0, loss0 = _run(z_dev, t_dev)
    assert torch.equal(_bits(grad0), _bits(grad)) and torch.equal(_bits(loss0), _bits(loss_rows))


# 16-bit parts take each thread's c from its first slot and fold the other
# slots as they arrive; a thread whose sum reaches 2^32 (an element about 22
# above that c) forms it again from its true maximum, and pass 1
# takes maxima on the bit patterns (packed signed 16-bit max, packed min for
# threads whose elements are all negative).  Rows that reach every branch:
# spikes in later slots, spikes on the target, all-negative rows, rows
# whose first slots are far below the rest, rows with one element 80 and 95
# above the rest (past the bound: the first of them once gave an infinite
# loss), rows shifted far up, mixed signs around zero.
@pytest.mark.parametrize("B,C,dtype", [(16, 128256, "bf16"), (16, 50257, "bf16"),
                                       (12, 300001, "f16"), (16, 128256, "f16")],
                         ids=["128256-bf16", "50257-bf16", "300001-f16", "128256-f16"])
def test_16bit_part_max_edge_rows(B, C, dtype):
    import torch
    ce = _ce()
    rng = np.random.Generator(np.random.PCG64(C + B))
    z = (rng.standard_normal((B, C)) * 4).astype(np.float32)
    t = rng.integers(0, C, B).astype(np.int32)
    cols = rng.integers(0, C, (B, 2))
    z[0, cols[0, 0]] = 1e4                      # spike in some later slot
    z[1, t[1]] = 1e4                            # spike on the target
    z[2] -= 200.0                               # every element negative
    z[3] = -np.abs(z[3])                        # all negative, max near zero
    z[3, cols[3, 0]] = -0.0
    z[4, cols[4, 0]] = -1e4                     # one very negative element
    z[5, cols[5]] = 1e4                         # spikes in two places (parts)
    z[6] += 1000.0                              # far up, no overflow
    # each thread's first slot far below its later slots: the first 8192
    # vectors' elements (16-bit: 8 per vector) of the row
    z[7, :8 * 1024] -= 1e4
    z[8, cols[8, 0]] = z[8].max() + 95.0        # past the bound, and past fp32's exp range
    z[9, cols[9, 0]] = z[9].max() + 80.0        # past the bound, inside fp32's exp range
    z[10] = np.where(rng.random(C) < 0.5, -np.abs(z[10]), np.abs(z[10]))
    z[11, :64] = 500.0                          # a run of equal maxima at the head
    bits = synth.bf16_bits_from_f32(z) if dtype == "bf16" else synth.f16_bits_from_f32(z)
    print(f"[part max rows] {B}x{C} {dtype}: {full_parity(bits, t, dtype, where=f'{C} {dtype}')}",
          flush=True)
    # the recompute gives the same bits
    zd, td = to_device(bits, t, dtype)
    g1, l1 = _run(zd, td)
    ce.part_polls(0)
    g0, l0 = _run(zd, td)
    assert torch.equal(_bits(g0), _bits(g1)) and torch.equal(_bits(l0), _bits(l1))
