"""GPU properties that hold at any size: bitwise determinism, full write
coverage, no writes outside the outputs, shift invariance, batch
independence, stream ordering, and the reduction against an exactly
rounded sum of the GPU's own per-row losses."""

from __future__ import annotations

import math

import numpy as np
import pytest

import synth
from oracle import reduce_loss

from _parity import F32_GRAD_ATOL, grad_to_host, run_gpu, to_device

pytestmark = pytest.mark.gpu

# (B, C, dtype, sigma, path): path 0 is the automatic choice
CASES = [
    (16, 10, "f32", 20.0, 0),       # short path
    (64, 1000, "f32", 2.0, 0),      # resident, 256 threads
    (8, 50257, "f32", 3.0, 0),      # two row parts, misaligned rows
    (4, 128256, "bf16", 4.0, 0),    # two row parts
    (300, 70001, "bf16", 4.0, 0),   # one row part with LDS slots, 2-byte aligned rows
    (8, 50257, "f32", 3.0, 2),      # resident, 1024 threads, misaligned rows
    (4, 128256, "bf16", 4.0, 2),    # resident with LDS prefetch
    (300, 70001, "bf16", 4.0, 2),   # LDS prefetch, several rows per workgroup
    (3, 200_000, "bf16", 4.0, 0),   # long rows: four parts
    (2, 100_003, "f32", 3.0, 0),    # long rows, misaligned
    (2, 300_001, "f32", 3.0, 0),    # past eight parts: streamed part (path 3)
]
IDS = [f"{b}x{c}-{d}-p{p}" for b, c, d, _, p in CASES]


@pytest.fixture(autouse=True)
def _reset_path():
    import softmax_cross_entropy_ce_amd as ce
    prev = ce.force_path(0)
    yield
    ce.force_path(prev)


def _force(path):
    import softmax_cross_entropy_ce_amd as ce
    ce.force_path(path)


@pytest.mark.parametrize("B,C,dtype,sigma,path", CASES, ids=IDS)
def test_bitwise_determinism(B, C, dtype, sigma, path):
    import torch
    _force(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=7)
    zd, td = to_device(z, t, dtype)
    ref = run_gpu(zd, td)
    for _ in range(5):
        out = run_gpu(zd, td)
        assert torch.equal(out[0].view(torch.int16 if dtype == "bf16" else torch.int32),
                           ref[0].view(torch.int16 if dtype == "bf16" else torch.int32))
        assert torch.equal(out[1].view(torch.int32), ref[1].view(torch.int32))
        assert torch.equal(out[2].view(torch.int32), ref[2].view(torch.int32))


@pytest.mark.parametrize("B,C,dtype,sigma,path", CASES, ids=IDS)
def test_full_coverage_and_guard_bands(B, C, dtype, sigma, path):
    """Outputs pre-filled with NaN come back NaN-free (every element
    written), and the guard bands around them keep their sentinel (nothing
    written outside)."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    _force(path)
    z, t = synth.make_inputs(B, C, dtype, sigma, seed=8)
    zd, td = to_device(z, t, dtype)
    pad = 4096
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    gbuf = torch.full((B * C + 2 * pad,), float("nan"), dtype=tdt, device=zd.device)
    lbuf = torch.full((B + 2 * pad,), float("nan"), dtype=torch.float32, device=zd.device)
    # keep the 16-byte congruence of grad and logits that the ABI requires
    grad = gbuf[pad:pad + B * C].view(B, C)
    loss_rows = lbuf[pad:pad + B]
    ce.fwd_grad_into(zd, td, grad, loss_rows)
    torch.cuda.synchronize()
    assert not torch.isnan(grad).any()
    assert not torch.isnan(loss_rows).any()
    assert torch.isnan(gbuf[:pad]).all() and torch.isnan(gbuf[pad + B * C:]).all()
    assert torch.isnan(lbuf[:pad]).all() and torch.isnan(lbuf[pad + B:]).all()


@pytest.mark.parametrize("B,C,dtype,sigma,path", CASES, ids=IDS)
def test_shift_invariance(B, C, dtype, sigma, path):
    """Adding a constant to every logit of a row leaves loss and gradient
    unchanged, to a bar derived from the kernels' arithmetic rather than bit
    for bit.  Logits sit on a grid (fp32: multiples of 2^-8 within +-64,
    shift 37; bf16: multiples of 2^-2 within +-8, shift 4) so that the
    shifted inputs are exact.

    Why not bitwise: every kernel forms an element's exponent as one fma,
    z*log2e - c, with c = fl(m * log2e) for the row maximum m.  fl(m log2e)
    and fl((m + k) log2e) differ from the exact products by different
    rounding errors, and each fma result is rounded once more, so a shift
    moves each exponent by at most ulp(c)/2 + ulp(c')/2 + ulp(x)/2 +
    ulp(x')/2: with |c|, |c'|, |x| <= 185 on the fp32 grid that is below
    3.5 * 2^-17 (log2 units), a relative change of each term, and of S, of
    at most 2e-5.  The gradient (at most 1/B) therefore moves by at most
    4e-5/B in fp32, inside 2 * F32_GRAD_ATOL; in bf16 the change is
    a few 1e-6 before rounding, so a result can land on the other side of
    a rounding boundary: at most 1 ulp (relative 2^-7).  The loss moves by
    well under 2e-5 relative.  Forming the exponent as (z - m) * log2e,
    exact on such grids, would cost a second instruction per element in
    both passes over the row."""
    _force(path)
    if dtype == "f32":
        z = synth.grid_logits(B, C, 2.0 ** -8, 64.0, seed=9)
        z2 = z + np.float32(37.0)
    else:
        zf = synth.grid_logits(B, C, 0.25, 8.0, seed=9)
        z = synth.bf16_bits_from_f32(zf)
        z2 = synth.bf16_bits_from_f32(zf + np.float32(4.0))
    t = np.random.Generator(np.random.PCG64(9)).integers(0, C, B).astype(np.int32)
    a = run_gpu(*to_device(z, t, dtype))
    b = run_gpu(*to_device(z2, t, dtype))
    if dtype == "f32":
        assert (a[0] - b[0]).abs().max().item() <= 2 * F32_GRAD_ATOL
    else:
        ga = a[0].float()
        gb = b[0].float()
        assert ((ga - gb).abs() <= ga.abs() * 2 ** -7 + 1e-30).all()
    la, lb = a[2].item(), b[2].item()
    assert abs(la - lb) <= 2e-5 * abs(la) + 1e-7


def test_batch_independence():
    """Row b's outputs times B do not depend on the other rows: a batch of
    32 and its first 8 rows alone agree (B is a power of two, so the 1/B
    scale is exact)."""
    import torch
    z, t = synth.make_inputs(32, 3000, "f32", 3.0, seed=10)
    a = run_gpu(*to_device(z, t, "f32"))
    b = run_gpu(*to_device(z[:8], t[:8], "f32"))
    assert torch.equal(a[0][:8] * 32, b[0] * 8)
    assert torch.equal(a[1][:8] * 32, b[1] * 8)


@pytest.mark.parametrize("B", [1, 7, 2048, 2049, 8192, 16384, 16385, 100_000, 2_097_152, 3_000_001])
def test_reduce_matches_exact_sum_of_gpu_rows(B):
    """The scalar equals the exactly rounded sum of the GPU's own per-row
    values to fp32 summation accuracy, and is bitwise reproducible."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    rng = np.random.Generator(np.random.PCG64(B))
    x = (rng.random(B, dtype=np.float32) * 3.0 / B).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    s1 = ce.reduce_loss(xd)
    s2 = ce.reduce_loss(xd)
    torch.cuda.synchronize()
    assert s1.view(torch.int32).item() == s2.view(torch.int32).item()
    exact = reduce_loss(x.astype(np.float64))
    assert abs(s1.item() - exact) <= 2e-6 * abs(exact)


def test_nondefault_stream_ordering():
    """Calls are ordered on the caller's current stream."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    z, t = synth.make_inputs(256, 5000, "bf16", 4.0, seed=12)
    zd, td = to_device(z, t, "bf16")
    ref = run_gpu(zd, td)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        zz = zd.clone()        # produced on s, consumed on s
        grad, rows = ce.fwd_grad(zz, td)
        loss = ce.reduce_loss(rows)
    s.synchronize()
    assert torch.equal(grad.view(torch.int16), ref[0].view(torch.int16))
    assert loss.item() == ref[2].item()


def test_invalid_target_does_not_disturb_other_rows():
    import torch
    z, t = synth.make_inputs(64, 700, "f32", 2.0, seed=13)
    a = run_gpu(*to_device(z, t, "f32"))
    t2 = t.copy()
    t2[5] = -7
    t2[6] = 700
    b = run_gpu(*to_device(z, t2, "f32"))
    keep = [i for i in range(64) if i not in (5, 6)]
    assert torch.equal(a[0][keep], b[0][keep])
    assert torch.isnan(b[0][5]).all() and torch.isnan(b[0][6]).all()
    assert math.isnan(b[2].item())


@pytest.mark.parametrize("nbytes", [16, 4096, 131072, 131088, (1 << 20) + 48, 3 * 131072 - 16])
def test_stream_copy_is_exact(nbytes):
    """The measurement reference copy moves every byte and nothing else."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    buf = torch.full((nbytes + 4096,), 0xA5, dtype=torch.uint8, device=src.device)
    dst = buf[2048:2048 + nbytes]
    ce.stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert (buf[:2048] == 0xA5).all() and (buf[2048 + nbytes:] == 0xA5).all()


def test_stream_handle_is_torchs_current_stream():
    """The binding passes the raw handle of torch's current stream, on the
    default stream and inside a stream context."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    dev = torch.device("cuda:0")
    assert ce._stream_ptr(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert ce._stream_ptr(dev) == s.cuda_stream
        assert ce._stream_ptr(torch.device("cuda")) == s.cuda_stream
    assert ce._stream_ptr(dev) == torch.cuda.current_stream(dev).cuda_stream
