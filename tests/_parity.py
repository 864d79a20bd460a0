"""Shared helpers of the GPU parity tests: run the HIP path through the
binding, and compare its outputs with the fp64 oracle to the stated bars.

Tolerances (from the definition of the bars):

* fp32 logits: gradient max |g_gpu - g_oracle| <= 1e-6 (absolute); scalar
  loss relative error <= 1e-5; per-row losses (a diagnostic) within
  1e-5 * (|max_c z| + ln C + 1) / B.
* bf16 logits: gradient within 1 bf16 ulp of the oracle's fp64 value
  rounded once to bf16 (nearest even), values below 2^-126 in magnitude
  counting as zero, plus an absolute slack of 2^-50 / B that covers the
  oracle's own rounding of softmax_t - 1 in fp64; scalar loss relative
  error <= 2e-3.
* fp16 logits: gradient within 1 fp16 ulp of the oracle's fp64 value
  rounded once to fp16 (nearest even, with fp16's subnormals, whose
  spacing 2^-24 is then the ulp), plus the same 2^-50 / B slack; the
  arithmetic is float32 on exactly widened inputs, as for fp32, so the
  scalar loss is held to fp32's 1e-5.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import ce_rows, reduce_loss, rne_bf16_bits, rne_f16_bits, widen_bf16, widen_f16

F32_GRAD_ATOL = 1e-6
F32_LOSS_RTOL = 1e-5
BF16_LOSS_RTOL = 2e-3
BF16_MAX_ULP = 1
TINY = 2.0 ** -126


def torch_mod():
    import torch
    return torch


def to_device(logits: np.ndarray, targets: np.ndarray, dtype: str, device="cuda:0"):
    torch = torch_mod()
    if dtype == "f32":
        z = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(device)
    else:
        z = torch.from_numpy(np.ascontiguousarray(logits).view(np.int16)).to(device).view(
            torch.bfloat16 if dtype == "bf16" else torch.float16)
    t = torch.from_numpy(np.ascontiguousarray(targets, dtype=np.int32)).to(device)
    return z, t


def grad_to_host(grad, dtype: str) -> np.ndarray:
    """fp32 gradient as float32 numpy; bf16 / fp16 gradient as uint16 bit
    patterns."""
    torch = torch_mod()
    if dtype == "f32":
        return grad.cpu().numpy()
    return grad.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(z_dev, t_dev):
    """ce_fwd_grad + ce_reduce_loss through the binding; host copies out."""
    import softmax_cross_entropy_ce_amd as ce
    torch = torch_mod()
    grad, loss_rows = ce.fwd_grad(z_dev, t_dev)
    loss = ce.reduce_loss(loss_rows)
    torch.cuda.synchronize()
    return grad, loss_rows, loss


def bf16_order(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bit patterns to integers that count ulps monotonically;
    magnitudes below 2^-126 map to zero."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    mag = np.where(mag < 0x0080, 0, mag)  # exponent field 0: subnormal or zero
    return np.where(b & 0x8000, -mag, mag)


def f16_order(bits: np.ndarray) -> np.ndarray:
    """Map fp16 bit patterns to integers that count ulps monotonically,
    subnormals included (their spacing 2^-24 is fp16's ulp there)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def widen_rows(logits_block: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(logits_block, dtype=np.float64)
    return widen_bf16(logits_block) if dtype == "bf16" else widen_f16(logits_block)


def compare_block(g_gpu: np.ndarray, l_gpu: np.ndarray, z: np.ndarray, t: np.ndarray, B: int,
                  dtype: str, where: str = ""):
    """Compare a block of rows (host arrays) with the oracle; raise on a
    violation.  Returns the worst errors seen (for logging) and the
    oracle's per-row losses of the block."""
    z64 = widen_rows(z, dtype)
    l_ora, g_ora = ce_rows(z64, t, B)
    l_ora_all = l_ora
    valid = (t >= 0) & (t < z.shape[1])
    out = {}
    # invalid targets: NaN loss and an all-NaN gradient row
    if (~valid).any():
        assert np.isnan(l_gpu[~valid]).all(), f"{where}: invalid-target loss not NaN"
        gi = widen_rows(g_gpu[~valid], dtype)
        assert np.isnan(gi).all(), f"{where}: invalid-target gradient not NaN"
    g_gpu, l_gpu, g_ora, l_ora, z64 = (g_gpu[valid], l_gpu[valid], g_ora[valid], l_ora[valid],
                                      z64[valid])
    if g_gpu.size == 0:
        return out, l_ora_all
    if dtype == "f32":
        err = np.abs(g_gpu.astype(np.float64) - g_ora)
        out["grad_abs"] = float(err.max())
        assert np.isfinite(g_gpu).all(), f"{where}: non-finite gradient"
        if out["grad_abs"] > F32_GRAD_ATOL:
            r, c = np.unravel_index(int(err.argmax()), err.shape)
            raise AssertionError(f"{where}: fp32 gradient error {out['grad_abs']:.3g} > "
                                 f"{F32_GRAD_ATOL} at row {r} col {c}: gpu {g_gpu[r, c]!r} "
                                 f"oracle {g_ora[r, c]!r}")
    else:
        rne, order = (rne_bf16_bits, bf16_order) if dtype == "bf16" else (rne_f16_bits, f16_order)
        want = rne(g_ora)
        ulp = np.abs(order(g_gpu) - order(want))
        slack = np.abs(widen_rows(g_gpu, dtype) - g_ora) <= 2.0 ** -50 / B
        bad = (ulp > BF16_MAX_ULP) & ~slack
        out["grad_ulp"] = int(ulp.max())
        if bad.any():
            r, c = np.argwhere(bad)[0]
            raise AssertionError(f"{where}: {dtype} gradient {ulp[r, c]} ulp from RNE(oracle) at "
                                 f"row {r} col {c}: gpu bits {g_gpu[r, c]:#06x} want "
                                 f"{want[r, c]:#06x} (oracle {g_ora[r, c]!r})")
    # per-row loss diagnostic
    C = z.shape[1]
    # both dtypes are accumulated in fp32 from exact inputs: one bar
    tol = 1e-5 * (np.abs(z64.max(axis=1)) + math.log(C) + 1.0) / B
    lerr = np.abs(l_gpu.astype(np.float64) - l_ora)
    out["loss_row_abs"] = float(lerr.max())
    if (lerr > tol).any():
        r = int(np.argmax(lerr - tol))
        raise AssertionError(f"{where}: per-row loss error {lerr[r]:.3g} > {tol[r]:.3g} at row "
                             f"{r}: gpu {l_gpu[r]!r} oracle {l_ora[r]!r}")
    return out, l_ora_all


def compare_scalar(loss_gpu: float, loss_rows_oracle_sum: float, dtype: str, where: str = ""):
    rtol = BF16_LOSS_RTOL if dtype == "bf16" else F32_LOSS_RTOL
    denom = max(abs(loss_rows_oracle_sum), 1e-30)
    rel = abs(loss_gpu - loss_rows_oracle_sum) / denom
    assert rel <= rtol or abs(loss_gpu - loss_rows_oracle_sum) <= 1e-30, (
        f"{where}: scalar loss {loss_gpu!r} vs oracle {loss_rows_oracle_sum!r} "
        f"(rel {rel:.3g} > {rtol})")
    return rel


def full_parity(logits: np.ndarray, targets: np.ndarray, dtype: str, block_elems=1 << 23,
                where: str = "") -> dict:
    """Run the GPU path on the whole input and compare every row (in row
    blocks) and the scalar with the oracle."""
    z_dev, t_dev = to_device(logits, targets, dtype)
    grad, loss_rows, loss = run_gpu(z_dev, t_dev)
    B, C = logits.shape
    lr = loss_rows.cpu().numpy()
    step = max(1, block_elems // C)
    worst: dict = {}
    ora_rows = []
    for lo in range(0, B, step):
        hi = min(B, lo + step)
        g = grad_to_host(grad[lo:hi], dtype)
        res, l_ora = compare_block(g, lr[lo:hi], logits[lo:hi], targets[lo:hi], B, dtype,
                                   where=f"{where} rows {lo}:{hi}")
        for k, v in res.items():
            worst[k] = max(worst.get(k, 0), v)
        ora_rows.append(l_ora)
    valid = (targets >= 0) & (targets < C)
    if valid.all():
        worst["loss_rel"] = compare_scalar(float(loss.item()), reduce_loss(np.concatenate(ora_rows)),
                                           dtype, where)
    else:
        assert math.isnan(float(loss.item()))
    return worst


# ---------------------------------------------------------------- path 5
def wave_vector_bytes(es: int, lens, addrs=()) -> int:
    """The vector bytes path 5 loads rows with: the widest of 16, 8 and 4
    that divides every row length and stride (lens, in elements) and every
    array base (addrs), else 0."""
    for vb in (16, 8, 4):
        if vb >= es and all(n % (vb // es) == 0 for n in lens) and all(a % vb == 0 for a in addrs):
            return vb
    return 0


def wave_takes(C: int, es: int, lens=None, addrs=()) -> bool:
    """Whether path 5 has a configuration for rows of C elements (rows of at
    most 64 lanes x 256 bytes, 128 bytes with 4-byte vectors)."""
    vb = wave_vector_bytes(es, lens if lens is not None else (C,), addrs)
    if vb == 0:
        return False
    for lb in (16, 32, 64, 128, 256):
        if lb >= vb and 64 * lb >= C * es:
            return not (vb == 4 and lb > 128)
    return False


def path_takes(path: int, C: int, dtype: str) -> bool:
    """Whether a forced path takes contiguous rows of C elements from
    16-byte aligned arrays (short: C <= 256; resident: at most 16384
    16-byte vectors; parts: an aligned body of at most 65536 vectors;
    wave: wave_takes)."""
    es = 4 if dtype == "f32" else 2
    if path == 1:
        return C <= 256
    if path == 2:
        return (C * es + 15) // 16 + 1 <= 16384
    if path == 4:
        return C // (16 // es) <= 65536
    if path == 5:
        return wave_takes(C, es)
    return True


def wave_bwd_takes(C: int, es: int, addrs=()) -> bool:
    """Whether path 5's softmax backward takes contiguous rows of C elements
    (as wave_takes, rows of at most 8 KB)."""
    return C * es <= 8192 and wave_takes(C, es, (C,), addrs)
