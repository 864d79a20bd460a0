"""Fused softmax cross-entropy for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libce_mi355x.so`` (C ABI in ``include/ce.h``).
It checks tensor dtypes, devices and contiguity, allocates outputs with
torch and passes raw device pointers plus torch's current HIP stream; every
step of the computation runs in the library's HIP kernels.  There is no CPU
or PyTorch fallback: if the library is missing, importing the binding's
functions raises.

The operation (rumus project page, milestone M7a; rumus 0.1.1
``cross_entropy.wgsl`` pass 1 and pass 2): for logits ``z`` of shape
``[B, C]`` and int32 targets ``t``::

    loss_rows[b] = (logsumexp(z[b]) - z[b, t[b]]) / B
    grad[b, c]   = (softmax(z[b])[c] - [c == t[b]]) / B
    loss         = sum_b loss_rows[b]

Beside it, on the same kernels: the row-wise softmax forward and backward
(rumus project page, milestone M8c) and the cross-entropy of a vocabulary
split into column shards (per-shard records, then a combine that writes
each shard's gradient).
"""

from __future__ import annotations

import ctypes
import functools
import os

__all__ = [
    "CEError", "lib", "fwd_grad", "fwd_grad_into", "reduce_loss", "reduce_loss_into",
    "cross_entropy", "cross_entropy_loss", "fwd_grad_scaled_into", "scale_grad_",
    "reduce_loss_noalloc_into",
    "fwd_loss", "fwd_loss_into", "fwd_grad_inplace_",
    "softmax_fwd", "softmax_fwd_into", "softmax_bwd", "softmax_bwd_into", "softmax",
    "shard_stats", "shard_stats_into", "shard_grad", "shard_grad_into",
    "reduce_workspace_bytes", "select_path", "force_path", "part_polls", "part_counter",
    "stream_copy", "version", "PATH_NAMES", "F32", "BF16", "F16", "NO_IGNORE",
    "fwd_grad_ex_into", "fwd_grad_ex", "fwd_workspace_bytes", "fwd_inplace_workspace_bytes",
    "inplace_workspace", "fwd_grad_loss_into",
]

F32 = 0
BF16 = 1
F16 = 2
NO_IGNORE = -(1 << 31)
PATH_NAMES = {1: "short", 2: "resident", 3: "long", 4: "parts", 5: "wave"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libce_mi355x.so")


class CEError(RuntimeError):
    """A negative status from the C library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing; build it with "
            "`python -m softmax_cross_entropy_ce_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    L.ce_fwd_grad.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp]
    L.ce_fwd_grad.restype = i32
    L.ce_reduce_workspace_bytes.argtypes = [i64]
    L.ce_reduce_workspace_bytes.restype = sz
    L.ce_reduce_loss.argtypes = [vp, i64, vp, vp, sz, vp]
    L.ce_reduce_loss.restype = i32
    L.ce_reduce_loss_noalloc.argtypes = [vp, i64, vp, vp]
    L.ce_reduce_loss_noalloc.restype = i32
    L.ce_fwd_grad_loss.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp, sz, vp]
    L.ce_fwd_grad_loss.restype = i32
    L.ce_status_string.argtypes = [i32]
    L.ce_status_string.restype = ctypes.c_char_p
    L.ce_version.argtypes = []
    L.ce_version.restype = ctypes.c_char_p
    L.ce_select_path.argtypes = [i64, i32]
    L.ce_select_path.restype = i32
    L.ce_debug_force_path.argtypes = [i32]
    L.ce_debug_force_path.restype = i32
    L.ce_debug_part_polls.argtypes = [i32]
    L.ce_debug_part_polls.restype = i32
    L.ce_debug_part_counter.argtypes = [vp]
    L.ce_debug_part_counter.restype = i32
    L.ce_debug_time_next_launch.argtypes = [vp, vp]
    L.ce_debug_time_next_launch.restype = i32
    L.ce_stream_copy.argtypes = [vp, vp, i64, vp]
    L.ce_stream_copy.restype = i32
    L.ce_fwd_grad_scaled.argtypes = [vp, vp, i64, i64, i32, vp, vp, vp, vp]
    L.ce_fwd_grad_scaled.restype = i32
    L.ce_scale_grad.argtypes = [vp, i64, i32, vp, vp]
    L.ce_scale_grad.restype = i32
    L.ce_fwd_loss.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.ce_fwd_loss.restype = i32
    L.ce_softmax_fwd.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    L.ce_softmax_fwd.restype = i32
    L.ce_softmax_bwd.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    L.ce_softmax_bwd.restype = i32
    L.ce_shard_stats.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp]
    L.ce_shard_stats.restype = i32
    L.ce_shard_grad.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp, i32, vp, vp, vp, vp]
    L.ce_shard_grad.restype = i32
    L.ce_fwd_workspace_bytes.argtypes = [ctypes.c_int32]
    L.ce_fwd_workspace_bytes.restype = sz
    L.ce_fwd_grad_ex.argtypes = [vp, i64, vp, i64, i64, i32, vp, i64, vp, vp, ctypes.c_int32, vp,
                                 sz, vp]
    L.ce_fwd_grad_ex.restype = i32
    L.ce_fwd_inplace_workspace_bytes.argtypes = [i64]
    L.ce_fwd_inplace_workspace_bytes.restype = sz
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().ce_status_string(int(status)).decode()


def version() -> str:
    return lib().ce_version().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise CEError(status, what)


def select_path(C: int, dtype: int) -> int:
    r = lib().ce_select_path(int(C), int(dtype))
    _check(0 if r > 0 else r, "ce_select_path")
    return r


def force_path(path: int) -> int:
    """Test hook: force a kernel path (0 = automatic).  Returns the previous."""
    r = lib().ce_debug_force_path(int(path))
    if r < 0:
        raise CEError(r, "ce_debug_force_path")
    return r


def part_polls(polls: int) -> int:
    """Test hook: polls of a path-4 row part for its partners' pairs before
    it recomputes the missing ones (0: always recompute).  Returns the
    previous value."""
    r = lib().ce_debug_part_polls(int(polls))
    if r < 0:
        raise CEError(r, "ce_debug_part_polls")
    return r


def part_counter(counter=None) -> None:
    """Test hook: a one-element int32/uint32 device tensor to which every
    path-4 part adds the number of partner pairs it recomputed (None turns
    counting off).
    The tensor must stay alive until the calls made with it have run."""
    if counter is None:
        ptr = None
    else:
        _check_cuda(counter)
        if counter.numel() < 1 or counter.element_size() != 4 or not counter.is_contiguous():
            raise ValueError("counter must be a contiguous 4-byte integer tensor")
        ptr = counter.data_ptr()
    _check(lib().ce_debug_part_counter(ptr), "ce_debug_part_counter")


def stream_copy(src, dst) -> None:
    """Measurement reference: copy src's bytes into dst with the library's
    streaming copy kernel (both contiguous device tensors of equal byte
    size, a multiple of 16)."""
    _check_cuda(src, dst)
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst differ in size")
    _check(lib().ce_stream_copy(src.data_ptr(), dst.data_ptr(), n, _stream_ptr(src.device)),
           "ce_stream_copy")


@functools.lru_cache(maxsize=64)
def reduce_workspace_bytes(B: int) -> int:
    return int(lib().ce_reduce_workspace_bytes(int(B)))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"logits must be float32, bfloat16 or float16, got {t.dtype}")


_raw_stream = None


def _stream_ptr(device) -> int:
    """The raw handle of torch's current HIP stream on ``device``.  torch's
    ``_cuda_getCurrentRawStream`` returns it without building a Stream
    object (about 0.1 us against 2 us); older builds without it take the
    public path."""
    global _raw_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return _raw_stream(idx)
    return torch.cuda.current_stream(device).cuda_stream


def _check_cuda(*ts) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on a HIP device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    dev = ts[0].device
    if any(t.device != dev for t in ts):
        raise ValueError("tensors must be on one device")


def _empty_congruent(x):
    """A new contiguous tensor of x's shape and dtype whose address has the
    same offset modulo 16 bytes as x's (the kernels read and write matching
    rows with the same 16-byte vector split, so the library requires it)."""
    torch = _torch()
    mis = x.data_ptr() % 16
    if mis == 0:
        return torch.empty(x.shape, dtype=x.dtype, device=x.device)
    es = x.element_size()
    n = x.numel()
    flat = torch.empty(n + 16 // es, dtype=x.dtype, device=x.device)
    off = ((mis - flat.data_ptr() % 16) % 16) // es
    return flat[off:off + n].view(x.shape)


def _empty_rows_congruent(x, ld: int):
    """As _empty_congruent for a [B, C] view with row stride ld: a [B, C]
    view of a new buffer with the same row stride and offset modulo 16."""
    torch = _torch()
    B, C = x.shape
    if ld == C:
        return _empty_congruent(x)
    es = x.element_size()
    mis = x.data_ptr() % 16
    flat = torch.empty(B * ld + 16 // es, dtype=x.dtype, device=x.device)
    off = ((mis - flat.data_ptr() % 16) % 16) // es
    return flat[off:off + B * ld].view(B, ld)[:, :C]


def _check_fwd_args(logits, targets, grad, loss_rows):
    torch = _torch()
    _check_cuda(logits, targets, grad, loss_rows)
    if logits.dim() != 2:
        raise ValueError("logits must be [B, C]")
    B, C = logits.shape
    if targets.dtype != torch.int32 or targets.shape != (B,):
        raise TypeError("targets must be int32 of shape [B]")
    if grad.dtype != logits.dtype or grad.shape != logits.shape:
        raise TypeError("grad must match logits in dtype and shape")
    if loss_rows.dtype != torch.float32 or loss_rows.shape != (B,):
        raise TypeError("loss_rows must be float32 of shape [B]")
    return B, C


def _check_scalar(x, what: str):
    torch = _torch()
    _check_cuda(x)
    if x.dtype != torch.float32 or x.numel() != 1:
        raise TypeError(f"{what} must be one float32 on the device")


def fwd_grad_into(logits, targets, grad, loss_rows) -> None:
    """Write the gradient and the per-row losses into preallocated tensors."""
    B, C = _check_fwd_args(logits, targets, grad, loss_rows)
    st = lib().ce_fwd_grad(logits.data_ptr(), targets.data_ptr(), B, C, _dtype_code(logits),
                           grad.data_ptr(), loss_rows.data_ptr(), _stream_ptr(logits.device))
    _check(st, "ce_fwd_grad")


def fwd_grad_loss_into(logits, targets, grad, loss_rows, loss, workspace=None) -> None:
    """The gradient, the per-row losses and the batch-mean loss (one float32
    tensor ``loss``) in one library call (ce_fwd_grad_loss: ce_fwd_grad,
    then ce_reduce_loss).  ``workspace``: device bytes of at least
    reduce_workspace_bytes(B), or None to allocate them when needed."""
    torch = _torch()
    B, C = _check_fwd_args(logits, targets, grad, loss_rows)
    _check_cuda(logits, loss)
    if loss.dtype != torch.float32 or loss.numel() != 1:
        raise TypeError("loss must be one float32")
    need = reduce_workspace_bytes(B)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().ce_fwd_grad_loss(logits.data_ptr(), targets.data_ptr(), B, C, _dtype_code(logits),
                                grad.data_ptr(), loss_rows.data_ptr(), loss.data_ptr(), wptr,
                                wbytes, _stream_ptr(logits.device))
    _check(st, "ce_fwd_grad_loss")


def fwd_grad_inplace_(logits, targets):
    """Overwrite logits with the gradient (softmax - onehot) / B and return
    the per-row losses (ce_fwd_grad_ex with the in-place workspace of
    torch's current stream, so rows of several parts stay on path 4)."""
    torch = _torch()
    loss_rows = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    fwd_grad_ex_into(logits, targets, logits, loss_rows)
    return loss_rows


def fwd_loss_into(logits, targets, loss_rows) -> None:
    """Per-row losses only (the logits are read once, no gradient)."""
    torch = _torch()
    _check_cuda(logits, targets, loss_rows)
    if logits.dim() != 2:
        raise ValueError("logits must be [B, C]")
    B, C = logits.shape
    if targets.dtype != torch.int32 or targets.shape != (B,):
        raise TypeError("targets must be int32 of shape [B]")
    if loss_rows.dtype != torch.float32 or loss_rows.shape != (B,):
        raise TypeError("loss_rows must be float32 of shape [B]")
    st = lib().ce_fwd_loss(logits.data_ptr(), targets.data_ptr(), B, C, _dtype_code(logits),
                           loss_rows.data_ptr(), _stream_ptr(logits.device))
    _check(st, "ce_fwd_loss")


def fwd_loss(logits, targets):
    """The per-row losses (already scaled by 1/B) of ``[B, C]`` logits."""
    torch = _torch()
    loss_rows = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    fwd_loss_into(logits, targets, loss_rows)
    return loss_rows


def fwd_grad_scaled_into(logits, targets, grad, loss_rows, grad_scale) -> None:
    """As fwd_grad_into, with the gradient multiplied by the device scalar
    grad_scale (one float32) in the same pass; loss_rows are not scaled."""
    B, C = _check_fwd_args(logits, targets, grad, loss_rows)
    _check_scalar(grad_scale, "grad_scale")
    st = lib().ce_fwd_grad_scaled(logits.data_ptr(), targets.data_ptr(), B, C,
                                  _dtype_code(logits), grad.data_ptr(), loss_rows.data_ptr(),
                                  grad_scale.data_ptr(), _stream_ptr(logits.device))
    _check(st, "ce_fwd_grad_scaled")


def scale_grad_(grad, scale) -> None:
    """The backward broadcast-scale: grad *= scale in place, scale a device
    float32 scalar (nothing is read back to the host; a scale of exactly 1
    leaves grad untouched without moving its bytes)."""
    _check_cuda(grad)
    _check_scalar(scale, "scale")
    st = lib().ce_scale_grad(grad.data_ptr(), grad.numel(), _dtype_code(grad), scale.data_ptr(),
                             _stream_ptr(grad.device))
    _check(st, "ce_scale_grad")


def fwd_workspace_bytes(ignore_index=None) -> int:
    return int(lib().ce_fwd_workspace_bytes(NO_IGNORE if ignore_index is None else int(ignore_index)))


def fwd_inplace_workspace_bytes(B: int) -> int:
    return int(lib().ce_fwd_inplace_workspace_bytes(int(B)))


# Zero-filled in-place workspaces of ce_fwd_grad_ex, one per (device,
# stream): a call leaves its row words zero again, so one workspace serves
# every call ordered on its stream; calls on other streams get their own.
_inplace_ws = {}


def inplace_workspace(device, B: int):
    """The cached in-place workspace of torch's current stream on ``device``,
    grown (zero-filled) to fit B rows."""
    torch = _torch()
    key = (device.index if device.index is not None else torch.cuda.current_device(),
           _stream_ptr(device))
    need = fwd_inplace_workspace_bytes(B)
    ws = _inplace_ws.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=device)
        _inplace_ws[key] = ws
    return ws


def _rows_view(x, what: str):
    """A [B, C] device tensor whose rows are contiguous (column stride 1);
    returns its row stride in elements."""
    if not x.is_cuda:
        raise ValueError("tensors must live on a HIP device")
    if x.dim() != 2:
        raise ValueError(f"{what} must be [B, C]")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError(f"{what} must have contiguous rows (column stride 1)")
    return x.stride(0) if x.shape[0] > 1 else max(x.shape[1], x.stride(0))


def fwd_grad_ex_into(logits, targets, grad, loss_rows, grad_scale=None, ignore_index=None,
                     workspace=None) -> None:
    """ce_fwd_grad_ex: logits and grad may be row-strided views (rows
    contiguous); grad None gives the losses only; grad_scale is an optional
    device scalar; rows whose target equals ignore_index give loss 0 and a
    zero gradient row, and the rest are averaged over the rows kept."""
    torch = _torch()
    ldz = _rows_view(logits, "logits")
    B, C = logits.shape
    _check_cuda(targets, loss_rows)
    if targets.dtype != torch.int32 or targets.shape != (B,):
        raise TypeError("targets must be int32 of shape [B]")
    if loss_rows.dtype != torch.float32 or loss_rows.shape != (B,):
        raise TypeError("loss_rows must be float32 of shape [B]")
    ldg = 0
    if grad is not None:
        ldg = _rows_view(grad, "grad")
        if grad.dtype != logits.dtype or grad.shape != logits.shape:
            raise TypeError("grad must match logits in dtype and shape")
    if grad_scale is not None:
        _check_scalar(grad_scale, "grad_scale")
    ii = NO_IGNORE if ignore_index is None else int(ignore_index)
    need = fwd_workspace_bytes(ignore_index)
    in_place = grad is not None and grad.data_ptr() == logits.data_ptr() and ldg == ldz
    if workspace is None and in_place:
        workspace = inplace_workspace(logits.device, B)
    elif need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    st = lib().ce_fwd_grad_ex(
        logits.data_ptr(), ldz, targets.data_ptr(), B, C, _dtype_code(logits),
        grad.data_ptr() if grad is not None else None, ldg, loss_rows.data_ptr(),
        grad_scale.data_ptr() if grad_scale is not None else None, ii,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream_ptr(logits.device))
    _check(st, "ce_fwd_grad_ex")


def fwd_grad_ex(logits, targets, ignore_index=None, grad_scale=None, with_grad: bool = True):
    """Return ``(grad, loss_rows)`` (grad None when with_grad is False) for
    row-strided logits, with the options of fwd_grad_ex_into.  grad has the
    logits' row stride."""
    torch = _torch()
    grad = _empty_rows_congruent(logits, _rows_view(logits, "logits")) if with_grad else None
    loss_rows = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    fwd_grad_ex_into(logits, targets, grad, loss_rows, grad_scale, ignore_index)
    return grad, loss_rows


def fwd_grad(logits, targets):
    """Return ``(grad, loss_rows)`` for ``[B, C]`` logits and int32 targets."""
    torch = _torch()
    grad = _empty_congruent(logits)
    loss_rows = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    fwd_grad_into(logits, targets, grad, loss_rows)
    return grad, loss_rows


def reduce_loss_into(loss_rows, out, workspace=None) -> None:
    torch = _torch()
    _check_cuda(loss_rows, out)
    if loss_rows.dtype != torch.float32 or loss_rows.dim() != 1:
        raise TypeError("loss_rows must be a float32 vector")
    if out.dtype != torch.float32 or out.numel() != 1:
        raise TypeError("out must be one float32")
    B = loss_rows.shape[0]
    need = reduce_workspace_bytes(B)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=loss_rows.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().ce_reduce_loss(loss_rows.data_ptr(), B, out.data_ptr(), wptr, wbytes,
                              _stream_ptr(loss_rows.device))
    _check(st, "ce_reduce_loss")


def reduce_loss_noalloc_into(loss_rows, out) -> None:
    """ce_reduce_loss_noalloc: the sum into ``out`` with no workspace (the
    library's per-GPU scratch holds the partial sums; calls that overlap on
    one GPU race)."""
    torch = _torch()
    _check_cuda(loss_rows, out)
    if loss_rows.dtype != torch.float32 or loss_rows.dim() != 1:
        raise TypeError("loss_rows must be a float32 vector")
    if out.dtype != torch.float32 or out.numel() != 1:
        raise TypeError("out must be one float32")
    st = lib().ce_reduce_loss_noalloc(loss_rows.data_ptr(), loss_rows.shape[0], out.data_ptr(),
                                      _stream_ptr(loss_rows.device))
    _check(st, "ce_reduce_loss_noalloc")


def reduce_loss(loss_rows):
    """The batch-mean loss as a 0-d float32 device tensor."""
    torch = _torch()
    out = torch.empty((), dtype=torch.float32, device=loss_rows.device)
    reduce_loss_into(loss_rows, out)
    return out


def _fwd_grad_loss(logits, targets):
    """``(loss, grad, loss_rows)`` in one library call (ce_fwd_grad_loss)."""
    torch = _torch()
    grad = _empty_congruent(logits)
    loss_rows = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device)
    loss = torch.empty((), dtype=torch.float32, device=logits.device)
    fwd_grad_loss_into(logits, targets, grad, loss_rows, loss)
    return loss, grad, loss_rows


def cross_entropy(logits, targets):
    """Return ``(loss, grad)``: the batch-mean loss (0-d device tensor) and
    the gradient with respect to the logits."""
    loss, grad, _ = _fwd_grad_loss(logits, targets)
    return loss, grad


_autograd_fn = None


def _function():
    global _autograd_fn
    if _autograd_fn is not None:
        return _autograd_fn
    torch = _torch()

    class CrossEntropyFunction(torch.autograd.Function):
        """Forward: the batch-mean loss and, in the same pass, its gradient
        (ce_fwd_grad_loss; with ignore_index ce_fwd_grad_ex + ce_reduce_loss).
        Backward: that gradient scaled in place by the upstream gradient
        (ce_scale_grad), a device scalar, so there is no host
        synchronisation; one backward per forward."""

        @staticmethod
        def forward(ctx, logits, targets, ignore_index=None):
            if ignore_index is None:
                loss, grad, _ = _fwd_grad_loss(logits.detach(), targets)
                ctx.grad = grad
                return loss
            grad, loss_rows = fwd_grad_ex(logits.detach(), targets, ignore_index=ignore_index)
            ctx.grad = grad
            return reduce_loss(loss_rows)

        @staticmethod
        def backward(ctx, grad_output):
            grad = ctx.grad
            if grad is None:
                raise RuntimeError("cross_entropy_loss: backward can run once per forward")
            ctx.grad = None
            scale_grad_(grad, grad_output.detach().to(torch.float32).reshape(1).contiguous())
            return grad, None, None

    _autograd_fn = CrossEntropyFunction
    return _autograd_fn


def cross_entropy_loss(logits, targets, ignore_index=None):
    """The batch-mean fused cross-entropy as a differentiable 0-d tensor:
    ``loss.backward()`` gives ``logits.grad = (softmax - onehot) / B`` times
    the upstream gradient, from the gradient formed in the forward pass.
    With ignore_index, rows whose target equals it are left out of the
    mean (the mean is over the other rows)."""
    return _function().apply(logits, targets, ignore_index)


# ---------------------------------------------------------------- softmax

def _check_pair(a, b, what: str):
    if b.dtype != a.dtype or b.shape != a.shape:
        raise TypeError(f"{what} must match in dtype and shape")


def softmax_fwd_into(x, y, lse=None) -> None:
    """Row-wise softmax of ``[B, C]`` x into y (y may be x itself), and the
    rows' log-sum-exp into lse (float32 [B]) when it is given."""
    torch = _torch()
    _check_cuda(x, y, *([lse] if lse is not None else []))
    if x.dim() != 2:
        raise ValueError("x must be [B, C]")
    _check_pair(x, y, "x and y")
    B, C = x.shape
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B,)):
        raise TypeError("lse must be float32 of shape [B]")
    st = lib().ce_softmax_fwd(x.data_ptr(), B, C, _dtype_code(x), y.data_ptr(),
                              lse.data_ptr() if lse is not None else None,
                              _stream_ptr(x.device))
    _check(st, "ce_softmax_fwd")


def softmax_fwd(x, with_lse: bool = False):
    """The row-wise softmax of ``[B, C]`` x; with ``with_lse`` also the rows'
    log-sum-exp (float32 [B])."""
    torch = _torch()
    y = _empty_congruent(x)
    lse = torch.empty(x.shape[0], dtype=torch.float32, device=x.device) if with_lse else None
    softmax_fwd_into(x, y, lse)
    return (y, lse) if with_lse else y


def softmax_bwd_into(y, dy, dx) -> None:
    """dx = y * (dy - rowsum(dy * y)), the backward of the row-wise softmax
    from its output y and the upstream gradient dy (dx may be y or dy)."""
    _check_cuda(y, dy, dx)
    if y.dim() != 2:
        raise ValueError("y must be [B, C]")
    _check_pair(y, dy, "y and dy")
    _check_pair(y, dx, "y and dx")
    B, C = y.shape
    st = lib().ce_softmax_bwd(y.data_ptr(), dy.data_ptr(), B, C, _dtype_code(y), dx.data_ptr(),
                              _stream_ptr(y.device))
    _check(st, "ce_softmax_bwd")


def softmax_bwd(y, dy):
    """dx for y and dy; dy is first copied to an address congruent to y's
    modulo 16 bytes if it is not (the library requires it)."""
    if (dy.data_ptr() - y.data_ptr()) % 16:
        t = _empty_congruent(y)
        t.copy_(dy)
        dy = t
    dx = _empty_congruent(y)
    softmax_bwd_into(y, dy, dx)
    return dx


_softmax_fn = None


def softmax(x):
    """Differentiable row-wise softmax of ``[B, C]`` x: the forward keeps its
    output for the backward (ce_softmax_fwd, then ce_softmax_bwd)."""
    global _softmax_fn
    if _softmax_fn is None:
        torch = _torch()

        class SoftmaxFunction(torch.autograd.Function):
            @staticmethod
            def forward(ctx, x):
                y = softmax_fwd(x.detach().contiguous())
                ctx.save_for_backward(y)
                return y

            @staticmethod
            def backward(ctx, dy):
                (y,) = ctx.saved_tensors
                return softmax_bwd(y, dy.contiguous())

        _softmax_fn = SoftmaxFunction
    return _softmax_fn.apply(x)


# ------------------------------------------------------ vocabulary shards

def shard_stats_into(logits, targets, col0: int, records) -> None:
    """Per-row record (c, sx, zt, own) of one vocabulary shard: the columns
    [col0, col0 + C) of the rows, as a contiguous ``[B, C]`` tensor, with
    the rows' global int32 targets.  records: float32 ``[B, 4]``."""
    torch = _torch()
    _check_cuda(logits, targets, records)
    if logits.dim() != 2:
        raise ValueError("logits must be [B, C]")
    B, C = logits.shape
    if targets.dtype != torch.int32 or targets.shape != (B,):
        raise TypeError("targets must be int32 of shape [B]")
    if records.dtype != torch.float32 or records.shape != (B, 4):
        raise TypeError("records must be float32 of shape [B, 4]")
    st = lib().ce_shard_stats(logits.data_ptr(), targets.data_ptr(), B, C, int(col0),
                              _dtype_code(logits), records.data_ptr(), _stream_ptr(logits.device))
    _check(st, "ce_shard_stats")


def shard_stats(logits, targets, col0: int):
    torch = _torch()
    rec = torch.empty((logits.shape[0], 4), dtype=torch.float32, device=logits.device)
    shard_stats_into(logits, targets, col0, rec)
    return rec


def shard_grad_into(logits, targets, col0: int, C_total: int, records, grad, loss_rows=None,
                    grad_scale=None) -> None:
    """One shard's gradient (and, when loss_rows is given, the rows' losses)
    from the records of all shards, float32 ``[N, B, 4]`` in shard order."""
    torch = _torch()
    extra = [t for t in (loss_rows, grad_scale) if t is not None]
    _check_cuda(logits, targets, records, grad, *extra)
    if logits.dim() != 2:
        raise ValueError("logits must be [B, C]")
    B, C = logits.shape
    if targets.dtype != torch.int32 or targets.shape != (B,):
        raise TypeError("targets must be int32 of shape [B]")
    if records.dtype != torch.float32 or records.dim() != 3 or records.shape[1:] != (B, 4):
        raise TypeError("records must be float32 of shape [N, B, 4]")
    _check_pair(logits, grad, "logits and grad")
    if loss_rows is not None and (loss_rows.dtype != torch.float32 or loss_rows.shape != (B,)):
        raise TypeError("loss_rows must be float32 of shape [B]")
    if grad_scale is not None:
        _check_scalar(grad_scale, "grad_scale")
    st = lib().ce_shard_grad(logits.data_ptr(), targets.data_ptr(), B, C, int(col0), int(C_total),
                             _dtype_code(logits), records.data_ptr(), records.shape[0],
                             grad.data_ptr(),
                             loss_rows.data_ptr() if loss_rows is not None else None,
                             grad_scale.data_ptr() if grad_scale is not None else None,
                             _stream_ptr(logits.device))
    _check(st, "ce_shard_grad")


def shard_grad(logits, targets, col0: int, C_total: int, records, with_loss: bool = False):
    torch = _torch()
    grad = _empty_congruent(logits)
    lr = torch.empty(logits.shape[0], dtype=torch.float32, device=logits.device) if with_loss else None
    shard_grad_into(logits, targets, col0, C_total, records, grad, lr)
    return (grad, lr) if with_loss else grad
