#!/usr/bin/env python3
"""Benchmark of fused softmax cross-entropy (forward + gradient + batch-mean
loss) on one MI355X.

A step is one pass of the whole path over one batch: ce_fwd_grad (per-row
loss and gradient) then ce_reduce_loss (the batch mean), on inputs already
resident in HBM.  The default workload is the LM-head case of 8192 rows of
128256 bf16 logits (N(0, 4)), int32 targets uniform in [0, C).

Prints one JSON line on stdout.  `value` is achieved HBM GB/s of the
counted bytes (logits read + gradient written) over the whole step;
rows/s is reported beside it.  `roofline` is for the dominant kernel
(ce_fwd_grad) timed alone with HIP events on the stream it runs on.
`cpu_baseline` is the fp64 numpy oracle timed on this host on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --mode copy --copy-mib 1024   # plain device copy, for counter calibration
    python bench.py --mode sweep                  # rates across row lengths, against a copy
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "ce_fwd_grad_{workload}_traffic.json")
CSRC = os.path.join(ROOT, "softmax_cross_entropy_ce_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str):
    """Measured HBM bytes per ce_fwd_grad launch, if counters were taken on
    the current kernel source (else None)."""
    try:
        with open(TRAFFIC_GLOB.format(workload=workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


class HipEvents:
    """HIP events created through the HIP runtime that the library and
    torch share (resolved through the library's handle), for
    ce_debug_time_next_launch: the library's next launch records them at
    the kernel's own start and end, with no event packets between the
    kernels of the timed loop."""

    def __init__(self):
        import ctypes
        import softmax_cross_entropy_ce_amd as ce
        self._c = ctypes
        L = ce.lib()
        self.L = L
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventCreateWithFlags.restype = ctypes.c_int
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        L.hipEventElapsedTime.restype = ctypes.c_int
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        L.hipEventDestroy.restype = ctypes.c_int
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventRecord.restype = ctypes.c_int
        self.events = []

    # hipEventDisableSystemFence: the events time kernels and synchronise
    # nothing (the host synchronises the device before reading them), so
    # they skip the system-scope fence, a cache write-back and invalidate
    # that otherwise follows each timed kernel.  Measured on lmhead128k, 20
    # steps with 4 pairs: 702.0 us per step and 697.5 us for the kernel with
    # default events, 699.5 and 694.4 us with these; lmhead50k 279.6 and
    # 276.5 against 278.6 and 274.6 us.
    FLAGS = 0x20000000

    def pairs(self, n: int):
        out = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                ev = self._c.c_void_p()
                if self.L.hipEventCreateWithFlags(self._c.byref(ev), self.FLAGS) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                self.events.append(ev)
                pair.append(ev)
            out.append(tuple(pair))
        return out

    def arm(self, pair) -> None:
        """The library's next launch on this thread records this pair."""
        self.L.ce_debug_time_next_launch(pair[0], pair[1])

    def record(self, ev, stream_handle: int) -> None:
        """Record one event on a stream (a marker between launches)."""
        if self.L.hipEventRecord(ev, stream_handle) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, pair) -> float:
        v = self._c.c_float()
        if self.L.hipEventElapsedTime(self._c.byref(v), pair[0], pair[1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(v.value)

    def close(self) -> None:
        for ev in self.events:
            self.L.hipEventDestroy(ev)
        self.events = []


# A timed kernel launch with default events cost the step about 7 us
# (measured on lmhead128k: 692 us per step without events, 699 us with a
# pair on every ce_fwd_grad, whether recorded by torch around the call or
# attached to the launch): the timestamps were taken after a system-scope
# release at the kernel's end, which HipEvents.FLAGS now skips.
# The timed loop attaches a pair to every EVENT_EVERY-th step,
# from the fourth on: by then the host is ahead of the GPU, so the slower
# host path of an armed launch does not leave the GPU idle; and never to
# the last step, whose event completion would otherwise add its latency to
# the wall clock (measured on 2,097,152 x 10 fp32 rows, 20 steps: 40.3 us
# per step with pairs on steps 0, 5, 10 and 15, 38.7 us on 4, 9, 14 and 19,
# 37.1 us with none).
EVENT_EVERY = 5
EVENT_OFFSET = 3


def timed_step_indices(steps: int) -> list:
    """The timed steps whose ce_fwd_grad launch carries an event pair:
    EVENT_OFFSET, EVENT_OFFSET + EVENT_EVERY, ..., never the last of more
    than one step, and at least one."""
    last = steps - 1 if steps > 1 else steps
    idx = list(range(min(EVENT_OFFSET, max(last - 1, 0)), last, EVENT_EVERY))
    return idx or [0]


def time_steps(zd, td, grad, loss_rows, loss, ws, steps: int, warmup: int) -> dict:
    """W untimed steps, then K steps timed by the wall clock between two
    device synchronisations; a step is one ce_fwd_grad_loss call (the
    gradient and per-row losses, then their sum).  The ce_fwd_grad launches of the steps
    timed_step_indices(K) record a pair of HIP events at their kernel's own
    start and end (ce_debug_time_next_launch) on the stream they run on;
    those give the kernel's duration."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    hev = HipEvents()
    timed = timed_step_indices(steps)
    pairs = dict(zip(timed, hev.pairs(len(timed))))
    for _ in range(warmup):
        ce.fwd_grad_loss_into(zd, td, grad, loss_rows, loss, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        pr = pairs.get(i)
        if pr is not None:
            hev.arm(pr)
        ce.fwd_grad_loss_into(zd, td, grad, loss_rows, loss, ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [hev.ms(pairs[i]) for i in timed]
    # ce_reduce_loss alone, after the timed region, timed the same way
    rpairs = hev.pairs(20)
    for pr in rpairs:
        hev.arm(pr)
        ce.reduce_loss_into(loss_rows, loss, ws)
    torch.cuda.synchronize()
    red_ms = [hev.ms(pr) for pr in rpairs]
    hev.close()
    return {"ms_per_step": wall * 1e3 / steps, "fwd_ms": fwd_ms, "red_ms": red_ms,
            "timed_region_s": wall, "timed_steps": timed}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(z, t, dtype: str, C: int, in_bytes: int, budget_s: float) -> dict:
    """Time the fp64 oracle on the host: the first rows of the workload on
    one thread, sized so that run takes about budget_s / 2 seconds, then the
    same rows in row blocks on a pool of threads (numpy releases the GIL in
    its array arithmetic).  `value` is the pool's rate; the one-thread rate
    is reported beside it."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import ce as oracle_ce
    B = z.shape[0]
    rows = max(1, min(B, (1 << 20) // C))
    t0 = time.perf_counter()
    oracle_ce(z[:rows], t[:rows], dtype)
    dt = time.perf_counter() - t0
    rows = int(min(B, max(rows, rows * 0.5 * budget_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    oracle_ce(z[:rows], t[:rows], dtype)
    dt1 = time.perf_counter() - t0
    # at most 16 threads (the host share of a benchmark run), never more than the host has
    workers = max(1, min(16, os.cpu_count() or 1))
    step = max(1, min(rows, (1 << 22) // C))
    blocks = [(lo, min(rows, lo + step)) for lo in range(0, rows, step)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda lh: oracle_ce(z[lh[0]:lh[1]], t[lh[0]:lh[1]], dtype)[0].sum(), blocks))
    dtn = time.perf_counter() - t0
    nbytes = rows * C * 2 * in_bytes
    threads = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                               "MKL_NUM_THREADS", "NUMEXPR_NUM_THREADS")}
    try:
        from threadpoolctl import threadpool_info
        threads["blas_pools"] = [{"api": i.get("internal_api"), "num_threads": i.get("num_threads")}
                                 for i in threadpool_info()]
    except Exception:  # threadpoolctl absent: the environment settings alone
        pass
    return {"value": round(nbytes / dtn / 1e9, 4), "unit": "GB/s", "cores": workers,
            "thread_settings": threads,
            "kind": "oracle", "rows_per_s": round(rows / dtn, 2),
            "one_core": {"value": round(nbytes / dt1 / 1e9, 4), "rows_per_s": round(rows / dt1, 2)},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"first {rows} of {B} rows, fp64 numpy; {workers} threads over "
                      f"{len(blocks)} row blocks {dtn:.1f} s, one thread {dt1:.1f} s"}


def copy_calibration(zd, grad, reps: int = 20) -> dict:
    """The library's streaming copy (ce_stream_copy: the row-part kernel's
    memory pattern, no arithmetic) of the logits into the gradient buffer,
    the same bytes read and written as ce_fwd_grad: the achievable rate.
    The runtime's own device copy is timed beside it."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)
    src, dst = zd.view(-1).view(torch.uint8), grad.view(-1).view(torch.uint8)
    nbytes = 2 * src.numel()
    # timed as ce_fwd_grad is in the steps: events on the kernel's launch
    ms = _event_median_ms(lambda: ce.stream_copy(src, dst), stream, reps, armed=True)
    ms_rt = _event_median_ms(lambda: dst.copy_(src), stream, reps)
    return {"kernel": "ce_stream_copy (1024 threads x 8 slots of 16 B, non-temporal)",
            "ms": round(ms, 5), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2),
            "runtime_copy_GBps": round(nbytes / (ms_rt * 1e-3) / 1e9, 2)}


def backward_scale(zd, td, grad, loss_rows, reps: int = 20) -> dict:
    """The backward of the fused loss on the workload's gradient: the
    broadcast scale ce_scale_grad by a device scalar (0.5: every element
    read and written; 1: the no-op early exit), and the forward with the
    scale folded in (ce_fwd_grad_scaled)."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)
    half = torch.tensor([0.5], dtype=torch.float32, device=zd.device)
    one = torch.tensor([1.0], dtype=torch.float32, device=zd.device)

    def timed(fn):
        return _event_median_ms(fn, stream, reps)

    nbytes = 2 * grad.numel() * grad.element_size()
    ms_half = timed(lambda: ce.scale_grad_(grad, half))
    ms_one = timed(lambda: ce.scale_grad_(grad, one))
    ms_fused = timed(lambda: ce.fwd_grad_scaled_into(zd, td, grad, loss_rows, half))
    return {"scale_grad_ms": round(ms_half, 5),
            "scale_grad_GBps": round(nbytes / (ms_half * 1e-3) / 1e9, 2),
            "scale_grad_one_ms": round(ms_one, 5),
            "fwd_grad_scaled_ms": round(ms_fused, 5)}


def loss_only_and_in_place(zd, td, grad, loss_rows, reps: int = 20) -> dict:
    """ce_fwd_loss (logits read once, per-row losses written) and the
    gradient in place of the logits (on a copy of them; each call then
    reads the previous call's gradient, a valid input of the same size):
    ce_fwd_grad_ex with the in-place workspace, so that rows of several parts
    stay on path 4, and ce_fwd_grad, which has no workspace."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)

    def timed(fn):
        return _event_median_ms(fn, stream, reps)

    in_bytes = zd.numel() * zd.element_size()
    ms_loss = timed(lambda: ce.fwd_loss_into(zd, td, loss_rows))
    grad.copy_(zd)
    ws = torch.zeros(ce.fwd_inplace_workspace_bytes(zd.shape[0]), dtype=torch.uint8,
                     device=zd.device)
    ms_inpl = timed(lambda: ce.fwd_grad_ex_into(grad, td, grad, loss_rows, workspace=ws))
    ms_plain = timed(lambda: ce.fwd_grad_into(grad, td, grad, loss_rows))
    gbs_loss = (in_bytes + 8 * zd.shape[0]) / (ms_loss * 1e-3) / 1e9
    gbs_inpl = (2 * in_bytes + 8 * zd.shape[0]) / (ms_inpl * 1e-3) / 1e9
    gbs_plain = (2 * in_bytes + 8 * zd.shape[0]) / (ms_plain * 1e-3) / 1e9
    return {"loss_only_ms": round(ms_loss, 5), "loss_only_GBps": round(gbs_loss, 2),
            "loss_only_frac": round(gbs_loss / PEAK_HBM_GBS, 4),
            "in_place_ms": round(ms_inpl, 5), "in_place_GBps": round(gbs_inpl, 2),
            "in_place_frac": round(gbs_inpl / PEAK_HBM_GBS, 4),
            "in_place_no_workspace_frac": round(gbs_plain / PEAK_HBM_GBS, 4)}


def _event_median_ms(fn, stream, reps: int, warm: int = 10, armed: bool = False) -> float:
    """Median time of fn over reps calls, each between a pair of HipEvents
    (no system fence, as in the timed steps): recorded on the stream around
    the call, or with armed attached to the call's first library launch
    (the kernel's own start and end, as for ce_fwd_grad in the timed
    steps)."""
    import torch
    hev = HipEvents()
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    pairs = hev.pairs(reps)
    handle = stream.cuda_stream
    for a, b in pairs:
        if armed:
            hev.arm((a, b))
            fn()
        else:
            hev.record(a, handle)
            fn()
            hev.record(b, handle)
    torch.cuda.synchronize()
    ms = statistics.median([hev.ms(pr) for pr in pairs])
    hev.close()
    return ms


GATE_FRAC = 0.75   # the LM-head workloads' bar: 75 % of peak HBM bandwidth
GATED = ("lmhead128k", "lmhead50k")


def gate(name: str, value: float, achieved: float, copy_gbs: float):
    """Whether a gated workload meets the 75 % bar, by the step (value) and
    by the kernel's own time (roofline.achieved), and by how many points of
    peak it misses; the copy of the same bytes shows how much room the
    memory system leaves.  None for workloads without the bar."""
    if name not in GATED:
        return None
    step, kern, copy = value / PEAK_HBM_GBS, achieved / PEAK_HBM_GBS, copy_gbs / PEAK_HBM_GBS
    return {"bar_frac": GATE_FRAC, "step_frac": round(step, 4), "kernel_frac": round(kern, 4),
            "met": bool(step >= GATE_FRAC and kern >= GATE_FRAC),
            "gap_points": round(100 * max(0.0, GATE_FRAC - min(step, kern)), 2),
            "copy_frac": round(copy, 4)}


def _rate(nbytes: int, ms: float) -> dict:
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 5), "GBps": round(gbs, 2), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "bytes": nbytes}


def graph_step(zd, td, grad, loss_rows, loss, ws, steps: int = 100) -> dict:
    """The step (ce_fwd_grad + ce_reduce_loss) captured once in a HIP graph
    and replayed: the per-step time without per-launch host overhead.  The
    replays are timed over `steps` back-to-back replays after 20 untimed
    ones."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ce.fwd_grad_into(zd, td, grad, loss_rows)
        ce.reduce_loss_into(loss_rows, loss, ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ce.fwd_grad_into(zd, td, grad, loss_rows)
        ce.reduce_loss_into(loss_rows, loss, ws)
    for _ in range(20):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    B, C = zd.shape
    return {**_rate(B * C * 2 * zd.element_size(), ms), "replays": steps}


def cold_fwd_grad(zd, td, grad, loss_rows, reps: int = 20) -> dict:
    """ce_fwd_grad with the 256 MB MALL (last-level cache) flushed before each
    call: 1 GiB of a scratch buffer is written between the calls, outside
    the timed events.  For the LM-head workloads (2 GB and 0.8 GB of logits)
    the cache cannot hold the inputs anyway; for small workloads the warm
    steady state of the timed steps can be served partly from it."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=zd.device)
    hev = HipEvents()
    pairs = hev.pairs(reps)
    for _ in range(3):
        ce.fwd_grad_into(zd, td, grad, loss_rows)
    for pr in pairs:
        scratch.fill_(1)
        hev.arm(pr)
        ce.fwd_grad_into(zd, td, grad, loss_rows)
    torch.cuda.synchronize()
    del scratch
    ms = statistics.median([hev.ms(pr) for pr in pairs])
    hev.close()
    B, C = zd.shape
    return _rate(B * C * 2 * zd.element_size() + 8 * B, ms)


def input_variants(zd, td, loss_rows, reps: int = 20) -> dict:
    """ce_fwd_grad on the workload's shape with fp16 logits, with logits and
    gradient rows at a padded stride (C + 64 elements) through
    ce_fwd_grad_ex, and with a quarter of the rows ignored (ignore_index,
    the count of kept rows on the device).  Same algorithmic bytes as the
    headline call (plus 4 B per row of targets for the count)."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)
    B, C = zd.shape
    out = {}
    zh = zd.to(torch.float16)
    gh = torch.empty_like(zh)
    ms = _event_median_ms(lambda: ce.fwd_grad_into(zh, td, gh, loss_rows), stream, reps)
    out["f16"] = _rate(B * C * 4 + 8 * B, ms)
    del zh, gh
    es = zd.element_size()
    wz = torch.empty((B, C + 64), dtype=zd.dtype, device=zd.device)
    wz[:, :C].copy_(zd)
    wg = torch.empty_like(wz)
    zv, gv = wz[:, :C], wg[:, :C]
    ms = _event_median_ms(lambda: ce.fwd_grad_ex_into(zv, td, gv, loss_rows), stream, reps)
    out["row_stride"] = {**_rate(B * C * 2 * es + 8 * B, ms), "ld": C + 64}
    del wz, wg, zv, gv
    gen = torch.Generator(device=zd.device).manual_seed(1)
    ti = torch.where(torch.rand(B, generator=gen, device=zd.device) < 0.25,
                     torch.full_like(td, -100), td)
    g = torch.empty_like(zd)
    ws = torch.empty(4, dtype=torch.uint8, device=zd.device)
    ms = _event_median_ms(lambda: ce.fwd_grad_ex_into(zd, ti, g, loss_rows, ignore_index=-100,
                                                      workspace=ws), stream, reps)
    out["ignore_index"] = {**_rate(B * C * 2 * es + 12 * B, ms), "ignored": 0.25}
    return out


def softmax_and_shards(zd, td, grad, loss_rows, reps: int = 20, nshards: int = 8,
                       attention: bool = False) -> dict:
    """The row-wise softmax forward (y and the log-sum-exp) and backward on
    the workload's shape, and the cross-entropy of its vocabulary cut into
    nshards column shards: one shard's record pass (ce_shard_stats) and
    gradient pass (ce_shard_grad, from the records of all shards).  Bytes
    counted: every array element read or written once, plus the per-row
    values.  Each call is one kernel, timed by HIP events at that kernel's
    own start and end (as ce_fwd_grad in the timed steps), so the 40-100 us
    shard kernels are not charged the host's call between two markers."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream(zd.device)
    B, C = zd.shape
    es = zd.element_size()
    out = {}
    ms = _event_median_ms(lambda: ce.softmax_fwd_into(zd, grad, loss_rows), stream, reps,
                          armed=True)
    out["softmax_fwd"] = _rate(2 * B * C * es + 4 * B, ms)
    y = grad.clone()          # a softmax output as y; the logits serve as dy
    dx = torch.empty_like(zd)
    ms = _event_median_ms(lambda: ce.softmax_bwd_into(y, zd, dx), stream, reps, armed=True)
    out["softmax_bwd"] = _rate(3 * B * C * es, ms)
    del y, dx
    edges = [C * k // nshards for k in range(nshards + 1)]
    shards = [zd[:, a:b].contiguous() for a, b in zip(edges[:-1], edges[1:])]
    recs = torch.stack([ce.shard_stats(s, td, a) for s, a in zip(shards, edges[:-1])])
    s0 = shards[0]
    g0 = torch.empty_like(s0)
    Cs = s0.shape[1]
    ms = _event_median_ms(lambda: ce.shard_stats_into(s0, td, 0, recs[0]), stream, reps,
                          armed=True)
    out["shard_stats"] = _rate(B * Cs * es + 4 * B + 16 * B, ms)
    ms = _event_median_ms(lambda: ce.shard_grad_into(s0, td, 0, C, recs, g0, loss_rows),
                          stream, reps, armed=True)
    out["shard_grad"] = _rate(2 * B * Cs * es + 4 * B + 16 * nshards * B + 4 * B, ms)
    out["shard"] = {"shards": nshards, "columns": Cs}
    del shards, recs, g0
    if not attention:
        return out
    # attention-shaped rows (the softmax of scaled dot products: batch 4 x
    # 32 heads x 2048 queries, 2048 keys), bf16, values from torch's device
    # generator (timing only)
    Ba, Ca = 4 * 32 * 2048, 2048
    gen = torch.Generator(device=zd.device).manual_seed(0)
    xa = torch.randn((Ba, Ca), generator=gen, device=zd.device).mul_(3).to(torch.bfloat16)
    ya = torch.empty_like(xa)
    ms = _event_median_ms(lambda: ce.softmax_fwd_into(xa, ya), stream, reps, armed=True)
    att = {"rows": Ba, "columns": Ca, "dtype": "bf16",
           "softmax_fwd": _rate(2 * Ba * Ca * 2, ms)}
    dya = torch.randn((Ba, Ca), generator=gen, device=zd.device).to(torch.bfloat16)
    dxa = torch.empty_like(xa)
    ms = _event_median_ms(lambda: ce.softmax_bwd_into(ya, dya, dxa), stream, reps, armed=True)
    att["softmax_bwd"] = _rate(3 * Ba * Ca * 2, ms)
    out["attention_rows"] = att
    return out


def second_workload(name: str, steps: int, warmup: int) -> dict:
    """The other gated workload of the default run (the 4096 x 50257 fp32
    LM head beside the 8192 x 128256 bf16 headline): the same step, W and
    K, timed the same way in the same process, with the library's copy of
    its own bytes beside it."""
    import numpy as np
    import torch
    import softmax_cross_entropy_ce_amd as ce
    import synth
    w = synth.WORKLOADS[name]
    B, C, es = w.B, w.C, w.in_bytes
    dev = torch.device("cuda:0")
    z, t = synth.make_workload(name)
    if w.dtype == "f32":
        zd = torch.from_numpy(z).to(dev)
    else:
        zd = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
    td = torch.from_numpy(t).to(dev)
    grad = torch.empty_like(zd)
    loss_rows = torch.empty(B, dtype=torch.float32, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    ws = torch.empty(max(ce.reduce_workspace_bytes(B), 1), dtype=torch.uint8, device=dev)
    res = time_steps(zd, td, grad, loss_rows, loss, ws, steps, warmup)
    metric_bytes = B * C * 2 * es
    fwd_bytes = metric_bytes + 8 * B
    fwd_avg = statistics.fmean(res["fwd_ms"])
    value = metric_bytes / (res["ms_per_step"] * 1e-3) / 1e9
    achieved = fwd_bytes / (fwd_avg * 1e-3) / 1e9
    cal = copy_calibration(zd, grad)
    out = {"config": {**w.describe(), "path": ce.PATH_NAMES[ce.select_path(C, ce.F32 if w.dtype == "f32" else ce.BF16)]},
           "steps": steps, "warmup": warmup,
           "value": round(value, 2), "unit": "GB/s", "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
           "ms_per_step": round(res["ms_per_step"], 5),
           "rows_per_s": round(B / (res["ms_per_step"] * 1e-3), 1),
           "fwd_grad_ms": {"mean": round(fwd_avg, 5),
                           "median": round(statistics.median(res["fwd_ms"]), 5),
                           "min": round(min(res["fwd_ms"]), 5), "max": round(max(res["fwd_ms"]), 5)},
           "roofline": {"bound": "hbm", "kernel": "ce_fwd_grad", "achieved": round(achieved, 2),
                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes_per_launch": fwd_bytes, "traffic": traffic_for(name)},
           "copy_calibration": {**cal, "fwd_grad_pct_of_copy": round(100 * achieved / cal["GBps"], 2)},
           "gate": gate(name, value, achieved, cal["GBps"])}
    del zd, td, grad, loss_rows, ws
    torch.cuda.empty_cache()
    return out


def run_copy(args) -> None:
    """Plain device-to-device copy of a known size (counter calibration)."""
    import torch
    n = args.copy_mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    y = torch.empty_like(x)
    for _ in range(args.warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n,
                      "GBps": round(2 * n / dt / 1e9, 1), "ms": round(dt * 1e3, 4)}), flush=True)


# even lengths at each path's boundaries and typical vocabularies, and odd
# lengths (no whole 16-byte vectors per row) from 33 to 4095
SWEEP_C = (33, 64, 81, 101, 255, 256, 300, 301, 512, 1000, 1001, 2047, 2048, 3000, 4095, 4096,
           8192, 12000, 16032, 32000, 50257, 65536, 128256, 200000)


def run_sweep(args) -> None:
    """Rates across row lengths: for each dtype and C, rows filling 1 GiB of
    logits; ce_stream_copy of the logits' bytes into the gradient buffer
    (the achievable rate), ce_fwd_grad, ce_fwd_loss, the softmax forward and
    backward, each the median of HIP-event times over 30 calls after 40.
    One JSON line per shape; rates in GB/s of the bytes each call must move
    (copy and fwd_grad 2 arrays, the loss 1, softmax forward 2, backward 3)."""
    import torch
    import softmax_cross_entropy_ce_amd as ce
    stream = torch.cuda.current_stream()
    for dt in ("bf16", "f32"):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        es = 4 if dt == "f32" else 2
        for C in (args.sweep_c or SWEEP_C):
            B = max(16, (1 << 30) // (C * es) // 16 * 16)
            gen = torch.Generator(device="cuda:0").manual_seed(C)
            z = (torch.randn(B, C, device="cuda:0", generator=gen) * 3).to(tdt)
            t = torch.randint(0, C, (B,), device="cuda:0", dtype=torch.int32, generator=gen)
            g, lr = torch.empty_like(z), torch.empty(B, device="cuda:0")
            dy = torch.randn(B, C, device="cuda:0", generator=gen).to(tdt)
            dx = torch.empty_like(z)
            n = B * C * es
            src, dst = z.view(-1).view(torch.uint8), g.view(-1).view(torch.uint8)

            def rate(fn, arrays):
                ms = _event_median_ms(fn, stream, 30, warm=40)
                return {"us": round(ms * 1e3, 1), "GBps": round(arrays * n / (ms * 1e-3) / 1e9, 1)}

            rec = {"mode": "sweep", "dtype": dt, "C": C, "B": B,
                   "path": ce.PATH_NAMES[ce.select_path(C, ce.F32 if dt == "f32" else ce.BF16)],
                   "copy": rate(lambda: ce.stream_copy(src, dst), 2),
                   "fwd_grad": rate(lambda: ce.fwd_grad_into(z, t, g, lr), 2),
                   "fwd_loss": rate(lambda: ce.fwd_loss_into(z, t, lr), 1),
                   "softmax_fwd": rate(lambda: ce.softmax_fwd_into(z, g, lr), 2),
                   "softmax_bwd": rate(lambda: ce.softmax_bwd_into(g, dy, dx), 3)}
            rec["fwd_grad_pct_of_copy"] = round(100 * rec["fwd_grad"]["GBps"] / rec["copy"]["GBps"], 1)
            print(json.dumps(rec), flush=True)
            del z, t, g, lr, dy, dx, src, dst
            torch.cuda.empty_cache()


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks take about 40 back-to-back lmhead128k steps (~30 ms)
    # to settle after idle: a step runs fast, then up to 30 % slower, then
    # settles.  The default warm-up covers that; the timed steps are the
    # steady state.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="lmhead128k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attention", action="store_true",
                    help="also time the row softmax on attention-shaped rows (262144 x 2048 bf16)")
    ap.add_argument("--no-second", action="store_true",
                    help="skip the second gated workload (lmhead50k) of the default run")
    ap.add_argument("--mode", choices=["ce", "copy", "sweep"], default="ce")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--sweep-c", type=lambda v: tuple(int(x) for x in v.split(",")), default=None,
                    help="row lengths for --mode sweep, comma-separated (default: the built-in list)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path is data-parallel over rows and each "
              "GPU would run the same kernel on its own rows; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        run_copy(args)
        return
    if args.mode == "sweep":
        run_sweep(args)
        return

    import numpy as np
    import torch

    import softmax_cross_entropy_ce_amd as ce
    import synth

    w = synth.WORKLOADS[args.workload]
    B, C, es = w.B, w.C, w.in_bytes
    dev = torch.device("cuda:0")
    log(f"[bench] {ce.version()} workload {w.name} B={B} C={C} {w.dtype}; generating inputs")
    t0 = time.perf_counter()
    z, t = synth.make_workload(w.name)
    log(f"[bench] inputs drawn in {time.perf_counter() - t0:.1f} s; uploading")
    if w.dtype == "f32":
        zd = torch.from_numpy(z).to(dev)
    else:
        zd = torch.from_numpy(z.view(np.int16)).to(dev).view(torch.bfloat16)
    td = torch.from_numpy(t).to(dev)
    grad = torch.empty_like(zd)
    loss_rows = torch.empty(B, dtype=torch.float32, device=dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    ws_bytes = ce.reduce_workspace_bytes(B)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    path = ce.select_path(C, ce.F32 if w.dtype == "f32" else ce.BF16)

    log(f"[bench] path {ce.PATH_NAMES[path]}; {args.warmup} warm-up steps, timing {args.steps}")
    res = time_steps(zd, td, grad, loss_rows, loss, ws, args.steps, args.warmup)
    fwd_ms, red_ms, ms_per_step = res["fwd_ms"], res["red_ms"], res["ms_per_step"]
    log(f"[bench] loss {loss.item():.6f}; fwd_grad median {statistics.median(fwd_ms):.4f} ms, "
        f"reduce median {statistics.median(red_ms):.4f} ms, step {ms_per_step:.4f} ms")

    metric_bytes = B * C * 2 * es                # logits read + gradient written
    fwd_bytes = metric_bytes + 8 * B             # + targets read + per-row loss written
    value = metric_bytes / (ms_per_step * 1e-3) / 1e9
    fwd_avg = statistics.fmean(fwd_ms)
    achieved = fwd_bytes / (fwd_avg * 1e-3) / 1e9
    cal = copy_calibration(zd, grad)
    bwd = backward_scale(zd, td, grad, loss_rows)
    variants = loss_only_and_in_place(zd, td, grad, loss_rows)
    sm = softmax_and_shards(zd, td, grad, loss_rows, attention=args.attention)
    cold = cold_fwd_grad(zd, td, grad, loss_rows)
    var = input_variants(zd, td, loss_rows)
    graph = graph_step(zd, td, grad, loss_rows, loss, ws)
    cal["fwd_grad_pct_of_copy"] = round(100 * achieved / cal["GBps"], 2)
    rec = {
        "metric": "fused CE fwd+grad: achieved HBM GB/s (% of peak) and rows/sec at C=128256 bf16"
                  if w.name == "lmhead128k" else f"fused CE fwd+grad achieved HBM GB/s ({w.name})",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accum_dtype": "f32",
        "data": "synthetic",
        "config": {**w.describe(), "path": ce.PATH_NAMES[path]},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "rows_per_s": round(B / (ms_per_step * 1e-3), 1),
        "fwd_grad_ms": {"mean": round(fwd_avg, 5), "median": round(statistics.median(fwd_ms), 5),
                        "min": round(min(fwd_ms), 5), "max": round(max(fwd_ms), 5),
                        "timed_steps": res["timed_steps"],
                        "how": "HIP events attached to the kernel's launch "
                               f"(every {EVENT_EVERY}th timed step from step {EVENT_OFFSET}, "
                               "never the last)"},
        "timed_region_s": round(res["timed_region_s"], 6),
        "reduce_ms": {"mean": round(statistics.fmean(red_ms), 5),
                      "median": round(statistics.median(red_ms), 5)},
        "roofline": {"bound": "hbm", "kernel": "ce_fwd_grad", "achieved": round(achieved, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes_per_launch": fwd_bytes,
                     "traffic": traffic_for(w.name)},
        "copy_calibration": cal,
        "gate": gate(w.name, value, achieved, cal["GBps"]),
        "backward_scale": bwd,
        "loss_only_and_in_place": variants,
        "softmax_and_shards": sm,
        "fwd_grad_cold": cold,
        "input_variants": var,
        "graph_step": graph,
    }
    if w.name == "lmhead128k" and not args.no_second:
        log("[bench] second gated workload lmhead50k (4096 x 50257 fp32)")
        rec["lmhead50k"] = second_workload("lmhead50k", args.steps, args.warmup)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for about {args.cpu_seconds:.0f} s")
        rec["cpu_baseline"] = cpu_baseline(z, t, w.dtype, C, es, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
