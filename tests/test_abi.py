"""The C-ABI library on the CPU: it loads, exports every function that
include/ce.h declares, and rejects invalid arguments with the documented
status before any HIP call (so none of these calls reaches a device)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import softmax_cross_entropy_ce_amd as ce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce.h")

OK, NULL, SHAPE, DTYPE, WORKSPACE, LAUNCH, ALIGN, ALIAS, PATH = 0, -1, -2, -3, -4, -5, -6, -7, -8

# Fake, never-dereferenced device addresses: every call below fails
# validation first.
Z = 0x10000000
G = 0x20000000
T = 0x30000000
L = 0x40000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ce_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L_ = ce.lib()
    names = declared_functions()
    assert names == sorted(["ce_fwd_grad", "ce_reduce_workspace_bytes", "ce_reduce_loss",
                            "ce_status_string", "ce_version", "ce_select_path",
                            "ce_debug_force_path", "ce_debug_part_polls",
                            "ce_debug_part_counter", "ce_stream_copy",
                            "ce_fwd_grad_scaled", "ce_scale_grad", "ce_fwd_loss",
                            "ce_softmax_fwd", "ce_softmax_bwd", "ce_shard_stats",
                            "ce_shard_grad", "ce_fwd_grad_ex", "ce_fwd_workspace_bytes",
                            "ce_reduce_loss_noalloc", "ce_debug_time_next_launch",
                            "ce_fwd_inplace_workspace_bytes", "ce_fwd_grad_loss"])
    for n in names:
        assert hasattr(L_, n), n


def test_version_and_status_strings():
    assert "gfx950" in ce.version()
    for s in (OK, NULL, SHAPE, DTYPE, WORKSPACE, LAUNCH, ALIGN, ALIAS, PATH):
        assert ce.status_string(s) and ce.status_string(s) != "unknown status"
    assert ce.status_string(-99) == "unknown status"


def fwd(z=Z, t=T, B=8, C=10, dtype=0, g=G, l=L):
    return ce.lib().ce_fwd_grad(z, t, B, C, dtype, g, l, None)


def test_fwd_grad_null_pointers():
    assert fwd(z=None) == NULL
    assert fwd(t=None) == NULL
    assert fwd(g=None) == NULL
    assert fwd(l=None) == NULL


def test_fwd_grad_shapes():
    assert fwd(B=0) == SHAPE
    assert fwd(B=-3) == SHAPE
    assert fwd(C=0) == SHAPE
    assert fwd(C=-1) == SHAPE
    assert fwd(C=(1 << 28) + 1) == SHAPE
    assert fwd(B=1 << 31) == SHAPE


def test_fwd_grad_dtype():
    assert fwd(dtype=3) == DTYPE
    assert fwd(dtype=-1) == DTYPE


def test_fwd_grad_alignment():
    assert fwd(z=Z + 2, dtype=0) == ALIGN          # fp32 needs 4-byte alignment
    assert fwd(z=Z + 1, dtype=1) == ALIGN          # bf16 needs 2-byte alignment
    assert fwd(z=Z + 4, g=G, dtype=0) == ALIGN     # logits and grad 16-byte congruent
    assert fwd(t=T + 2) == ALIGN
    assert fwd(l=L + 1) == ALIGN


def test_fwd_grad_alias():
    # a partial overlap of grad and logits is refused (grad == logits is the
    # in-place call, accepted)
    assert fwd(z=Z, g=Z + 16, B=8, C=10) == ALIAS
    assert fwd(z=Z + 16, g=Z, B=8, C=10) == ALIAS


def test_reduce_workspace_sizes():
    f = ce.reduce_workspace_bytes
    assert f(0) == 0 and f(-5) == 0
    # up to 16384 rows one workgroup sums them in a single launch
    assert f(1) == 0 and f(8) == 0 and f(2048) == 0 and f(16384) == 0
    assert f(16385) == 9 * 4                                # chunks of 2048 rows
    # 2M rows: 1024 first-level partial sums of one 2048-row round each
    assert f(2_097_152) == 1024 * 4
    # chunks are whole rounds of 2048 rows: 3M rows take chunks of 4096
    assert f(3_000_001) == 733 * 4
    # past 2^39 rows a chunk's bytes would not fit a buffer resource
    assert f(1 << 39) == 1024 * 4 and f((1 << 39) + 1) == 0


def red(x=L, B=8, out=G, ws=None, wsb=0):
    return ce.lib().ce_reduce_loss(x, B, out, ws, wsb, None)


def test_reduce_loss_validation():
    assert red(x=None) == NULL
    assert red(out=None) == NULL
    assert red(B=0) == SHAPE
    assert red(B=(1 << 39) + 1) == SHAPE
    assert red(x=L + 2) == ALIGN
    assert red(B=1 << 20) == WORKSPACE                      # workspace needed, none given
    need = ce.reduce_workspace_bytes(1 << 20)
    assert red(B=1 << 20, ws=T, wsb=need - 1) == WORKSPACE  # too small
    assert red(B=1 << 20, ws=T + 2, wsb=need) == ALIGN


def test_reduce_loss_noalloc_validation():
    """Refusals happen on the host, before any HIP call (so they run here
    without a GPU): NULL pointers, B outside [1, CE_NOALLOC_MAX_ROWS],
    misaligned pointers."""
    f = ce.lib().ce_reduce_loss_noalloc
    assert f(None, 8, G, None) == NULL
    assert f(L, 8, None, None) == NULL
    assert f(L, 0, G, None) == SHAPE
    assert f(L, -1, G, None) == SHAPE
    assert f(L, (1 << 31), G, None) == SHAPE
    assert f(L + 2, 8, G, None) == ALIGN
    assert f(L, 8, G + 1, None) == ALIGN


@pytest.mark.parametrize("name,C,dtype,path", [
    ("tiny", 10, 0, 1),
    ("classifier", 1000, 0, 5),
    ("skinny", 10, 0, 1),
    ("lmhead50k", 50257, 0, 4),
    ("lmhead128k", 128256, 1, 4),
    ("four-parts-bf16", 200_000, 1, 4),
    ("four-parts-f32", 100_000, 0, 4),
    ("short-limit", 256, 0, 1),
    ("just-over-short", 258, 1, 5),
    # path 5 up to 8 KB of 16-bit or 4 KB of fp32 elements, where the row
    # allows 16-, 8- or 4-byte vectors (16-bit rows of odd length do not:
    # those stay on path 2 up to 256 16-byte vectors and take one row part
    # above); longer rows go to the row parts
    ("wave-limit-f32", 1024, 0, 5),
    ("over-wave-f32", 1025, 0, 4),
    ("wave-limit-bf16", 4096, 1, 5),
    ("over-wave-bf16", 4100, 1, 4),
    ("wave-4-byte-vectors", 1023, 0, 5),
    ("odd-bf16", 257, 1, 2),
    ("odd-bf16-resident-limit", 2039, 1, 2),
    ("odd-bf16-one-part", 2041, 1, 4),
    ("odd-bf16-limit", 4095, 1, 4),
    ("over-odd-bf16-limit", 4097, 1, 4),
    # four parts of 12 x 1024 vectors (16-bit) or 8 x 1024 (fp32), then
    # eight parts of 8 x 1024 vectors: aligned body of at most 65536 vectors
    ("four-parts-limit-bf16", 393_216, 1, 4),
    ("eight-parts-bf16", 393_224, 1, 4),
    ("parts-limit-bf16", 524_288, 1, 4),
    ("over-parts-bf16", 524_296, 1, 3),
    ("four-parts-limit-f32", 131_072, 0, 4),
    ("eight-parts-f32", 131_076, 0, 4),
    ("parts-limit-f32", 262_144, 0, 4),
    ("over-parts-f32", 262_148, 0, 3),
])
def test_path_selection(name, C, dtype, path):
    assert ce.select_path(C, dtype) == path


def test_force_path_round_trip():
    prev = ce.force_path(3)
    try:
        assert ce.select_path(10, 0) == 3
        assert ce.force_path(1) == 3
        # a row too long for the short path is refused, before any launch
        assert fwd(C=1000) == PATH
    finally:
        ce.force_path(prev)
    assert ce.select_path(10, 0) == 1
    assert ce.lib().ce_debug_force_path(7) == PATH
    assert ce.lib().ce_debug_force_path(6) == PATH
    prev = ce.force_path(4)
    try:
        assert ce.select_path(10, 1) == 4
    finally:
        ce.force_path(prev)


def test_part_hooks_round_trip():
    prev = ce.part_polls(0)
    try:
        assert ce.part_polls(5) == 0
    finally:
        ce.part_polls(prev)
    assert prev == 64
    assert ce.lib().ce_debug_part_polls(-1) == PATH
    ce.part_counter(None)


def test_stream_copy_validation():
    cp = ce.lib().ce_stream_copy
    assert cp(None, G, 16, None) == NULL
    assert cp(Z, None, 16, None) == NULL
    assert cp(Z, G, 0, None) == SHAPE
    assert cp(Z, G, 24, None) == SHAPE      # not a multiple of 16
    assert cp(Z + 8, G, 16, None) == ALIGN
    assert cp(Z, Z + 16, 64, None) == ALIAS


def test_fwd_grad_scaled_validation():
    f = ce.lib().ce_fwd_grad_scaled
    assert f(Z, T, 8, 10, 0, G, L, None, None) == NULL          # grad_scale required
    assert f(Z, T, 8, 10, 0, G, L, L + 2, None) == ALIGN
    assert f(None, T, 8, 10, 0, G, L, L, None) == NULL
    assert f(Z, T, 0, 10, 0, G, L, L, None) == SHAPE
    assert f(Z, T, 8, 10, 5, G, L, L, None) == DTYPE


def test_scale_grad_validation():
    f = ce.lib().ce_scale_grad
    assert f(None, 16, 0, L, None) == NULL
    assert f(G, 16, 0, None, None) == NULL
    assert f(G, 0, 0, L, None) == SHAPE
    assert f(G, 16, 7, L, None) == DTYPE
    assert f(G + 2, 16, 0, L, None) == ALIGN      # fp32 grad 2-byte aligned
    assert f(G, 16, 0, L + 1, None) == ALIGN
    assert f(G, 16, 0, G + 8, None) == ALIAS      # scale inside grad


def test_fwd_loss_validation():
    f = ce.lib().ce_fwd_loss
    assert f(None, T, 8, 10, 0, L, None) == NULL
    assert f(Z, None, 8, 10, 0, L, None) == NULL
    assert f(Z, T, 8, 10, 0, None, None) == NULL
    assert f(Z, T, 0, 10, 0, L, None) == SHAPE
    assert f(Z, T, 8, 0, 0, L, None) == SHAPE
    assert f(Z, T, 8, 10, 9, L, None) == DTYPE
    assert f(Z + 2, T, 8, 10, 0, L, None) == ALIGN
    prev = ce.force_path(4)
    try:
        assert f(Z, T, 8, 10, 0, L, None) == PATH   # no row parts for the loss alone
    finally:
        ce.force_path(prev)


def test_in_place_two_part_rows_refuse_forced_parts():
    prev = ce.force_path(4)
    try:
        assert fwd(z=Z, g=Z, B=8, C=128256, dtype=1) == PATH
    finally:
        ce.force_path(prev)


def smf(x=Z, B=8, C=10, dtype=0, y=G, lse=L):
    return ce.lib().ce_softmax_fwd(x, B, C, dtype, y, lse, None)


def test_softmax_fwd_validation():
    assert smf(x=None) == NULL
    assert smf(y=None) == NULL
    assert smf(dtype=5) == DTYPE
    assert smf(B=0) == SHAPE and smf(C=0) == SHAPE and smf(C=(1 << 28) + 1) == SHAPE
    assert smf(x=Z + 2) == ALIGN
    assert smf(y=G + 4) == ALIGN                 # x and y 16-byte congruent
    assert smf(lse=L + 2) == ALIGN
    assert smf(x=Z, y=Z + 16) == ALIAS           # partial overlap
    prev = ce.force_path(4)
    try:
        assert smf(x=Z, y=Z, C=128256, dtype=1) == PATH   # in place, two-part rows
    finally:
        ce.force_path(prev)


def smb(y=Z, dy=T, B=8, C=10, dtype=0, dx=G):
    return ce.lib().ce_softmax_bwd(y, dy, B, C, dtype, dx, None)


def test_softmax_bwd_validation():
    assert smb(y=None) == NULL and smb(dy=None) == NULL and smb(dx=None) == NULL
    assert smb(dtype=3) == DTYPE
    assert smb(B=0) == SHAPE and smb(C=-1) == SHAPE and smb(B=1 << 31) == SHAPE
    assert smb(y=Z + 2) == ALIGN
    assert smb(dy=T + 4) == ALIGN                # y and dy 16-byte congruent
    assert smb(dx=G + 8) == ALIGN                # y and dx 16-byte congruent
    assert smb(y=Z, dx=Z + 16) == ALIAS          # dx partly over y
    assert smb(dy=T, dx=T - 16) == ALIAS         # dx partly over dy
    prev = ce.force_path(4)
    try:
        assert smb() == PATH                     # no row parts for the backward
        ce.force_path(1)
        assert smb(C=300) == PATH                # short path: C <= 256
    finally:
        ce.force_path(prev)


def sst(z=Z, t=T, B=8, C=10, col0=0, dtype=0, rec=L):
    return ce.lib().ce_shard_stats(z, t, B, C, col0, dtype, rec, None)


def test_shard_stats_validation():
    assert sst(z=None) == NULL and sst(t=None) == NULL and sst(rec=None) == NULL
    assert sst(dtype=3) == DTYPE
    assert sst(B=0) == SHAPE and sst(col0=-1) == SHAPE and sst(col0=1 << 31) == SHAPE
    assert sst(rec=L + 4) == ALIGN               # records are 16-byte aligned
    assert sst(t=T + 2) == ALIGN
    prev = ce.force_path(4)
    try:
        assert sst() == PATH                     # records need no row parts
    finally:
        ce.force_path(prev)


def sgr(z=Z, t=T, B=8, C=10, col0=0, ctot=10, dtype=0, rec=L, n=1, g=G, lo=None, sc=None):
    return ce.lib().ce_shard_grad(z, t, B, C, col0, ctot, dtype, rec, n, g, lo, sc, None)


def test_shard_grad_validation():
    assert sgr(z=None) == NULL and sgr(t=None) == NULL
    assert sgr(rec=None) == NULL and sgr(g=None) == NULL
    assert sgr(dtype=4) == DTYPE
    assert sgr(B=0) == SHAPE and sgr(C=0) == SHAPE
    assert sgr(n=0) == SHAPE and sgr(n=1025) == SHAPE
    assert sgr(col0=-1) == SHAPE
    assert sgr(col0=5, ctot=14) == SHAPE         # col0 + C beyond the row
    assert sgr(ctot=9) == SHAPE                  # the row shorter than the shard
    assert sgr(ctot=1 << 31) == SHAPE
    assert sgr(rec=L + 8) == ALIGN
    assert sgr(g=G + 4) == ALIGN
    assert sgr(lo=L + 2) == ALIGN and sgr(sc=T + 1) == ALIGN
    assert sgr(z=Z, g=Z + 16) == ALIAS           # grad partly over the logits
    assert sgr(g=L - 64) == ALIAS                # grad over the records


NO_IGNORE = -(1 << 31)
WS = 0x50000000


def fex(z=Z, ldz=10, t=T, B=8, C=10, dtype=0, g=G, ldg=10, l=L, sc=None, ii=NO_IGNORE, ws=None,
        wsb=0):
    return ce.lib().ce_fwd_grad_ex(z, ldz, t, B, C, dtype, g, ldg, l, sc, ii, ws, wsb, None)


def test_fwd_workspace_bytes():
    assert ce.fwd_workspace_bytes() == 0 and ce.fwd_workspace_bytes(-100) == 4
    assert ce.fwd_workspace_bytes(0) == 4


def test_fwd_inplace_workspace_bytes():
    f = ce.fwd_inplace_workspace_bytes
    # 256 bytes (the ignore_index count in the first 4), then 18 64-bit
    # words a row
    assert f(1) == 256 + 144 and f(8192) == 256 + 144 * 8192
    assert f((1 << 31) - 1) == 256 + 144 * ((1 << 31) - 1)
    assert f(0) == 0 and f(-1) == 0 and f(1 << 31) == 0


def test_fwd_grad_ex_validation():
    assert fex(z=None) == NULL and fex(t=None) == NULL and fex(l=None) == NULL
    assert fex(dtype=3) == DTYPE
    assert fex(B=0) == SHAPE and fex(C=0) == SHAPE
    assert fex(ldz=9) == SHAPE                     # row stride below C
    assert fex(ldg=9) == SHAPE
    assert fex(ldz=12, ldg=10) == ALIGN            # rows 8 bytes apart modulo 16
    assert fex(g=G + 4) == ALIGN
    assert fex(sc=L + 2) == ALIGN
    assert fex(ii=-100) == WORKSPACE               # ignore_index needs the count's workspace
    assert fex(ii=-100, ws=WS, wsb=3) == WORKSPACE
    assert fex(ii=-100, ws=WS + 2, wsb=4) == ALIGN
    # grad overlapping logits with another stride, or partly
    assert fex(z=Z, g=Z + 16 * 4, ldz=14, ldg=10) == ALIAS
    assert fex(z=Z, g=Z, ldz=14, ldg=10) == ALIAS  # same base, other stride: not in place
    prev = ce.force_path(4)
    try:
        assert fex(g=None) == PATH                 # loss only: no row parts
        assert fex(z=Z, g=Z, ldz=128256, ldg=128256, C=128256, dtype=1) == PATH
    finally:
        ce.force_path(prev)


C_CLIENT = r"""
#include "ce.h"
#include <stdio.h>
/* A plain C client: every call below fails validation (or is host-only),
   so nothing reaches a device. */
int main(void) {
  if (ce_fwd_grad(0, 0, 8, 10, CE_F32, 0, 0, 0) != CE_ERR_NULL) return 1;
  if (ce_softmax_fwd(0, 8, 10, CE_F16, 0, 0, 0) != CE_ERR_NULL) return 2;
  if (ce_softmax_bwd(0, 0, 8, 10, CE_BF16, 0, 0) != CE_ERR_NULL) return 3;
  if (ce_shard_grad(0, 0, 8, 10, 0, 10, CE_F32, 0, 1, 0, 0, 0, 0) != CE_ERR_NULL) return 4;
  if (ce_fwd_workspace_bytes(CE_NO_IGNORE) != 0 || ce_fwd_workspace_bytes(-100) != 4) return 5;
  if (ce_reduce_workspace_bytes(16384) != 0) return 6;
  if (ce_select_path(128256, CE_BF16) != 4) return 7;
  printf("%s\n", ce_version());
  return 0;
}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++11")])
def test_header_builds_a_plain_client(tmp_path, compiler, std):
    """include/ce.h compiles as strict C99 (and as C++11) with every warning
    an error, and a client links against the library and runs."""
    import shutil
    import subprocess
    cc = shutil.which(compiler)
    if cc is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("client.c" if compiler == "gcc" else "client.cpp")
    src.write_text(C_CLIENT)
    libdir = os.path.dirname(ce._LIB_PATH)
    exe = tmp_path / "client"
    lang = ["-x", "c++"] if compiler == "g++" else []
    res = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror",
                          f"-I{os.path.join(ROOT, 'include')}", *lang, str(src), "-x", "none",
                          f"-L{libdir}", "-lce_mi355x", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr[-2000:])
    assert "gfx950" in run.stdout


def test_fwd_grad_loss_refuses_before_launch():
    """The whole-step call checks the reduction's arguments before it
    launches anything (fake device addresses: every call here is refused)."""
    f = ce.lib().ce_fwd_grad_loss
    S = L + 65536
    assert f(Z, T, 8, 10, 0, G, L, None, None, 0, None) == NULL           # no loss scalar
    assert f(Z, T, 8, 10, 0, G, L, S + 2, None, 0, None) == ALIGN         # misaligned scalar
    assert f(Z, T, 1 << 20, 10, 0, G, L, S, None, 0, None) == WORKSPACE   # reduction needs scratch
    need = ce.reduce_workspace_bytes(1 << 20)
    assert f(Z, T, 1 << 20, 10, 0, G, L, S, WS, need - 4, None) == WORKSPACE
    assert f(Z, T, 1 << 20, 10, 0, G, L, S, WS + 2, need, None) == ALIGN
    # then the forward's own checks
    assert f(Z, T, 0, 10, 0, G, L, S, None, 0, None) == SHAPE
    assert f(Z, T, 8, 10, 5, G, L, S, None, 0, None) == DTYPE
    assert f(Z, T, 8, 10, 0, None, L, S, None, 0, None) == NULL
