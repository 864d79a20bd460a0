"""The library's host code (argument validation, path and workspace
arithmetic) under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: both translation units are compiled with the sanitizers on their host
side only (the gfx950 code is built as usual), linked into a C++ client,
and the client drives every entry point with invalid and extreme arguments
(sizes up to INT64_MAX, strides that would overflow a span, misaligned and
overlapping pointers).  Every call must be refused before any HIP call, with
no sanitizer report.  The build takes about two and a half minutes; it
starts in the background right after collection (tests/conftest.py), and
is cached under tests/.san_build by a digest of the sources, so later runs
reuse it."""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "softmax_cross_entropy_ce_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
CACHE = os.path.join(ROOT, "tests", ".san_build")
ROCM = "/opt/rocm"

CLIENT = r"""
#include "ce.h"
#include <stdint.h>
#include <stdio.h>

static int fails = 0;
#define REFUSED(call)                                                        \
  do {                                                                       \
    int st_ = (call);                                                        \
    if (st_ >= 0) {                                                          \
      fprintf(stderr, "line %d: %s returned %d\n", __LINE__, #call, st_);    \
      ++fails;                                                               \
    }                                                                        \
  } while (0)
#define EQ(a, b)                                                             \
  do {                                                                       \
    if ((a) != (b)) {                                                        \
      fprintf(stderr, "line %d: %s != %s\n", __LINE__, #a, #b);              \
      ++fails;                                                               \
    }                                                                        \
  } while (0)

int main(void) {
  /* fake, never dereferenced device addresses (every call is refused) */
  char* Z = (char*)(uintptr_t)0x100000000ull;
  char* G = (char*)(uintptr_t)0x200000000ull;
  int32_t* T = (int32_t*)(uintptr_t)0x300000000ull;
  float* L = (float*)(uintptr_t)0x400000000ull;
  const int64_t MAXI = INT64_MAX, MINI = INT64_MIN;
  const int64_t Bs[] = {0, -1, MINI, (int64_t)1 << 31, MAXI};
  const int64_t Cs[] = {0, -1, MINI, ((int64_t)1 << 28) + 1, MAXI};
  for (unsigned i = 0; i < sizeof Bs / sizeof Bs[0]; ++i) {
    for (int dt = 0; dt < 3; ++dt) {
      REFUSED(ce_fwd_grad(Z, T, Bs[i], 10, dt, G, L, 0));
      REFUSED(ce_fwd_grad(Z, T, 8, Cs[i], dt, G, L, 0));
      REFUSED(ce_fwd_grad_loss(Z, T, Bs[i], 10, dt, G, L, L + 4096, 0, 0, 0));
      REFUSED(ce_fwd_grad_loss(Z, T, 8, Cs[i], dt, G, L, L + 4096, 0, 0, 0));
      REFUSED(ce_fwd_loss(Z, T, Bs[i], 10, dt, L, 0));
      REFUSED(ce_fwd_loss(Z, T, 8, Cs[i], dt, L, 0));
      REFUSED(ce_fwd_grad_scaled(Z, T, 8, Cs[i], dt, G, L, L, 0));
      REFUSED(ce_softmax_fwd(Z, Bs[i], 10, dt, G, L, 0));
      REFUSED(ce_softmax_fwd(Z, 8, Cs[i], dt, G, L, 0));
      REFUSED(ce_softmax_bwd(Z, G, Bs[i], 10, dt, Z + (1 << 20), 0));
      REFUSED(ce_softmax_bwd(Z, G, 8, Cs[i], dt, Z + (1 << 20), 0));
      REFUSED(ce_shard_stats(Z, T, Bs[i], 10, 0, dt, L, 0));
      REFUSED(ce_shard_stats(Z, T, 8, Cs[i], 0, dt, L, 0));
      REFUSED(ce_shard_grad(Z, T, Bs[i], 10, 0, 10, dt, L, 2, G, L, 0, 0));
      REFUSED(ce_shard_grad(Z, T, 8, Cs[i], 0, MAXI, dt, L, 2, G, L, 0, 0));
      REFUSED(ce_scale_grad(G, Bs[i] < 0 ? Bs[i] : -Bs[i] - 1, dt, L, 0));
      /* strides: below C, and so large that a span would overflow */
      REFUSED(ce_fwd_grad_ex(Z, 9, T, 8, 10, dt, G, 10, L, 0, CE_NO_IGNORE, 0, 0, 0));
      REFUSED(ce_fwd_grad_ex(Z, MAXI, T, Bs[i] == 0 ? 3 : Bs[i], 10, dt, G, MAXI, L, 0,
                             CE_NO_IGNORE, 0, 0, 0));
      REFUSED(ce_fwd_grad_ex(Z, MAXI, T, 8, 10, dt, G, 10, L, 0, CE_NO_IGNORE, 0, 0, 0));
      REFUSED(ce_fwd_grad_ex(Z, MAXI / 2, T, 8, MAXI / 4, dt, 0, 0, L, 0, -100, 0, 0, 0));
    }
    REFUSED(ce_fwd_grad(Z, T, 8, 10, 3, G, L, 0));
    REFUSED(ce_fwd_grad(Z, T, 8, 10, -1, G, L, 0));
  }
  /* null pointers, misalignment, overlaps */
  REFUSED(ce_fwd_grad(0, T, 8, 10, CE_F32, G, L, 0));
  REFUSED(ce_fwd_grad(Z, 0, 8, 10, CE_F32, G, L, 0));
  REFUSED(ce_fwd_grad(Z, T, 8, 10, CE_F32, 0, L, 0));
  REFUSED(ce_fwd_grad(Z, T, 8, 10, CE_F32, G, 0, 0));
  REFUSED(ce_fwd_grad(Z + 2, T, 8, 10, CE_F32, G, L, 0));
  REFUSED(ce_fwd_grad(Z, T, 8, 10, CE_F32, G + 4, L, 0));
  REFUSED(ce_fwd_grad(Z, T, 8, 10, CE_F32, Z + 16, L, 0));
  REFUSED(ce_fwd_grad(Z, T, 8, 10, CE_BF16, Z + 1, L, 0));
  REFUSED(ce_fwd_grad(Z, (int32_t*)(Z + 2), 8, 10, CE_F32, G, L, 0));
  /* the reduction */
  EQ(ce_reduce_workspace_bytes(0), 0u);
  EQ(ce_reduce_workspace_bytes(MINI), 0u);
  EQ(ce_reduce_workspace_bytes(MAXI), 0u);
  EQ(ce_reduce_workspace_bytes(16384), 0u);
  EQ(ce_reduce_workspace_bytes(16385), 36u);
  EQ(ce_reduce_workspace_bytes((int64_t)1 << 39), 4096u);
  REFUSED(ce_reduce_loss(L, MAXI, L + 4, 0, 0, 0));
  REFUSED(ce_reduce_loss(L, 0, L + 4, 0, 0, 0));
  REFUSED(ce_reduce_loss(L, 1 << 20, L + 4, 0, 0, 0));
  REFUSED(ce_reduce_loss(L, 1 << 20, L + 4, G, 3, 0));
  REFUSED(ce_reduce_loss(0, 8, L, 0, 0, 0));
  /* the whole step: the reduction's arguments are refused before a launch */
  REFUSED(ce_fwd_grad_loss(Z, T, 8, 10, 0, G, L, 0, 0, 0, 0));
  REFUSED(ce_fwd_grad_loss(Z, T, 8, 10, 0, G, L, (float*)(Z + 2), 0, 0, 0));
  REFUSED(ce_fwd_grad_loss(Z, T, 1 << 20, 10, 0, G, L, L + 4096, 0, 0, 0));
  REFUSED(ce_fwd_grad_loss(Z, T, 1 << 20, 10, 0, G, L, L + 4096, G, 3, 0));
  REFUSED(ce_fwd_grad_loss(Z, T, 1 << 20, 10, 0, G, L, L + 4096, Z + 2, 4096, 0));
  REFUSED(ce_reduce_loss_noalloc(L, MAXI, L + 4, 0));
  REFUSED(ce_reduce_loss_noalloc(L, 0, L + 4, 0));
  REFUSED(ce_reduce_loss_noalloc((float*)(Z + 2), 8, L, 0));
  /* workspace sizes, paths, copies, strings */
  EQ(ce_fwd_workspace_bytes(CE_NO_IGNORE), 0u);
  EQ(ce_fwd_workspace_bytes(-100), 4u);
  EQ(ce_fwd_inplace_workspace_bytes(0), 0u);
  EQ(ce_fwd_inplace_workspace_bytes(MINI), 0u);
  EQ(ce_fwd_inplace_workspace_bytes(MAXI), 0u);
  EQ(ce_fwd_inplace_workspace_bytes(1), 400u);
  EQ(ce_fwd_inplace_workspace_bytes(2147483647), (size_t)256 + (size_t)144 * 2147483647);
  for (int64_t c = 1; c < ((int64_t)1 << 29); c = c * 3 + 1)
    for (int dt = 0; dt < 3; ++dt) (void)ce_select_path(c, dt);
  REFUSED(ce_select_path(0, CE_F32));
  REFUSED(ce_select_path(MAXI, CE_F32));
  REFUSED(ce_select_path(10, 7));
  REFUSED(ce_stream_copy(Z, G, 0, 0));
  REFUSED(ce_stream_copy(Z, G, MINI, 0));
  REFUSED(ce_stream_copy(Z, G, 17, 0));
  REFUSED(ce_stream_copy(Z, Z + 16, 64, 0));
  REFUSED(ce_shard_grad(Z, T, 8, 10, 0, 10, CE_F32, L, 0, G, L, 0, 0));
  REFUSED(ce_shard_grad(Z, T, 8, 10, 0, 10, CE_F32, L, 1025, G, L, 0, 0));
  REFUSED(ce_shard_grad(Z, T, 8, 10, MINI, 10, CE_F32, L, 2, G, L, 0, 0));
  REFUSED(ce_shard_grad(Z, T, 8, 10, MAXI, MAXI, CE_F32, L, 2, G, L, 0, 0));
  for (int s = -20; s <= 5; ++s)
    if (ce_status_string(s) == 0) ++fails;
  REFUSED(ce_debug_force_path(-1));
  REFUSED(ce_debug_force_path(99));
  REFUSED(ce_debug_part_polls(-1));
  printf("%s\n", ce_version());
  return fails == 0 ? 0 : 1;
}
"""


def _digest() -> str:
    h = hashlib.sha256(CLIENT.encode())
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


_pending = None   # the two HIP compiles, when started early by start_build()


def _have_compilers() -> bool:
    return (os.path.exists(os.path.join(ROCM, "bin", "hipcc"))
            and os.path.exists(os.path.join(ROCM, "llvm", "bin", "clang++")))


def _hip_compiles(out: str):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(out, exist_ok=True)
    # sanitizers on the host side of the HIP translation units only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs = []
    for src in ("ce_api.hip", "ce_wave.hip"):
        obj = os.path.join(out, src.replace(".hip", ".o"))
        jobs.append((obj, subprocess.Popen([hipcc, *common, *san, "-c", os.path.join(CSRC, src),
                                            "-o", obj], stdout=subprocess.PIPE,
                                           stderr=subprocess.STDOUT, text=True)))
    return jobs


def start_build() -> None:
    """Start the two HIP compiles in the background (called by conftest
    after collection, so that they overlap the other CPU tests); the test
    waits for them."""
    global _pending
    if _pending is not None or not _have_compilers():
        return
    out = os.path.join(CACHE, _digest())
    if os.path.exists(os.path.join(out, "client")):
        return
    shutil.rmtree(CACHE, ignore_errors=True)
    _pending = (out, _hip_compiles(out))


def _build(out: str) -> str:
    global _pending
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    if _pending is not None and _pending[0] == out:
        jobs = _pending[1]
    else:
        jobs = _hip_compiles(out)
    _pending = None
    client_src = os.path.join(out, "client.cpp")
    with open(client_src, "w") as f:
        f.write(CLIENT)
    client_obj = os.path.join(out, "client.o")
    res = subprocess.run([clangxx, "-std=c++11", "-g", "-Wall", "-Werror",
                          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                          f"-I{INCLUDE}", "-c", client_src, "-o", client_obj],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    for obj, proc in jobs:
        log = proc.communicate()[0]
        assert proc.returncode == 0, log[-3000:]
    exe = os.path.join(out, "client")
    res = subprocess.run([clangxx, "-fsanitize=address,undefined", *[o for o, _ in jobs], client_obj,
                          f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
                          f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan():
    if not _have_compilers():
        pytest.skip("ROCm compilers not available")
    out = os.path.join(CACHE, _digest())
    exe = os.path.join(out, "client")
    if not os.path.exists(exe):
        if _pending is None:
            shutil.rmtree(CACHE, ignore_errors=True)
        exe = _build(out)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.returncode, run.stdout[-2000:], run.stderr[-4000:])
    assert "gfx950" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
