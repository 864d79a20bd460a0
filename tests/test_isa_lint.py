"""Lint of the gfx950 assembly of the HIP library (CPU only: hipcc
cross-compiles).

* No kernel uses scratch memory (a register spill in a hot loop).
* No packed fp32 VALU instruction is emitted (the library is built with that
  feature disabled).
* No store (or 16-byte compare-and-swap) wider than 8 bytes has its data
  registers overwritten by a VALU instruction less than two wait states later: such a store reads its data
  registers after it issues, and the compiler does not insert the wait
  states when the store's soffset is a register.  A silent corruption of
  exactly this kind was seen on the GPU; the kernels guard every 16-byte
  store, and this test keeps it that way.
* Every kernel fits in the 160 KB of LDS of a compute unit; the row-part
  kernels, which run two 1024-thread workgroups per compute unit, fit in
  64 VGPRs and half the LDS.
* No kernel writes through the scalar data cache (scalar stores, scalar
  atomics, scalar cache write-back or invalidate of written data): every
  store, including the mailbox words the row parts trade, is a vector
  memory instruction.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from softmax_cross_entropy_ce_amd import build as B

PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma|mov)_f32\b")
SCALAR_WRITE = re.compile(r"^\s+s_(store|buffer_store|scratch_store|atomic|buffer_atomic|"
                          r"dcache_wb|dcache_discard)\w*", re.M)


def _vregs(tok: str) -> set[int]:
    tok = tok.rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def wide_store_hazards(asm: str, wait_states: int = 2) -> list[str]:
    lines = asm.splitlines()
    func, out = None, []
    for i, line in enumerate(lines):
        if re.match(r"^[_A-Za-z][\w.]*:", line):
            func = line.split(":")[0]
        m = re.match(r"\s+(buffer|global|flat)_(store_dwordx[34]|atomic_cmpswap_x2)\s+(.*)", line)
        if not m:
            continue
        ops = m.group(3).split()
        if m.group(2).startswith("atomic"):
            # the 16-byte data operand (new value and compare value)
            data = next((r for r in map(_vregs, ops) if len(r) == 4), set())
        else:
            data = _vregs(ops[1] if m.group(1) == "global" else ops[0])
        ws, j = 0, i + 1
        while j < len(lines) and ws < wait_states:
            t = lines[j].strip()
            j += 1
            if not t or t.startswith((";", ".")) or t.endswith(":"):
                continue
            parts = t.split()
            if parts[0] == "s_nop":
                ws += int(parts[1], 0) + 1
                continue
            if parts[0].startswith("v_") and len(parts) > 1 and _vregs(parts[1]) & data:
                out.append(f"{func}: {line.strip()} -> {t}")
                break
            ws += 1
    return out


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    work = tmp_path_factory.mktemp("isa")
    flags = [f for f in B.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    procs = []
    for src in B.SOURCES:
        out = work / (os.path.splitext(src)[0] + ".s")
        cmd = [hipcc, *flags, "--cuda-device-only", "-S", f"-I{B.INCLUDE}", f"-I{B.CSRC}",
               os.path.join(B.CSRC, src), "-o", str(out)]
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                             stderr=subprocess.STDOUT, text=True)))
    for out, proc in procs:
        log = proc.communicate()[0]
        assert proc.returncode == 0, log[-4000:]
    return "\n".join(out.read_text() for out, _ in procs)


def _kernel_meta(asm: str) -> dict[str, dict[str, int]]:
    meta: dict[str, dict[str, int]] = {}
    name = None
    for line in asm.splitlines():
        m = re.match(r"\s+\.amdhsa_kernel\s+(\S+)", line)
        if m:
            name = m.group(1)
            meta[name] = {}
            continue
        if name:
            m = re.match(r"\s+\.amdhsa_(private_segment_fixed_size|group_segment_fixed_size|"
                         r"next_free_vgpr)\s+(\d+)", line)
            if m:
                meta[name][m.group(1)] = int(m.group(2))
            if ".end_amdhsa_kernel" in line:
                name = None
    return meta


def test_kernels_present(device_asm):
    meta = _kernel_meta(device_asm)
    names = " ".join(meta)
    for k in ("ce_short_kernel", "ce_tiny_kernel", "ce_row_kernel", "ce_row_lds_kernel",
              "ce_reduce_kernel", "ce_part_kernel", "ce_shard_grad_kernel", "ce_scale_kernel",
              "ce_count_kept_kernel", "sm_bwd_short_kernel", "sm_bwd_row_kernel",
              "sm_bwd_part_kernel", "ce_wave_kernel", "sm_bwd_wave_kernel",
              "ce_shard_grad_tiny_kernel", "ce_staged_kernel", "sm_bwd_staged_kernel"):
        assert k in names, k


def test_no_scratch(device_asm):
    meta = _kernel_meta(device_asm)
    spills = {k: v["private_segment_fixed_size"] for k, v in meta.items()
              if v.get("private_segment_fixed_size", 0)}
    assert not spills, spills


def test_lds_fits(device_asm):
    meta = _kernel_meta(device_asm)
    for k, v in meta.items():
        assert v.get("group_segment_fixed_size", 0) <= 160 * 1024, k


def test_1024_thread_kernels_fit_registers(device_asm):
    meta = _kernel_meta(device_asm)
    for k, v in meta.items():
        if "Li1024E" in k or "ce_row_lds_kernel" in k:
            assert v["next_free_vgpr"] <= 128, (k, v["next_free_vgpr"])


def test_part_kernels_fit_two_per_cu(device_asm):
    """The row-part kernels of the loss and softmax (ce_part_kernel) and of
    the softmax backward (sm_bwd_part_kernel) run two 1024-thread
    workgroups per CU: at most 64 VGPRs and half the LDS each."""
    meta = _kernel_meta(device_asm)
    parts = {k: v for k, v in meta.items() if "ce_part_kernel" in k or "sm_bwd_part_kernel" in k}
    assert any("sm_bwd_part_kernel" in k for k in parts)
    for k, v in parts.items():
        assert v["next_free_vgpr"] <= 64, (k, v["next_free_vgpr"])
        assert v.get("group_segment_fixed_size", 0) <= 80 * 1024, k


def test_no_scalar_memory_writes(device_asm):
    hits = SCALAR_WRITE.findall(device_asm)
    assert not hits, hits[:5]


def test_scalar_write_pattern_matches():
    assert SCALAR_WRITE.search("\ts_store_dword s0, s[2:3], 0x0\n")
    assert SCALAR_WRITE.search("\ts_atomic_add s0, s[2:3], 0x0\n")
    assert SCALAR_WRITE.search("\ts_dcache_wb\n")
    assert not SCALAR_WRITE.search("\ts_load_dwordx2 s[0:1], s[4:5], 0x0\n")
    assert not SCALAR_WRITE.search("\tglobal_atomic_cmpswap_x2 v1, v[2:5], s[0:1]\n")


def test_no_packed_fp32(device_asm):
    hits = PACKED_FP32.findall(device_asm)
    assert not hits, hits[:5]


def test_no_wide_store_hazard(device_asm):
    bad = wide_store_hazards(device_asm)
    assert not bad, bad[:10]


def test_hazard_scanner_catches_the_pattern():
    """The scanner flags the sequence that corrupted stores on the GPU and
    accepts it once two wait states separate the write."""
    bad = ("k:\n\tbuffer_store_dwordx4 v[58:61], v1, s[24:27], s48 offen nt\n"
           "\t; sched_barrier mask(0x00000000)\n\tv_mov_b32_e32 v58, s15\n")
    good = bad.replace("\t; sched_barrier", "\ts_nop 1\n\t; sched_barrier")
    assert wide_store_hazards(bad) and not wide_store_hazards(good)
    cas = "k:\n\tglobal_atomic_cmpswap_x2 v36, v[34:37], s[0:1] offset:-16\n\tv_mov_b32_e32 v34, s62\n"
    cas_ok = cas.replace("\tv_mov", "\ts_mov_b32 s48, s33\n\ts_mov_b32 s49, s33\n\tv_mov")
    assert wide_store_hazards(cas) and not wide_store_hazards(cas_ok)
