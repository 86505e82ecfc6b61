"""The compiled gfx950 code reads no matrix-core result too early across a branch.

A matrix-core (MFMA) instruction writes its result registers several cycles after it issues;
the compiler pads straight-line code with wait states before the first vector-ALU read, but a
uniform branch placed between an MFMA and that read once left the taken path with too few
(the warm-up loss kernel read stale partial sums in exactly the registers read first after the
branch).  The kernels are written so that no branch sits there; this test compiles every HIP
source to gfx950 assembly, follows each branch found within a few instructions after an MFMA,
and counts the instructions (and s_nop cycles) before the first read of the MFMA's
destination on the taken path (a walk ends at an unconditional branch; a register written on
the path no longer holds the result).  Twelve cover the longest (16-pass) MFMA shapes in use.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_sparse_02_amd import build as B

NEED = 12


def _regs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


def _instrs(lines, start):
    for k in range(start, len(lines)):
        u = lines[k].strip()
        if u and not u.startswith((";", ".", "_")):
            yield u


def short_paths(asm: str):
    """(function, line, wait states, instruction) of every taken-branch path on which an
    MFMA destination is read by a vector-ALU instruction after fewer than NEED wait states."""
    lines = asm.split("\n")
    labels = {l.split(":")[0]: i for i, l in enumerate(lines) if re.match(r"^\.LBB\w+:", l)}
    func, found = "", []
    for i, l in enumerate(lines):
        if re.match(r"^_Z\w+:", l):
            func = l.split(":")[0]
        m = re.match(r"\s+v_mfma\S*\s+(v\[\d+:\d+\]|v\d+),", l)
        if not m:
            continue
        dst, ws = _regs(m.group(1)), 0
        for u in _instrs(lines, i + 1):
            if ws >= NEED or u.startswith("s_endpgm"):
                break
            if u.startswith("s_nop"):
                ws += int(u.split()[1]) + 1
                continue
            ws += 1
            bm = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", u)
            if not (bm and bm.group(1) in labels):
                continue
            ws2, live = ws, set(dst)
            for u2 in _instrs(lines, labels[bm.group(1)] + 1):
                if ws2 >= NEED or not live or u2.startswith(("s_endpgm", "s_branch")):
                    break
                if u2.startswith("s_nop"):
                    ws2 += int(u2.split()[1]) + 1
                    continue
                if u2.startswith("v_") and not u2.startswith("v_mfma"):
                    ops = re.findall(r"v\[\d+:\d+\]|v\d+", u2)
                    if len(ops) > 1 and set().union(*[_regs(o) for o in ops[1:]]) & live:
                        found.append((func, i + 1, ws2, u2))
                        break
                    if ops:                   # a register written here no longer holds the result
                        live -= _regs(ops[0])
                ws2 += 1
            if u.startswith("s_branch"):      # the lines after it are not on this path
                break
    return found


def test_scanner_flags_a_read_right_after_a_branch():
    asm = "\n".join(["_Zk:", "\tv_mfma_f32_16x16x32_bf16 v[34:37], v[26:29], v[30:33], v[46:49]",
                     "\ts_cbranch_scc1 .LBB0_2", "\tv_cmp_gt_i32_e32 vcc, v1, v2", ".LBB0_2:",
                     "\tv_fma_f32 v34, v34, v79, -v89"])
    assert len(short_paths(asm)) == 1
    padded = asm.replace("\ts_cbranch_scc1", "\ts_nop 7\n\ts_nop 7\n\ts_cbranch_scc1")
    assert short_paths(padded) == []
    # a register written on the path before the read no longer holds the result, and the
    # lines after an unconditional branch are not on the path
    overwritten = asm.replace(".LBB0_2:", ".LBB0_2:\n\tv_mov_b32_e32 v34, 0")
    assert short_paths(overwritten) == []
    jumped = "\n".join(["_Zk:", "\tv_mfma_f32_16x16x32_bf16 v[34:37], v[26:29], v[30:33], v[46:49]",
                        "\ts_branch .LBB0_3", ".LBB0_2:", "\tv_fma_f32 v34, v34, v79, -v89",
                        ".LBB0_3:", "\ts_nop 7", "\ts_nop 7", "\tv_add_f32_e32 v1, v34, v2"])
    assert short_paths(jumped) == []


def test_compiled_kernels_have_no_short_mfma_paths():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    sources = [s for s in B.SOURCES if s.endswith(".hip")]
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [hipcc, *B.COMMON, *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
                   os.path.join(B.CSRC, src), "-o", out]
            subprocess.run(cmd, check=True, capture_output=True)
            with open(out) as f:
                return src, short_paths(f.read())
        with ThreadPoolExecutor(max_workers=len(sources)) as ex:
            results = list(ex.map(one, sources))
    bad = [(src, p) for src, paths in results for p in paths]
    assert not bad, bad[:5]
