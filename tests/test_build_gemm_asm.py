"""Build-property checks of the grouped GEMM's device code (no GPU needed).

The GEMM's stage loop keeps 128 fp32 accumulators and the operand fragments
of two MFMA windows per lane, with eight waves per CU (two per SIMD), so it
runs at the 256-register limit of a wave.  A register spill inside a stage
loop would put a scratch load on the vector-memory counter that the stage
barrier waits on, behind the stage's in-flight direct-to-LDS loads, and
serialize the loop.  These tests compile mx_gemm.hip for gfx950 with the
library's own flags and check, for every GEMM kernel, that it still fits two
waves per SIMD and that no loop issuing MFMAs touches scratch memory.
"""

import os
import re
import shutil
import subprocess

import pytest

from mxfp8_block_scaled_06_amd import build as b


def _hipcc():
    try:
        return b.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    cc = _hipcc()
    if cc is None or shutil.which(cc) is None and not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mx_gemm.s"
    cmd = [cc, *b.HIP_FLAGS, "-I", b.INCLUDE, "-I", b.CSRC, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "mx_gemm.hip"), "-o", str(out)]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert proc.returncode == 0, proc.stdout[-4000:]
    return out.read_text().splitlines()


def _kernels(lines):
    """{kernel symbol: (first line, last line)} of every grouped GEMM kernel."""
    spans = {}
    cur = None
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3mxk19grouped_gemm_kernel\S*):", l)
        if m:
            cur = m.group(1)
            spans[cur] = [i, None]
        elif cur is not None and l.startswith(".Lfunc_end") and spans[cur][1] is None:
            spans[cur][1] = i
            cur = None
    return {k: tuple(v) for k, v in spans.items()}


def test_every_gemm_kernel_fits_two_waves_per_simd(gemm_asm):
    kernels = _kernels(gemm_asm)
    assert len(kernels) == 4, kernels          # modes 0 / 1, bf16 / fp32 output
    text = "\n".join(gemm_asm)
    # the per-kernel resource summary the compiler prints after each kernel body
    for name, (lo, hi) in kernels.items():
        tail = "\n".join(gemm_asm[hi:hi + 40])
        vg = int(re.search(r"; NumVgprs: (\d+)", tail).group(1))
        ag = int(re.search(r"; NumAgprs: (\d+)", tail).group(1))
        occ = int(re.search(r"; Occupancy: (\d+)", tail).group(1))
        assert vg + ag <= 256, (name, vg, ag)
        assert occ >= 2, (name, occ)
    assert "grouped_gemm_kernel" in text


def _loop_blocks(lines):
    """Basic blocks of the GEMM kernels as (kernel, loop headers enclosing the
    block, block lines), from the compiler's loop annotations ("Loop Header",
    "in Loop: Header=", "Parent Loop") on each block label."""
    blocks, cur = [], None
    kern = None
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3mxk19grouped_gemm_kernel\S*):", l)
        if m:
            kern, cur = m.group(1), None
            continue
        if kern is None:
            continue
        if l.startswith(".Lfunc_end"):
            kern, cur = None, None
            continue
        m = re.match(r"^(\.LBB(\d+_\d+)|; %bb\.\d+):(.*)$", l)
        if m:
            ann, j = m.group(3), i + 1
            while j < len(lines) and re.match(r"^\s+;", lines[j]):
                ann += " " + lines[j]
                j += 1
            loops = set(re.findall(r"(?:Header=|Parent Loop )BB(\d+_\d+)", ann))
            if "Loop Header" in ann and m.group(2):
                loops.add(m.group(2))
            cur = (kern, loops, [])
            blocks.append(cur)
        elif cur is not None:
            cur[2].append(l)
    return blocks


def test_no_stage_loop_spills(gemm_asm):
    """No loop that issues MFMAs (counting every block the compiler places in
    it, nested loops included) holds a scratch access."""
    per_loop = {}
    for kern, loops, body in _loop_blocks(gemm_asm):
        mfma = sum("v_mfma" in x for x in body)
        scratch = sum("scratch_" in x for x in body)
        for h in loops:
            m, s = per_loop.get((kern, h), (0, 0))
            per_loop[(kern, h)] = (m + mfma, s + scratch)
    assert per_loop, "no loops found"
    offenders = {k: v for k, v in per_loop.items() if v[0] and v[1]}
    assert not offenders, offenders
