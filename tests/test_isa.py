"""Checks on the gfx950 assembly of the chunk kernels (CPU only: hipcc cross-compiles).

The pipelined kernel's T solve issues ``v_fmac_f32_dpp`` from inline assembly, so
the compiler's hazard recognizer does not guard it.  On this architecture a DPP
source register written by a VALU instruction needs two wait states before the
DPP read; the kernel relies on its DPP sources only ever being loaded from LDS.
This test rebuilds the kernel's assembly with the library's own flags and checks
that property on every DPP instruction, and that no kernel spills to scratch.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_38_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _asm(src, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    from gated_delta_rule_38_amd.build import FLAGS
    out = tmp_path / (os.path.basename(src) + ".s")
    flags = [f for f in FLAGS if f != "-fPIC"]
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)],
                       capture_output=True, text=True, cwd=CSRC)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm_text):
    """(number of DPP instructions, list of hazards) for gfx9-family DPP reads:
    a VALU write of a DPP instruction's src0 within the two preceding wait states."""
    lines = [l.strip() for l in asm_text.splitlines()]
    lines = [l for l in lines if l and not l.startswith((";", "."))]
    n, bad = 0, []
    for k, line in enumerate(lines):
        op = line.split()[0]
        if not op.endswith("_dpp"):
            continue
        n += 1
        src = _vregs(line.split()[2].rstrip(","))
        waits, j = 0, k - 1
        while waits < 2 and j >= 0:
            prev = lines[j].split()
            if prev[0].endswith(":"):
                j -= 1
                continue
            if prev[0] == "s_nop":
                waits += int(prev[1], 0) + 1
            else:
                if prev[0].startswith("v_") and not prev[0].startswith(("v_cmp", "v_readfirstlane", "v_readlane")):
                    if _vregs(prev[1].rstrip(",")) & src:
                        bad.append((lines[j], line))
                waits += 1
            j -= 1
    return n, bad


def test_hazard_checker_catches_a_planted_hazard():
    planted = """
    v_mov_b32_e32 v5, 1.0
    v_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
    v_add_f32_e32 v6, v7, v8
    s_nop 1
    v_fmac_f32_dpp v1, v6, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
    ds_read_b128 v[8:11], v0
    v_fmac_f32_dpp v1, v9, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf
    """
    n, bad = dpp_hazards(planted)
    assert n == 3
    assert len(bad) == 1 and "v5" in bad[0][1]


@pytest.mark.parametrize("src", ["kda_chunk_pipe.hip", "kda_chunk.hip"])
def test_chunk_kernel_isa(src, tmp_path):
    text = _asm(os.path.join(CSRC, src), tmp_path)
    n, bad = dpp_hazards(text)
    assert not bad, f"DPP read-after-VALU-write hazards: {bad[:5]}"
    if src == "kda_chunk_pipe.hip":
        assert n >= 120, "the T sweep's row-broadcast FMAs are missing"
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)]
    assert spills and max(spills) == 0
    scratch = [int(x) for x in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)]
    assert scratch and max(scratch) == 0
