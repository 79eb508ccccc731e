"""The inverse in the bf16 chunk kernels fuses a DPP row broadcast into v_fmac
through inline assembly, which the compiler's hazard recognizer does not see
into.  gfx950 needs two wait states between a vector-ALU write of a VGPR and a
DPP read of it; this test compiles each kernel source to gfx950 assembly (no
GPU needed) with the flags the build uses for that file, and checks that no
broadcast source is written by a vector-ALU instruction within the two
preceding instructions."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# both bf16 chunk kernels run the inverse with the fused broadcast
SOURCES = [os.path.join(ROOT, "gated_delta_rule_101_amd", "csrc", f) for f in ("kda_chunk_pipe.hip", "kda_chunk_ps.hip")]


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm_text):
    insts = [l.strip() for l in asm_text.split("\n")]
    insts = [l for l in insts if l and not l.startswith((";", ".")) and not l.endswith(":")]
    checked, bad = 0, []
    for idx, t in enumerate(insts):
        if "_dpp" not in t.split()[0]:
            continue
        ops = [o.strip() for o in t.split(None, 1)[1].split(",")]
        src0 = _vregs(ops[1])
        checked += 1
        waits, j = 0, idx - 1
        while j >= 0 and waits < 2:
            op = insts[j].split()[0]
            if op == "s_nop":
                waits += int(insts[j].split()[1], 0) + 1
                j -= 1
                continue
            if op.startswith("v_") and not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
                parts = insts[j].split(None, 1)
                dst = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
                if _vregs(dst) & src0:
                    bad.append((insts[j], t))
            waits += 1
            j -= 1
    return checked, bad


@pytest.mark.parametrize("src", SOURCES, ids=[os.path.basename(x) for x in SOURCES])
def test_dpp_broadcast_sources_have_their_wait_states(tmp_path, src):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    from gated_delta_rule_101_amd.build_lib import HIPCC_FLAGS, SOURCE_FLAGS
    # the flags the shipped object is built with (optimisation level and scheduler included)
    flags = [f for f in [*HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), [])] if f != "-fPIC"]
    if any(f.startswith("-O") for f in SOURCE_FLAGS.get(os.path.basename(src), [])):
        flags = [f for f in flags if not f.startswith("-O")] + \
                [f for f in SOURCE_FLAGS[os.path.basename(src)] if f.startswith("-O")]
    out = tmp_path / "k.o"
    subprocess.run([hipcc, *flags, "--save-temps", "-c", src, "-o", str(out)], cwd=tmp_path,
                   check=True, capture_output=True)
    asm = [f for f in os.listdir(tmp_path) if f.endswith(".s") and "gfx950" in f]
    assert asm, os.listdir(tmp_path)
    checked, bad = dpp_hazards(open(tmp_path / asm[0]).read())
    assert checked > 0
    assert not bad, bad[:5]


def test_hazard_checker_catches_a_planted_hazard():
    planted = "v_mov_b32_e32 v7, v3\nv_fmac_f32_dpp v9, v7, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
    assert len(dpp_hazards(planted)[1]) == 1
    spaced = "v_mov_b32_e32 v7, v3\ns_nop 1\nv_fmac_f32_dpp v9, v7, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
    assert dpp_hazards(spaced)[1] == []
