"""Matrix-core operand hazards in the built kernels (host only, no GPU).

A matrix-core instruction may read a VGPR only two or more wait states after
a VALU instruction wrote it.  The compiler inserts those wait states for the
instructions it generates, but it cannot see writes made inside inline asm
(the decode's packed fp16 half-adds are asm), so the asm has to provide them
itself.  When it did not, an MFMA one instruction after the last half-add read
a stale operand under some schedules.  This test compiles every GEMM source to
gfx950 assembly and checks, for every MFMA, the distance (in issued
instructions plus s_nop wait states) back to the nearest VALU write of its A
or B operand registers.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from linear_exl3_input_amd import build as b

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

MIN_WAIT_STATES = 2
REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)")


def _regs(spec: str) -> set:
    out = set()
    for m in REG.finditer(spec):
        if m.group(1):
            out |= {f"{m.group(1)}{k}" for k in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add(f"{m.group(4)}{m.group(5)}")
    return out


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    flags = [f for f in b.COMMON if f not in ("-fPIC",)]
    subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", out], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out


def _violations(asm_path: str, window: int = 8) -> list:
    lines = [l.strip() for l in open(asm_path)]
    ins = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    bad = []
    for n, x in enumerate(ins):
        if not x.startswith("v_mfma"):
            continue
        ops = x.split(None, 1)[1].split(",")
        srcs = _regs(ops[1]) | _regs(ops[2])
        waits = 0
        for m in range(n - 1, max(n - 1 - window, -1), -1):
            y = ins[m]
            if y.startswith("s_nop"):
                waits += int(y.split()[1]) + 1
                continue
            if y.startswith("v_") and not y.startswith(("v_mfma", "v_accvgpr")):
                if _regs(y.split(None, 1)[1].split(",")[0]) & srcs:
                    if waits < MIN_WAIT_STATES:
                        bad.append(f"{os.path.basename(asm_path)}: {y[:60]} -> {waits} -> {x[:60]}")
                    break
            waits += 1
            if waits >= MIN_WAIT_STATES:
                break
    return bad


def test_every_mfma_operand_written_two_wait_states_earlier(tmp_path):
    srcs = [os.path.join(b.CSRC, f"gemm_b{bits}.hip") for bits in range(1, 9)]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        outs = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    total = sum(sum(1 for l in open(o) if l.strip().startswith("v_mfma")) for o in outs)
    assert total > 1000  # every width compiled to its GEMM kernels
    bad = [v for o in outs for v in _violations(o)]
    assert not bad, f"{len(bad)} MFMA operand reads too soon after a VALU write, e.g. {bad[:3]}"


def test_checker_sees_a_too_close_write(tmp_path):
    """The checker itself: a planted one-wait-state write is reported, a
    two-wait-state one is not."""
    asm = tmp_path / "planted.s"
    asm.write_text("v_add_f16_sdwa v41, v1, v1\n"
                   "v_lshrrev_b32_e32 v2, 8, v3\n"
                   "v_mfma_f32_16x16x32_f16 a[0:3], v[14:17], v[40:43], a[0:3]\n"
                   "v_add_f16_sdwa v45, v1, v1\n"
                   "s_nop 1\n"
                   "v_mfma_f32_16x16x32_f16 a[4:7], v[14:17], v[44:47], a[4:7]\n")
    bad = _violations(str(asm))
    assert len(bad) == 1 and "v41" in bad[0]
