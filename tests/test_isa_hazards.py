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
    srcs = [os.path.join(b.CSRC, f"gemm_b{bits}.hip") for bits in range(1, 9)] + [os.path.join(b.CSRC, "gemm_dense.hip")]
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


# A vector instruction reading a matrix-core result needs more wait states
# than the product has passes (gfx950: 8-pass 16x16x32 fp16 products need 11
# before a VALU or accumulation-register read of their destination).  The
# compiler counts them for the products it emits; the wide dense kernel's
# products are asm (accumulators pinned to accumulation registers) and wait
# behind an explicit drain, which this checks.
MIN_RESULT_WAIT_STATES = 11


def _result_violations(asm_path: str, window: int = 40) -> list:
    lines = [l.strip() for l in open(asm_path)]
    ins = [l for l in lines if l and not l.startswith((";", ".")) and not l.endswith(":")]
    bad = []
    for n, x in enumerate(ins):
        if not x.startswith("v_mfma"):
            continue
        dst = _regs(x.split(None, 1)[1].split(",")[0])
        waits = 0
        for y in ins[n + 1:n + 1 + window]:
            if y.startswith("s_nop"):
                waits += int(y.split()[1]) + 1
            else:
                if not y.startswith("v_mfma") and " " in y:
                    ops = y.split(None, 1)[1].split(",")
                    reads = set().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else set()
                    if y.startswith(("v_accvgpr_read", "global_store", "buffer_store", "ds_write", "scratch_store")):
                        reads |= set().union(*[_regs(o) for o in ops])
                    if reads & dst:
                        if waits < MIN_RESULT_WAIT_STATES:
                            bad.append(f"{os.path.basename(asm_path)}: {x[:50]} -> {waits} -> {y[:50]}")
                        break
                    if _regs(ops[0]) & dst and not y.startswith("v_mfma"):
                        break  # overwritten before any read
                waits += 1
            if waits >= MIN_RESULT_WAIT_STATES:
                break
    return bad


def test_mfma_results_read_after_their_passes(tmp_path):
    out = _asm(os.path.join(b.CSRC, "gemm_dense.hip"), str(tmp_path))
    assert sum(1 for l in open(out) if "v_mfma_f32_16x16x32_f16 a[" in l) > 32  # the asm products
    bad = _result_violations(out)
    assert not bad, f"{len(bad)} MFMA results read too soon, e.g. {bad[:3]}"


def test_result_checker_sees_a_too_early_read(tmp_path):
    asm = tmp_path / "planted_result.s"
    asm.write_text("v_mfma_f32_16x16x32_f16 a[0:3], v[14:17], v[40:43], a[0:3]\n"
                   "s_nop 3\n"
                   "v_accvgpr_read_b32 v5, a2\n"
                   "v_mfma_f32_16x16x32_f16 a[4:7], v[14:17], v[40:43], a[4:7]\n"
                   "s_nop 7\n"
                   "s_nop 7\n"
                   "v_accvgpr_read_b32 v6, a5\n")
    bad = _result_violations(str(asm))
    assert len(bad) == 1 and "v5, a2" in bad[0]
