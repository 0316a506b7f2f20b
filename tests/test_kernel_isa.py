"""Static checks of the register-streamed grouped GEMM's gfx950 assembly (no
GPU needed: the kernel source is compiled to assembly here).

Its MFMAs are written as inline assembly, which the compiler's hazard
recognizer does not look into, so the wait states it would insert around a
compiler-visible MFMA are the source's own responsibility:
  - a VALU write of a VGPR that an MFMA reads next needs wait states before
    the MFMA issues (a zero operand materialised just before the accumulator
    clear was once read stale this way);
  - the kernels must not spill to scratch (every accumulator and weight
    fragment lives in registers).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "scatter_grouped_gemm_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
MIN_WAIT_STATES = 4  # VALU write -> MFMA source read, with margin


def _regs(tok):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {tok} if m else set()


@pytest.fixture(scope="module")
def wreg_asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "gemm_wreg.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "gemm_wreg.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _instructions(text):
    insts = []
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            insts.append(("LABEL", []))
        elif not s.startswith("."):
            parts = s.replace(",", " ").split()
            insts.append((parts[0], parts[1:]))
    return insts


def test_valu_writes_are_settled_before_mfma_reads(wreg_asm):
    insts = _instructions(wreg_asm)
    n_mfma, bad = 0, []
    for i, (op, ops) in enumerate(insts):
        if not op.startswith("v_mfma"):
            continue
        n_mfma += 1
        srcs = set().union(*(_regs(t) for t in ops[1:]))
        ws = 0
        for j in range(i - 1, max(-1, i - 12), -1):
            op2, ops2 = insts[j]
            if op2 == "LABEL":
                break
            if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & srcs:
                if ws < MIN_WAIT_STATES:
                    bad.append((op2, ops2[0], op, ws))
                break
            ws += int(ops2[0]) + 1 if op2 == "s_nop" else 1
            if ws >= MIN_WAIT_STATES:
                break
    assert n_mfma > 1000
    assert not bad, bad[:10]


def test_no_scratch_and_full_accumulator_file(wreg_asm):
    kernels = re.findall(r"\.name:\s+(\S*gemm_wreg_kernel\S*)", wreg_asm)
    assert len(kernels) == 6  # {bf16, fp8} x {plain, SiLU bf16, SiLU e4m3}
    assert not re.search(r"\bscratch_(load|store)", wreg_asm)
    for m in re.finditer(r"\.private_segment_fixed_size:\s+(\d+)", wreg_asm):
        assert int(m.group(1)) == 0
