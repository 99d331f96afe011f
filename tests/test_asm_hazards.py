"""Host check of the compiled sparse-MLA kernel (no GPU needed).

The sparse-MLA kernel issues its MFMAs as inline asm (so that S and O can live
in different register files), which the compiler's hazard recognizer cannot see
into.  The asm carries its own wait states; this test compiles the kernel for
gfx950 with the build's flags and checks, on the generated code, that

* no MFMA reads a VGPR that a VALU instruction wrote less than 2 wait states
  before (the count the compiler itself inserts for the builtin on gfx950),
* no VALU instruction reads an arch-VGPR MFMA result less than 12 wait states
  after the MFMA (likewise), and
* the kernel does not spill (a spill would put scratch traffic into the loop).

A wait state is one instruction, or N+1 for ``s_nop N``.  A label closer than
the required distance is reported too: a branch into it could bring a VALU write
from elsewhere."""
import os
import re
import shutil
import subprocess

import pytest

from sparse_attention_08_amd import _build

KERNEL = "mla_bf16_kernel"


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.match(r"[va]\d+$", tok) else set()


def _wait_states(line):
    op = line.split()[0]
    return int(line.split()[1]) + 1 if op == "s_nop" else 1


def _operands(line):
    parts = line.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def scan(lines):
    """Problems found in one kernel's instruction lines (labels end with ':')."""
    problems = []
    for i, ins in enumerate(lines):
        if not ins.startswith("v_mfma"):
            continue
        ops = _operands(ins)
        srcs = _regs(ops[1]) | _regs(ops[2])
        ws = 0
        for p in reversed(lines[max(0, i - 16):i]):
            if p.endswith(":"):
                problems.append(f"label {p} {ws} wait states before {ins}")
                break
            op = p.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma") and _operands(p):
                if _regs(_operands(p)[0]) & srcs:
                    problems.append(f"{p} writes an operand of {ins} {ws} wait states before it")
                    break
            ws += _wait_states(p)
            if ws >= 2:
                break
        dst = _regs(ops[0])
        if not any(r.startswith("v") for r in dst):
            continue  # accumulation registers: read only by accvgpr moves after a fence
        ws = 0
        for n in lines[i + 1:i + 24]:
            if n.endswith(":"):
                if ws < 12:
                    problems.append(f"label {n} {ws} wait states after {ins}")
                break
            op = n.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma"):
                if any(_regs(o) & dst for o in _operands(n)[1:]) and ws < 12:
                    problems.append(f"{n} reads the result of {ins} {ws} wait states after it")
                    break
            ws += _wait_states(n)
            if ws >= 12:
                break
    return problems


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mla.s"
    cmd = [cc, *_build.COMMON, "--cuda-device-only", "-S", os.path.join(_build.CSRC, "mla.hip"),
           "-o", str(out)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    text = out.read_text()
    start = next(m.start() for m in re.finditer(r"^(\S*" + KERNEL + r"\S*):", text, re.M))
    end = text.index(".Lfunc_end", start)
    body = []
    for raw in text[start:end].splitlines()[1:]:
        ln = raw.split(";")[0].strip()
        if not ln or (ln.startswith(".") and not re.match(r"\.LBB\d+_\d+:", ln)):
            continue
        body.append(ln)
    meta = text[text.index(".name:           " + next(
        n for n in re.findall(r"\.name:\s+(\S+)", text) if KERNEL in n)):]
    return body, meta


def test_mfma_hazards_covered(kernel_asm):
    body, _ = kernel_asm
    assert sum(1 for ln in body if ln.startswith("v_mfma")) > 100
    problems = scan(body)
    assert not problems, "\n".join(problems[:10])


def test_no_spills(kernel_asm):
    _, meta = kernel_asm
    spills = int(re.search(r"\.vgpr_spill_count:\s+(\d+)", meta).group(1))
    assert spills == 0


def test_scanner_catches_planted_hazards():
    # the scan itself, on hand-made sequences
    write_then_mfma = ["v_mov_b32_e32 v18, v3", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]
    assert scan(write_then_mfma)
    covered = ["v_mov_b32_e32 v18, v3", "s_nop 1", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]
    assert not scan(covered)
    early_read = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_nop 7",
                  "v_max_f32_e32 v30, v1, v1"]
    assert scan(early_read)
    late_read = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_nop 7", "s_nop 3",
                 "v_max_f32_e32 v30, v1, v1"]
    assert not scan(late_read)
