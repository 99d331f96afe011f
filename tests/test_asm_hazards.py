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

A wait state is one instruction, or N+1 for ``s_nop N``.  The check follows
every control-flow path (fall-through and branch targets) within those
distances."""
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


def _cfg(lines):
    """Successor and predecessor lists of the instruction lines (labels end with ':')."""
    label_at = {ln[:-1]: i for i, ln in enumerate(lines) if ln.endswith(":")}
    succ = [[] for _ in lines]
    pred = [[] for _ in lines]
    for i, ln in enumerate(lines):
        op = ln.split()[0]
        nxt = []
        if op.startswith("s_cbranch") or op == "s_branch":
            target = ln.split()[1]
            if target in label_at:
                nxt.append(label_at[target])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(lines):
            nxt.append(i + 1)
        succ[i] = nxt
        for j in nxt:
            pred[j].append(i)
    return succ, pred


def scan(lines):
    """Problems found in one kernel's instruction lines (labels end with ':').

    Every path is followed, through branches and into labels, in both
    directions: backwards from an MFMA for a VALU write of one of its operands,
    forwards from an MFMA with an arch-VGPR result for a VALU read of it."""
    succ, pred = _cfg(lines)
    problems = []

    def back(i, srcs, ws, mfma, seen):
        for j in pred[i]:
            if (j, ws) in seen:
                continue
            seen.add((j, ws))
            p = lines[j]
            if p.endswith(":"):
                back(j, srcs, ws, mfma, seen)
                continue
            op = p.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma") and _operands(p):
                if _regs(_operands(p)[0]) & srcs:
                    problems.append(f"{p} writes an operand of {mfma} {ws} wait states before it")
                    continue
            w = ws + _wait_states(p)
            if w < 2:
                back(j, srcs, w, mfma, seen)

    def fwd(i, dst, ws, mfma, seen):
        for j in succ[i]:
            if (j, ws) in seen:
                continue
            seen.add((j, ws))
            n = lines[j]
            if n.endswith(":"):
                fwd(j, dst, ws, mfma, seen)
                continue
            op = n.split()[0]
            if op.startswith("v_") and not op.startswith("v_mfma"):
                if any(_regs(o) & dst for o in _operands(n)[1:]):
                    problems.append(f"{n} reads the result of {mfma} {ws} wait states after it")
                    continue
            w = ws + _wait_states(n)
            if w < 12:
                fwd(j, dst, w, mfma, seen)

    for i, ins in enumerate(lines):
        if not ins.startswith("v_mfma"):
            continue
        ops = _operands(ins)
        back(i, _regs(ops[1]) | _regs(ops[2]), 0, ins, set())
        dst = _regs(ops[0])
        if any(r.startswith("v") for r in dst):
            # accumulation registers are read only by accvgpr moves after a fence
            fwd(i, dst, 0, ins, set())
    return problems


@pytest.fixture(scope="module")
def mla_asm(tmp_path_factory):
    try:
        cc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "mla.s"
    cmd = [cc, *_build.COMMON, "--cuda-device-only", "-S", os.path.join(_build.CSRC, "mla.hip"),
           "-o", str(out)]
    p = subprocess.run(cmd, capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    return out.read_text()


@pytest.fixture(scope="module", params=[KERNEL, "mla_fp8_kernel"])
def kernel_asm(mla_asm, request):
    text, kernel = mla_asm, request.param
    start = next(m.start() for m in re.finditer(r"^(\S*" + kernel + r"\S*):", text, re.M))
    end = text.index(".Lfunc_end", start)
    body = []
    for raw in text[start:end].splitlines()[1:]:
        ln = raw.split(";")[0].strip()
        if not ln or (ln.startswith(".") and not re.match(r"\.LBB\d+_\d+:", ln)):
            continue
        body.append(ln)
    meta = text[text.index(".name:           " + next(
        n for n in re.findall(r"\.name:\s+(\S+)", text) if kernel in n)):]
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
    # through a taken branch: the read at the target is 2 wait states away
    branch_read = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_cbranch_scc1 .LBB0_9",
                   "s_nop 7", "s_nop 7", ".LBB0_9:", "v_max_f32_e32 v30, v1, v1"]
    assert scan(branch_read)
    # a write on the path that jumps to the MFMA's block
    branch_write = ["v_mov_b32_e32 v18, v3", "s_branch .LBB0_4", "s_nop 7", ".LBB0_4:",
                    "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]
    assert scan(branch_write)
    # both paths into a join far enough from the MFMA: clean
    join = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", "s_cbranch_scc1 .LBB0_7",
            "s_nop 7", ".LBB0_7:", "s_nop 7", "s_nop 3", "v_max_f32_e32 v30, v1, v1"]
    assert not scan(join)
