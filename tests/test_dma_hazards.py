"""The LDS copies (global_load_lds_dwordx4) are issued from inline assembly,
and the compiler inserts no wait states before an inline-asm instruction.
Two gfx9 hazards apply to them:
  * a VALU write of an SGPR (v_readfirstlane_b32, which turns a wave-uniform
    base address into scalar registers) must be followed by 5 wait states
    before a VMEM instruction reads that SGPR -- read earlier, the copy can
    take the register's previous value as its address;
  * an SALU write of M0 (the copy's LDS address) needs 1 wait state before
    the copy.
This test compiles every source that issues copies to gfx950 assembly (no GPU
needed) and checks both for every copy, scanning back through straight-line
code (a label or branch ends the scan; the copies' own leading s_nop covers
what lies beyond)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VALU_SGPR_TO_VMEM = 5
SALU_M0_TO_LDS_DMA = 1


def _sregs(text):
    out = set()
    for a, b, c in re.findall(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b", text):
        out |= set(range(int(a), int(b) + 1)) if a else {int(c)}
    return out


def _dest(instr):
    """Registers an instruction writes: its first operand."""
    body = instr.split(None, 1)[1] if " " in instr else ""
    first = body.split(",")[0].strip()
    if first == "m0":
        return {"m0"}
    return _sregs(first)


def _violations(asm_lines):
    out = []
    for j, line in enumerate(asm_lines):
        t = line.strip()
        if not t.startswith("global_load_lds"):
            continue
        reads = _sregs(t.split(None, 1)[1])
        ws = 0
        for i in range(j - 1, -1, -1):
            u = asm_lines[i].strip()
            if not u or u.startswith((";", ".")) and not re.match(r"^\.LBB\d+_\d+:", u):
                continue
            if re.match(r"^(\.LBB\d+_\d+|_Z\w+):", u) or u.startswith(("s_branch", "s_cbranch", "s_setpc")):
                break
            if ws >= VALU_SGPR_TO_VMEM:
                break
            dest = _dest(u)
            if u.startswith("v_") and dest & reads:
                out.append((j + 1, i + 1, ws, "VALU SGPR write"))
            if u.startswith("s_") and "m0" in dest and ws < SALU_M0_TO_LDS_DMA:
                out.append((j + 1, i + 1, ws, "M0 write"))
            nop = re.match(r"s_nop\s+(\d+)", u)
            ws += int(nop.group(1)) + 1 if nop else 1
    return out


def test_scanner_flags_short_gaps():
    """The scan itself: a readfirstlane two instructions before a copy that
    reads its register is flagged, as is an M0 write right before it; five
    wait states clear both."""
    early = ["v_readfirstlane_b32 s0, v12", "s_mov_b32 m0, s3", "s_nop 0",
             "global_load_lds_dwordx4 v126, s[0:1]"]
    bad = _violations(early)
    assert [b[3] for b in bad] == ["VALU SGPR write"]
    assert [b[3] for b in _violations(["s_mov_b32 m0, s3", "global_load_lds_dwordx4 v1, s[4:5]"])] == ["M0 write"]
    fixed = ["v_readfirstlane_b32 s0, v12", "s_mov_b32 m0, s3", "s_nop 4",
             "global_load_lds_dwordx4 v126, s[0:1]"]
    assert _violations(fixed) == []
    other = ["v_readfirstlane_b32 s7, v12", "global_load_lds_dwordx4 v126, s[0:1] offset:1024"]
    assert _violations(other) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not installed")
@pytest.mark.parametrize("src", ["mmq.hip"])
def test_lds_copies_wait_for_their_registers(tmp_path, src):
    from quant_integer_gemm_amd import build
    out = tmp_path / (src + ".s")
    r = subprocess.run([build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
                        os.path.join(ROOT, "quant_integer_gemm_amd", "csrc", src), "-o", str(out)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = out.read_text().split("\n")
    assert sum(1 for l in lines if l.strip().startswith("global_load_lds")) > 0
    bad = _violations(lines)
    assert not bad, f"copies too close to a write of their registers (copy line, write line, wait states): {bad[:5]}"
