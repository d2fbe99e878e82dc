"""The kernels' inline-asm epilogue instructions read MFMA results, and the
compiler inserts no wait states before an inline-asm read (read too early,
a result is wrong).  The kernels therefore order each read after another
MFMA has issued, or after enough other instructions.  This test compiles
csrc/mmq.hip to gfx950 assembly (no GPU needed) and checks, for every MFMA
whose result an inline-asm instruction reads before anything overwrites it,
that another MFMA issues in between or that at least 24 wait states pass
(the XDL-write to VALU-read requirement is at most 19).  The scan follows
straight-line code and stops at branches."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NEED_WAIT_STATES = 24


def _regs(tok):
    if tok[0]:
        return set(range(int(tok[0]), int(tok[1]) + 1))
    return {int(tok[2])}


def _violations(asm_lines):
    out = []
    starts = [i for i, l in enumerate(asm_lines) if re.match(r"^_Z\w+:", l)]
    for st in starts:
        end = next((i for i in range(st, len(asm_lines)) if asm_lines[i].startswith(".Lfunc_end")), len(asm_lines))
        for i in range(st, end):
            t = asm_lines[i].strip()
            if not t.startswith("v_mfma"):
                continue
            m = re.match(r"v_mfma\S*\s+v\[(\d+):(\d+)\]", t)
            if not m:
                continue
            live = set(range(int(m.group(1)), int(m.group(2)) + 1))
            ws, mfma_between, in_asm = 0, False, False
            for j in range(i + 1, end):
                u = asm_lines[j].strip()
                if u.startswith(";;#ASMSTART"):
                    in_asm = True
                    continue
                if u.startswith(";;#ASMEND"):
                    in_asm = False
                    continue
                if not u or u.startswith((".", ";")):
                    continue
                if u.startswith(("s_branch", "s_cbranch", "s_setpc", "s_endpgm")):
                    break
                nop = re.match(r"s_nop\s+(\d+)", u)
                body = u.split(None, 1)[1] if " " in u else ""
                toks = re.findall(r"v\[(\d+):(\d+)\]|v(\d+)", body)
                srcs = set()
                for tk in toks[1:]:
                    srcs |= _regs(tk)
                if in_asm and not nop and srcs & live:
                    if not mfma_between and ws < NEED_WAIT_STATES:
                        out.append((asm_lines[st].split(":")[0], i + 1, j + 1, ws))
                    break
                if u.startswith("v_mfma"):
                    mfma_between = True
                if toks and not u.startswith(("s_", "ds_write", "global_store", "scratch_store", "buffer_store")):
                    live -= _regs(toks[0])
                    if not live:
                        break
                ws += int(nop.group(1)) + 1 if nop else 1
    return out


def test_scanner_flags_an_early_read():
    """The scan itself: an inline-asm read right after its MFMA is flagged;
    one after another MFMA, or after 24 wait states, is not."""
    early = ["_Zk:", "v_mfma_i32_32x32x32_i8 v[8:23], v[0:3], v[4:7], v[24:39]", ";;#ASMSTART",
             "v_fma_f32 v40, v8, v41, v42", ";;#ASMEND", ".Lfunc_end0:"]
    assert len(_violations(early)) == 1
    after_mfma = early[:2] + ["v_mfma_i32_32x32x32_i8 v[44:59], v[0:3], v[4:7], v[24:39]"] + early[2:]
    assert _violations(after_mfma) == []
    after_nops = early[:2] + ["s_nop 7", "s_nop 7", "s_nop 7"] + early[2:]
    assert _violations(after_nops) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is not installed")
def test_no_early_inline_asm_read_of_mfma_results(tmp_path):
    from quant_integer_gemm_amd import build
    out = tmp_path / "mmq.s"
    r = subprocess.run([build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S",
                        os.path.join(ROOT, "quant_integer_gemm_amd", "csrc", "mmq.hip"), "-o", str(out)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = out.read_text().split("\n")
    assert sum(1 for l in lines if l.strip().startswith("v_mfma")) > 0
    bad = _violations(lines)
    assert not bad, f"inline-asm reads of MFMA results too early (kernel, mfma line, read line, wait states): {bad[:5]}"
