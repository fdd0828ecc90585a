"""Wait-state hazards around the kernels' inline assembly (CPU: compiles to gfx950 assembly).

Several kernels issue their global loads as inline assembly, so the compiler's
hazard recognizer does not see them as memory instructions.  On gfx9 a vector
ALU instruction that writes a scalar register (v_readlane, v_readfirstlane,
v_cmp into an SGPR pair...) needs five wait states before a memory instruction
reads that register; between compiler-generated instructions the compiler
inserts them, before an inline-asm block it does not.  If the compiler spills a
scalar base address and reloads it with v_readlane right before such a load,
the load reads the stale register and accesses a wild address.

This test compiles the library's sources for gfx950 and checks, in every
kernel, that no scalar register read inside an inline-asm block was written by
a vector ALU instruction among the five instructions before it (each
instruction is at least one wait state; s_nop N counts N + 1).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp32_gemm_04_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S"]

SGPR = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b")


def sgprs(text):
    out = set()
    for a, b, c in SGPR.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def valu_sgpr_dest(line):
    """Scalar registers a vector ALU instruction writes, if any."""
    op = line.split()[0] if line.split() else ""
    if not op.startswith("v_"):
        return set()
    if op.startswith(("v_readlane", "v_readfirstlane")):
        return sgprs(line.split(",")[0])
    if op.startswith("v_cmp") and "_e64" in op:
        return sgprs(line.split(",")[0])
    return set()


def wait_states(line):
    op = line.split()[0] if line.split() else ""
    if op == "s_nop":
        return int(line.split()[1], 0) + 1
    return 1


def hazards(asm):
    found = []
    for func in re.split(r"\n(?=_Z\w+:)", asm):
        name = func.split(":", 1)[0].strip()
        lines = [l.strip() for l in func.split("\n")]
        recent = []  # (sgprs written, wait states since)
        in_asm = False
        for l in lines:
            if l.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if l.startswith(";;#ASMEND"):
                in_asm = False
                continue
            if not l or l.startswith((";", ".")) or l.endswith(":"):
                continue
            if in_asm:
                reads = sgprs(l.split(" ", 1)[1]) if " " in l else set()
                for regs, ws in recent:
                    if regs & reads and ws < 5:
                        found.append((name[:70], l))
            ws_here = wait_states(l)
            recent = [(r, w + ws_here) for r, w in recent if w + ws_here < 5]
            written = valu_sgpr_dest(l)
            if written:
                recent.append((written, 0))
    return found


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("source,extra", [
    ("sgemm.hip", []),
    ("mfma_dl.hip", ["-Xarch_device", "-mllvm=--misched=gcn-max-ilp"]),
])
def test_no_valu_sgpr_write_before_inline_asm_read(tmp_path, source, extra):
    out = tmp_path / (source + ".s")
    subprocess.run([HIPCC] + FLAGS + extra + ["-o", str(out), os.path.join(CSRC, source)],
                   check=True, capture_output=True)
    found = hazards(out.read_text())
    assert not found, "VALU-written SGPR read by inline asm too soon: %s" % found[:5]


def test_scanner_finds_the_hazard():
    """The scanner itself: a v_readlane right before an inline-asm load reading
    the same register is reported; five wait states in between are not."""
    bad = "\n".join(["_Zk:", "v_readlane_b32 s1, v145, 1", ";;#ASMSTART",
                     "global_load_dwordx2 v[80:81], v0, s[0:1] nt", ";;#ASMEND"])
    good = "\n".join(["_Zk:", "v_readlane_b32 s1, v145, 1", "s_nop 4", ";;#ASMSTART",
                      "global_load_dwordx2 v[80:81], v0, s[0:1] nt", ";;#ASMEND"])
    assert hazards(bad) and not hazards(good)
