"""Wait-state hazards around the kernels' inline assembly (CPU: compiles to gfx950 assembly).

Several kernels issue their global loads as inline assembly, so the compiler's
hazard recognizer does not see them as memory instructions.  On gfx9 a vector
ALU instruction that writes a scalar register (v_readlane, v_readfirstlane,
v_cmp into an SGPR pair...) needs five wait states before a memory instruction
reads that register; between compiler-generated instructions the compiler
inserts them, before an inline-asm block it does not.  If the compiler spills a
scalar base address and reloads it with v_readlane right before such a load,
the load reads the stale register and accesses a wild address.

A second hazard of the same origin: the destination registers of an asm load
fill asynchronously, and a copy the compiler places after the load (where two
code paths with loads of their own merge) reads them before the data lands.

These tests compile the library's sources for gfx950 and check, in every
kernel, that no scalar register read inside an inline-asm block was written by
a vector ALU instruction among the five instructions before it (each
instruction is at least one wait state; s_nop N counts N + 1), and that no
instruction touches an asm load's destination before a wait covers it along
the fall-through path (early_reads).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))



def _shipped_build():
    """The library's own build description (fp32_gemm_04_amd/_build.py), loaded
    by path so that importing it needs no built library: the scan compiles
    exactly the translation units and flags that are shipped."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_sgemm_build_for_scan", os.path.join(ROOT, "fp32_gemm_04_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


_BUILD = _shipped_build()
FLAGS = list(_BUILD.FLAGS) + ["--cuda-device-only", "-S"]
CSRC = _BUILD.CSRC
HIPCC = _BUILD.HIPCC

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


VGPR = re.compile(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b")


def vgprs(text):
    out = set()
    for a, b, c in VGPR.findall(text):
        if c:
            out.add(int(c))
        else:
            out.update(range(int(a), int(b) + 1))
    return out


def _vmem(op):
    return op.startswith(("global_", "buffer_", "flat_", "scratch_"))


def _step(state, line, in_asm, report=None):
    """One instruction of the in-flight analysis: state maps each register an
    asm load is still filling to the number of vector memory operations
    issued after that load (a `s_waitcnt vmcnt(N)` retires it once N have)."""
    op = line.split()[0]
    if op == "s_waitcnt":
        m = re.search(r"vmcnt\((\d+)\)", line)
        if m:
            n = int(m.group(1))
            state = {r: c for r, c in state.items() if c < n}
        return state
    if not in_asm and report is not None:
        touched = vgprs(line.split(None, 1)[1]) if " " in line else set()
        if touched & set(state):
            report.append(line)
    if _vmem(op):
        state = {r: min(c + 1, 64) for r, c in state.items()}
        if in_asm and "load" in op and "_lds" not in op:
            for r in vgprs(line.split(None, 1)[1].split(",")[0]):
                state[r] = 0
    return state


def _blocks(func):
    """Basic blocks of one kernel's assembly: (instructions, successors),
    an instruction being (text, inside an inline-asm block)."""
    blocks, labels = [[]], {}
    in_asm = False
    for raw in func.split("\n")[1:]:
        l = raw.strip()
        if l.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if l.startswith(";;#ASMEND"):
            in_asm = False
            continue
        m = re.match(r"^(\.LBB\w+):", l)
        if m:
            if blocks[-1]:
                blocks.append([])
            labels[m.group(1)] = len(blocks) - 1
            continue
        if not l or l.startswith((";", ".")) or l.endswith(":"):
            continue
        blocks[-1].append((l, in_asm))
        op = l.split()[0]
        if op in ("s_branch", "s_endpgm") or op.startswith(("s_cbranch", "s_setpc")):
            blocks.append([])
    succ = []
    for i, b in enumerate(blocks):
        last = b[-1][0] if b else ""
        op = last.split()[0] if last else ""
        target = labels.get(last.split()[1]) if len(last.split()) > 1 else None
        if op == "s_branch":
            nxt = [target]
        elif op.startswith("s_cbranch"):
            nxt = [target, i + 1]
        elif op == "s_endpgm" or op.startswith("s_setpc"):
            nxt = []
        else:
            nxt = [i + 1]
        succ.append([j for j in nxt if j is not None and j < len(blocks)])
    return blocks, succ


def early_reads(asm):
    """Instructions that touch a register an inline-asm load may still be
    filling, along fall-through paths.

    Loads issued by inline assembly fill their destination registers
    asynchronously, and the compiler does not know it: it may copy such a
    register right after the asm statement (for instance where two code paths
    with loads of their own merge), reading it before the data arrives.  The
    scan follows the code in text order through conditional branches (along
    their fall-through side, a path that runs when the branch is not taken);
    an unconditional branch or the end of the program ends the path, since
    the block after it is reached only by jumps.  On the path, each asm load
    in flight counts the vector memory operations (loads, stores, LDS DMA)
    issued after it and is retired by a `s_waitcnt vmcnt(N)` once N have
    been; any instruction outside the asm blocks that reads or writes a
    register still being filled is reported."""
    found = []
    for func in re.split(r"\n(?=_Z\w+:)", asm):
        if not func.startswith("_Z"):
            continue
        name = func.split(":", 1)[0].strip()
        blocks, _ = _blocks(func)
        state = {}
        for b in blocks:
            report = []
            for line, in_asm in b:
                state = _step(state, line, in_asm, report)
            found += [(name[:70], l) for l in report]
            last = b[-1][0].split()[0] if b else ""
            if last in ("s_branch", "s_endpgm") or last.startswith("s_setpc"):
                state = {}
    return found


SOURCES = [(name, list(extra)) for name, extra in _BUILD.SOURCES.items()]


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    """gfx950 assembly of each translation unit, compiled once for the module."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")
    jobs = []
    for source, extra in SOURCES:  # both compiles at once
        path = d / (source + ".s")
        cmd = [HIPCC] + FLAGS + extra + ["-o", str(path), os.path.join(CSRC, source)]
        jobs.append((source, path, subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                                    stderr=subprocess.DEVNULL)))
    out = {}
    for source, path, proc in jobs:
        assert proc.wait() == 0, "hipcc failed on " + source
        out[source] = path.read_text()
    return out


@pytest.mark.parametrize("source", [src for src, _ in SOURCES])
def test_no_early_use_of_asm_load_results(assembly, source):
    found = early_reads(assembly[source])
    assert not found, "asm load destination used while in flight: %s" % found[:5]


def test_scanner_finds_early_reads():
    """The scanner itself: a copy of an asm load's destination before the
    wait is reported; the same copy after `s_waitcnt vmcnt(0)` is not, nor is
    a use of a register whose load an older wait already covered."""
    load = ["_Zk:", ";;#ASMSTART", "global_load_dwordx2 v[80:81], v2, s[74:75] nt", ";;#ASMEND"]
    bad = "\n".join(load + ["v_mov_b32_e32 v90, v80"])
    good = "\n".join(load + ["s_waitcnt vmcnt(0)", "v_mov_b32_e32 v90, v80"])
    older = "\n".join(load + [";;#ASMSTART", "global_load_dwordx2 v[82:83], v2, s[74:75] nt",
                               ";;#ASMEND", "s_waitcnt vmcnt(1)", "v_mov_b32_e32 v90, v80"])
    assert early_reads(bad) and not early_reads(good) and not early_reads(older)


@pytest.mark.parametrize("source", [src for src, _ in SOURCES])
def test_no_valu_sgpr_write_before_inline_asm_read(assembly, source):
    found = hazards(assembly[source])
    assert not found, "VALU-written SGPR read by inline asm too soon: %s" % found[:5]


def test_scanner_finds_the_hazard():
    """The scanner itself: a v_readlane right before an inline-asm load reading
    the same register is reported; five wait states in between are not."""
    bad = "\n".join(["_Zk:", "v_readlane_b32 s1, v145, 1", ";;#ASMSTART",
                     "global_load_dwordx2 v[80:81], v0, s[0:1] nt", ";;#ASMEND"])
    good = "\n".join(["_Zk:", "v_readlane_b32 s1, v145, 1", "s_nop 4", ";;#ASMSTART",
                      "global_load_dwordx2 v[80:81], v0, s[0:1] nt", ";;#ASMEND"])
    assert hazards(bad) and not hazards(good)
