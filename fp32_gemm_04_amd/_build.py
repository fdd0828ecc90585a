"""Compile the HIP sources of libsgemm for gfx950 into the package folder."""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libsgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU instructions stay off: plain fp32 code must not be
    # turned into them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]
# Translation units and their own extra flags.  The direct-load kernels use
# the ILP machine scheduler: with the default one the accumulators of the
# two unrolled slabs are renamed and copied back every iteration (measured
# on the 160x160 kernel: 10 extra 64-bit moves per loop trip).  The other
# kernels keep the default, under which they do not spill.
SOURCES = {
    "sgemm.hip": [],
    "mfma_dl.hip": ["-Xarch_device", "-mllvm=--misched=gcn-max-ilp"],
    "conv.hip": [],
}


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    """Compile libsgemm.so (always recompiles) and return its path."""
    with tempfile.TemporaryDirectory(prefix="sgemm_build_") as tmpdir:
        objects, procs = [], []
        for name, extra in SOURCES.items():
            obj = os.path.join(tmpdir, name + ".o")
            cmd = [HIPCC, *FLAGS, *extra, "-c", "-o", obj, os.path.join(CSRC, name)]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd)))
            objects.append(obj)
        for cmd, proc in procs:
            if proc.wait() != 0:
                raise subprocess.CalledProcessError(proc.returncode, cmd)
        tmp = output + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objects]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
