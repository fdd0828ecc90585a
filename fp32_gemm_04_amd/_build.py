"""Compile the HIP sources of libsgemm for gfx950 into the package folder."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "sgemm.hip")]
DEPENDS = [os.path.join(HERE, "csrc", f) for f in ("common.hpp", "mfma_tile.hpp", "skinny.hpp", "valu_tile.hpp")]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libsgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Packed fp32 VALU instructions stay off: plain fp32 code must not be
    # turned into them.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]


def build(output: str = LIBRARY, verbose: bool = False) -> str:
    """Compile libsgemm.so (always recompiles) and return its path."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
