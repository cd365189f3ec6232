"""Build the HIP library libfos.so in-tree with hipcc for gfx950.

Run ``python -m nvfp4_adaptive_block_amd.build`` (or ``__graft_entry__.build()``).
The flags are part of the library's numerics: no FMA contraction, no fast
math, HIP's correctly rounded single-precision division, packed FP32
arithmetic disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libfos.so")
SOURCES = [os.path.join(CSRC, f) for f in ("fos_api.hip", "fos_kernels.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(out: str = LIB, extra: list[str] | None = None, quiet: bool = True, sources: list[str] | None = None) -> str:
    """Compile `sources` (default: the library) into the shared object `out`
    with the library's flags and include paths. Other sources built this way
    (test kernels that call the device helpers) get the same numerics."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC, *(sources or SOURCES), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    if msgs and not quiet:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
