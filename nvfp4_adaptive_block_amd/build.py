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


def kernel_source_hash() -> str:
    """First 16 hex digits of the SHA-256 of the kernel sources: profile
    summaries carry it, so figures taken on other kernel code are not used."""
    import hashlib
    h = hashlib.sha256()
    for f in ("fos_kernels.hip", "fos_device.h", "fos_kernels.h"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


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


RESOURCE_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
                   "Occupancy [waves/SIMD]": "occupancy_waves_per_simd", "SGPRs Spill": "sgpr_spill",
                   "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}


# the instances the benchmark's profile summaries cover (bf16, four-over-six
# MSE exact unless named), and their fused and 16x16 / fp32 relatives
RESOURCE_KERNELS = (
    "void fos::k_1x16<1, 0, 1, 1, 0, 0, 2, 0>(", "void fos::k_1x16<1, 0, 1, 1, 0, 0, 0, 0>(",
    "void fos::k_1x16<48, 0, 1, 1, 1, 0, 0, 1>(", "void fos::k_16x16<0, 1, 1, 0, 0, 0>(",
    "void fos::k_16x16<2, 1, 1, 0, 0, 0>(", "void fos::k_fused_onchip<0, 1, 1, 0, 0, 0>(",
    "void fos::k_fused_onchip<0, 1, 1, 1, 0, 1>(", "void fos::k_fused<0, 1, 1, 0, 0>(",
    "void fos::k_fused_row<0, 1, 1, 0, 0>(", "void fos::k_fused_grouped<0, 1, 1, 0, 0>(",
    "void fos::k_fused_list<0, 1, 1, 1, 0>(", "void fos::k_colwise<0, 1, 1, 0, 0>(", "void fos::k_dequant<0, 0>(",
    "void fos::k_amax_tensor<0>(")


def resource_usage(out: str) -> str:
    """Compile the kernels for gfx950 with the compiler's resource-usage
    remarks and write one `name | field=value ...` line per kernel of
    RESOURCE_KERNELS (VGPRs, SGPRs, spills, LDS and the waves per SIMD the
    resources allow) to `out`, names demangled as the profilers print them."""
    import re
    cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")], "-I", INCLUDE, "-I", CSRC,
           "--cuda-device-only", "-c", "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage",
           os.path.join(CSRC, "fos_kernels.hip")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise RuntimeError("hipcc failed")
    kernels, cur = [], None
    for ln in r.stderr.splitlines():
        m = re.search(r"remark: (?:\s*)(Function Name|[A-Za-z][^:]*?): (.*?) \[-Rpass", ln)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = {"mangled": val}
            kernels.append(cur)
        elif cur is not None and key in RESOURCE_FIELDS:
            cur[RESOURCE_FIELDS[key]] = val
    names = subprocess.run(["c++filt"], input="\n".join(k["mangled"] for k in kernels), capture_output=True,
                           text=True).stdout.splitlines()
    lines = ["# gfx950 kernel resources of fos_kernels.hip, from the compiler's resource-usage remarks:",
             "#   python3 -m nvfp4_adaptive_block_amd.build --resource-usage <this file>",
             "# occupancy_waves_per_simd is what the registers and LDS allow (at most 8)",
             f"# kernel_source_sha256_16 = {kernel_source_hash()}"]
    for k, name in sorted(zip(kernels, names), key=lambda kv: kv[1]):
        if not name.startswith(RESOURCE_KERNELS):
            continue
        fields = " ".join(f"{v}={k.get(v, '?')}" for v in RESOURCE_FIELDS.values())
        lines.append(f"{name} | {fields}")
    open(out, "w").write("\n".join(lines) + "\n")
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--resource-usage":
        print(resource_usage(sys.argv[2]))
    else:
        print(build(quiet=False))
