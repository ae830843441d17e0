"""Build the HIP library libmla_kv.so in place (gfx950), with hipcc.

    python -m mla_latent_kv_20_amd.build          # or build() from Python

Every call compiles from source.  The library is written next to this file, with
kernel_resources.txt: the compiler's register, LDS and scratch figures of every kernel.  A
kernel that spills to scratch fails the build.
"""

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_kv.so")
RESOURCES = os.path.join(HERE, "kernel_resources.txt")
SOURCES = ["api.cpp", "decode_bf16.hip", "absorb_bf16.hip", "merge_f32.hip", "fused_bf16.hip", "prologue.hip",
           "quant_fp8.hip", "decode_fp8.hip", "fold.hip", "calib.hip", "noalloc.hip", "plan.cpp"]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source into libmla_kv.so; returns its path; raises on failure."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 VALU forms are disabled for all device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics",
           "-I", os.path.join(HERE, "..", "include"),
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
    errs = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    table = resource_table(lines)
    with open(RESOURCES, "w") as f:
        f.write(format_resources(table))
    spills = [k for k, r in table.items() if r.get("ScratchSize [bytes/lane]", 0) or r.get("VGPRs Spill", 0)]
    if spills:
        raise RuntimeError("kernels spill to scratch: " + ", ".join(spills))
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def resource_table(lines):
    """Per-kernel figures from the compiler's kernel-resource-usage remarks."""
    table, name = {}, None
    for l in lines:
        m = re.search(r"remark: Function Name: (\S+)", l)
        if m:
            name = m.group(1)
            table[name] = {}
            continue
        m = re.search(r"remark:\s+([^:]+): (\S+) \[-Rpass-analysis=kernel-resource-usage\]", l)
        if m and name:
            try:
                table[name][m.group(1).strip()] = int(m.group(2))
            except ValueError:
                table[name][m.group(1).strip()] = m.group(2)
    return table


def format_resources(table) -> str:
    cols = ["VGPRs", "AGPRs", "TotalSGPRs", "ScratchSize [bytes/lane]", "VGPRs Spill", "LDS Size [bytes/block]",
            "Occupancy [waves/SIMD]"]
    out = ["kernel\t" + "\t".join(cols)]
    for k in sorted(table):
        out.append(k + "\t" + "\t".join(str(table[k].get(c, "")) for c in cols))
    return "\n".join(out) + "\n"


if __name__ == "__main__":
    print(build(verbose=True))
