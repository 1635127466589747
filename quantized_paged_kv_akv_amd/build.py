"""Build libakv.so (hand-written HIP for gfx950) in-tree with hipcc.

    python -m quantized_paged_kv_akv_amd.build

Always recompiles.  The library lands next to this file so it travels with
the source tree.  The build fails if any kernel spills registers to scratch
memory: a spill in the streaming loop costs more than any tuning gains.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libakv.so")
SOURCES = ["akv_host.cpp", "merge.hip", "quantize.hip", "decode.hip", "ring.cpp", "calib.hip", "publish.hip", "lossless.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernel-argument preloading: up to 16 dwords of leading scalar kernel
    # arguments arrive in scalar registers at wave start instead of through a
    # load from the argument buffer (the combine pass and the split kernels'
    # first reads wait one round trip less; the code object keeps a prologue
    # that loads them the old way where the firmware does not preload)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I", os.path.join(ROOT, "include"),
]


def resource_usage(text: str) -> dict:
    """Per-kernel VGPRs, scratch bytes per lane and occupancy from the
    compiler's kernel-resource-usage remarks."""
    table, name = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            table[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            table[name][m.group(1).split(" ")[0]] = int(m.group(2))
    return table


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(HERE, "csrc", s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    usage = resource_usage(out)
    spills = {k: v["ScratchSize"] for k, v in usage.items() if v.get("ScratchSize", 0) > 0}
    if spills:
        os.remove(tmp)
        raise RuntimeError(f"kernels spill to scratch (bytes/lane): {spills}")
    if verbose:
        rest = "\n".join(line for line in out.splitlines() if "warning:" in line or "error:" in line)
        if rest.strip():
            print(rest)
        for k, v in sorted(usage.items()):
            print(f"  {k}: {v}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
