"""Builds the HIP library ``libcgl_moe.so`` in-tree for gfx950 with hipcc.

Every source is compiled with ``-ffp-contract=off`` (no implicit fused
multiply-add: the kernels write every fma they mean) and without fast-math,
so fp32 division and rounding are IEEE; packed fp32 instructions are disabled
(``-packed-fp32-ops``).

The build fails if any kernel needs scratch memory (register spills): spill
code in the 256-row expert-MLP kernels has produced wrong results on gfx950
(one weight fragment reloaded with stale data), so every kernel must fit its
registers.  The compiler's per-kernel resource report is kept in
``_build/kernel_resources.txt``.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcgl_moe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
RESOURCES = os.path.join(BUILD_DIR, "kernel_resources.txt")

SOURCES = ["moe_api.hip", "route.hip", "layout.hip", "dispatch.hip", "combine.hip", "backward.hip", "fused.hip", "mlp.hip",
           "layer.hip"]
ARCH = os.environ.get("CGL_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


_REMARK = re.compile(r"remark:\s+(Function Name|ScratchSize \[bytes/lane\]|VGPRs|AGPRs|VGPRs Spill|SGPRs Spill):\s+(\S+)")


def kernel_resources(stderr: str) -> list[dict]:
    """Per-kernel entries of hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    out: list[dict] = []
    for key, val in _REMARK.findall(stderr):
        if key == "Function Name":
            out.append({"name": val})
        elif out:
            out[-1][key] = int(val)
    return out


def _compile(src: str) -> tuple[str, list[dict]]:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, kernel_resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    kernels = [k for _, ks in results for k in ks]
    with open(RESOURCES, "w") as f:
        for k in kernels:
            f.write(f"{k['name']} VGPRs={k.get('VGPRs')} AGPRs={k.get('AGPRs')} "
                    f"scratch={k.get('ScratchSize [bytes/lane]')} vgpr_spill={k.get('VGPRs Spill')}\n")
    spilling = [k["name"] for k in kernels if k.get("ScratchSize [bytes/lane]", 0) or k.get("VGPRs Spill", 0)]
    if not kernels:
        raise RuntimeError("hipcc printed no kernel resource report")
    if spilling:
        raise RuntimeError("kernels use scratch memory (register spills): " + ", ".join(spilling))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
