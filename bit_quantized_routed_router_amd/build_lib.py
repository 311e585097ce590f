"""Build libds4moe.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_quantized_routed_router_amd.build_lib

Every .hip file is compiled for gfx950 with packed-fp32 instructions turned
off; the codec file additionally with -ffp-contract=off (its quantizer must
reproduce each IEEE step exactly).  Objects go to _build/, the shared library
next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libds4moe.so")

ARCH = os.environ.get("DS4MOE_ARCH", "gfx950")
COMMON = [
    "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fconstexpr-steps=100000000", "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
SOURCES = {
    "codec.hip": ["-ffp-contract=off"],
    "route.hip": [],
    "decode.hip": [],
    "prefill.hip": [],
    "hc.hip": [],
    "dense.hip": [],
    "capi.cpp": ["-x", "hip"],
    "trace.cpp": ["-x", "hip"],
}


def _compile(name: str, extra: list[str]) -> str:
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD, name + ".o")
    cmd = COMMON + extra + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if lines:
            print("\n".join(lines), file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
