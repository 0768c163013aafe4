"""Build libisoquant.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m compressed_space_attention_amd.build [--verbose] [--resource-usage]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libisoquant.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed-fp32 instructions stay disabled on this target.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The leading scalar arguments of the kernels (up to 14 dwords) arrive in
    # SGPRs at wave launch: no kernel-argument load on the prologue's
    # critical path.
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra: list[str]) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    objs = [o for o, _ in results]
    if verbose or resource_usage:
        for o, err in results:
            lines = [l for l in err.splitlines() if "packed-fp32-ops" not in l]
            if lines:
                print(f"== {os.path.basename(o)}\n" + "\n".join(lines))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(a.verbose, a.resource_usage))
    sys.exit(0)
