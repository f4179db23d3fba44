"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

Usage:  python -m gated_delta_rule_conv1d_amd.build   (or call build()).
Each translation unit compiles in parallel to an object file under _build/,
then one link produces gated_delta_rule_conv1d_amd/libgdn.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgdn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["gdn_api.hip", "conv1d.hip", "norm_gate.hip", "gates.hip", "recurrent.hip", "chunk_fwd.hip", "chunk_bwd.hip", "state_wide.hip",
           "profile.hip", "probe.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libgdn.so")


def flags():
    return ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
            # keep the compiler away from packed fp32 vector instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(ln for ln in proc.stdout.splitlines() if noise not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
