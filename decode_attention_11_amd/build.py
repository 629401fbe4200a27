"""Compile the gfx950 HIP sources into decode_attention_11_amd/libmla_decode.so.

Usage: python -m decode_attention_11_amd.build [--resource-usage]
hipcc cross-compiles for gfx950 without a GPU present.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off: hipcc would otherwise form v_pk_* fp32 ops on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(resource_usage: bool = False, extra=None) -> str:
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if extra:
        cmd += list(extra)
    tmp = LIB + ".tmp"
    cmd += ["-o", tmp, *sources()]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{msgs}")
    os.replace(tmp, LIB)
    if msgs and resource_usage:
        print(msgs)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv))
