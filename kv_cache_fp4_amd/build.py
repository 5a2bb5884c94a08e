"""Compile libkvfp4.so (HIP, gfx950) in-tree with hipcc.

Code object version 5 keeps the kernels loadable by the HIP runtime that torch bundles
(which may be older than the /opt/rocm compiler).

Flags that the arithmetic depends on:
  -ffp-contract=off                           no fused multiply-add unless written as fma
  -fhip-fp32-correctly-rounded-divide-sqrt    IEEE division for the per-block scale steps
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                              no packed-fp32 VALU instructions
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("kvfp4.hip", "kvfp4_attend.hip")]
LIB = os.path.join(PKG, "libkvfp4.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def compile_hip(srcs, out: str, extra_includes=()) -> str:
    if isinstance(srcs, str):
        srcs = [srcs]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    for d in extra_includes:
        inc += ["-I", d]
    cmd = [HIPCC, *HIP_FLAGS, *inc, "-o", out + ".tmp", *srcs]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> str:
    return compile_hip(SRCS, LIB)


if __name__ == "__main__":
    print(build())
