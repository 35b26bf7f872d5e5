"""Build libspecverify.so in-tree with hipcc for gfx950.

Usage: ``python -m rejection_sampling_verification_spec_amd.build_lib`` (or
``__graft_entry__.build()``).  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "specverify.hip")
SOURCES = [SRC, os.path.join(HERE, "csrc", "gamma_policy.cpp")]
OUT = os.path.join(HERE, "libspecverify.so")
PROBE_SRC = os.path.join(HERE, "csrc", "stream_probe.hip")
PROBE_OUT = os.path.join(HERE, "libsvprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",          # every fused multiply-add is written out as fmaf
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = OUT, extra=()) -> str:
    """Builds libspecverify.so and the benchmark's streaming-read probe, libsvprobe.so."""
    for srcs, dst in ((SOURCES, out), ([PROBE_SRC], PROBE_OUT)):
        tmp = dst + ".tmp"
        cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *srcs]
        subprocess.run(cmd, check=True)
        os.replace(tmp, dst)
    return out


def assembly(out_dir: str) -> str:
    """Device assembly of the library (for reading the generated gfx950 code)."""
    os.makedirs(out_dir, exist_ok=True)
    s = os.path.join(out_dir, "specverify-gfx950.s")
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")], "--cuda-device-only", "-S",
           "-o", s, SRC]
    subprocess.run(cmd, check=True)
    return s


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
