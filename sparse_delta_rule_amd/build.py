"""Build libsdm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m sparse_delta_rule_amd.build

The library is built in-tree, next to this file, from csrc/*.hip; then the
plain C example caller in examples/ is compiled against it, and the reference
access patterns that the benchmark measures the rows' ceiling with
(ceiling/*.hip) are built into libsdm_ceiling.so.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsdm.so")
CEILING_LIB = os.path.join(HERE, "libsdm_ceiling.so")
ARCH = os.environ.get("SDM_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",  # every fused multiply-add in the kernels is written out
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


EXAMPLE_SRC = os.path.join(HERE, "examples", "sdm_example.c")
EXAMPLE = os.path.join(HERE, "examples", "sdm_example")


def build_example(verbose: bool = False) -> str:
    """The plain C example caller (examples/sdm_example.c), linked against the
    in-tree libsdm.so (found next to the examples folder at run time) and the HIP
    runtime."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = os.environ.get("CC", "gcc")
    tmp = EXAMPLE + ".tmp"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
           "-I", os.path.join(ROOT, "include"), "-o", tmp, EXAMPLE_SRC, "-L", HERE, "-lsdm",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/..",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"{cc} failed ({r.returncode}) building {EXAMPLE}")
    os.replace(tmp, EXAMPLE)
    return EXAMPLE


def _hipcc(out: str, srcs: list, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {out}")
    os.replace(tmp, out)
    return out


def build_ceiling(verbose: bool = False) -> str:
    return _hipcc(CEILING_LIB, sorted(glob.glob(os.path.join(HERE, "ceiling", "*.hip"))), verbose)


def build(verbose: bool = False) -> str:
    _hipcc(LIB, sources(), verbose)
    build_example(verbose)
    build_ceiling(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
