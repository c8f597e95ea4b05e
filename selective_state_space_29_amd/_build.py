"""Builds the native parts of the package in-tree.

* ``libmamba_scan.so``: the HIP kernels and the C ABI (hipcc, gfx950 only). Packed-fp32 VALU
  instructions are disabled (``-target-feature -packed-fp32-ops``): the kernels' arithmetic is
  plain fp32 FMA/MUL plus the hardware transcendentals.
* ``gen/libssm_gen.so``: the seeded input generator (plain gcc).
* ``probe/libmscan_rates.so``: FMA and exp issue-rate microkernels the benchmark reports its
  rooflines against (not part of the scan library).
"""

from __future__ import annotations

import os
import subprocess

from . import gen as _gen

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmamba_scan.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(
        os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp"))
    )


def build_hip(out: str = LIB, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-o", tmp, os.path.join(CSRC, "mamba_scan.hip")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


RATES_SRC = os.path.join(HERE, "probe", "rates.hip")
RATES_LIB = os.path.join(HERE, "probe", "libmscan_rates.so")


def build_rates(out: str = RATES_LIB) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    subprocess.run([hipcc, *HIPCC_FLAGS, "-o", tmp, RATES_SRC], check=True)
    os.replace(tmp, out)
    return out


def build_all() -> None:
    build_hip()
    build_rates()
    _gen.build(force=True)
