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
HEADER = os.path.join(os.path.dirname(HERE), "include", "mamba_scan.h")
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


def units():
    """Translation units: the C-ABI entry points and one per kernel family."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_hip(out: str = LIB, extra=(), jobs=None, incremental=False) -> str:
    """Compile every translation unit to an object in parallel, then link the shared library.
    ``incremental``: skip units whose object is newer than every file its last compile read
    (for development; a plain build compiles everything)."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]

    def deps_of(obj, src):
        """The files a unit was built from, from the dependency list its last compile wrote."""
        try:
            text = open(obj + ".d").read().replace("\\\n", " ")
        except OSError:
            return None
        files = text.split(":", 1)[1].split() if ":" in text else []
        return [f for f in files if os.path.exists(f)] or None

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src)[:-4] + ".o")
        if incremental and os.path.exists(obj):
            deps = deps_of(obj, src)
            if deps and max(os.path.getmtime(f) for f in deps + [src]) < os.path.getmtime(obj):
                return obj
        subprocess.run([hipcc, *compile_flags, *extra, "-MMD", "-MF", obj + ".d", "-c", "-o", obj, src],
                       check=True)
        return obj

    srcs = units()
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
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
