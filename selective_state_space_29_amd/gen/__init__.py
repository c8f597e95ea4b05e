"""Seeded, counter-based input generator (SplitMix64 words, Box-Muller normals).

The definitions are in ``gen.c``. This module only wraps them: it holds none of the scan's
arithmetic, and both the HIP path and the fp64 oracle are fed from it. Value ``i`` of a stream is
a pure function of ``(seed, stream, i)``, so any slice of a tensor (one row of a 3.3 GB input,
say) can be regenerated alone, bit-identical to the same slice of the whole tensor.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libssm_gen.so")
_lib = None

NORMAL, UNIFORM = 0, 1
_OUT_KIND = {"f32": 0, "bf16": 1, "f64": 2}
_NP_DTYPE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}


def build(force: bool = True) -> str:
    """Compile gen.c into libssm_gen.so next to it (plain gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.ssm_gen_fill.restype = ctypes.c_int
        lib.ssm_gen_fill.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.ssm_gen_words.restype = None
        lib.ssm_gen_words.argtypes = [
            ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
        ]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _fill(seed, stream, dist, lo, hi, shape, dtype, offset):
    if dtype not in _OUT_KIND:
        raise ValueError(f"dtype must be one of {sorted(_OUT_KIND)}, got {dtype!r}")
    out = np.empty(shape, dtype=_NP_DTYPE[dtype])
    rc = _load().ssm_gen_fill(
        int(seed), int(stream), dist, float(lo), float(hi), int(offset), int(out.size),
        _OUT_KIND[dtype], out.ctypes.data, _threads(),
    )
    if rc != 0:
        raise ValueError("ssm_gen_fill rejected its arguments")
    return out


def normal(seed: int, stream: int, shape, dtype: str = "f32", offset: int = 0) -> np.ndarray:
    """N(0,1) values ``offset .. offset+prod(shape)-1`` of stream ``(seed, stream)``."""
    return _fill(seed, stream, NORMAL, 0.0, 0.0, shape, dtype, offset)


def uniform(seed: int, stream: int, shape, lo: float, hi: float, dtype: str = "f32",
            offset: int = 0) -> np.ndarray:
    """U[lo, hi) values ``offset .. offset+prod(shape)-1`` of stream ``(seed, stream)``."""
    return _fill(seed, stream, UNIFORM, lo, hi, shape, dtype, offset)


def words(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """Raw SplitMix64 words of a stream (used to pin the stream definition)."""
    out = np.empty(count, dtype=np.uint64)
    _load().ssm_gen_words(int(seed), int(stream), int(offset), int(count), out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly (the 16 bits become the high half)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
