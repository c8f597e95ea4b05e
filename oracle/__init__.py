"""fp64 CPU oracle of the selective-scan forward and backward passes (``scan_oracle.c``) and of the
block's upstream stages that produce the scan's inputs (``block_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU-baseline leg may use
it; the product path never does. It shares no code with the HIP library. Which passage of the
pages each step follows is stated in ``scan_oracle.c``.

Every function of the oracle is pinned by CPU tests against things other than itself
(brute-force sums, a closed form, the delta -> 0 limit, hand-computed L=1/L=2 cases, scipy's
``lfilter`` and numpy's ``cumsum`` special cases, invariants, and the pages' own einsum loop run
in torch fp64). One reading is not pinned by any page value: the exp branch taken when
``delta_softplus`` is false ("parity unpinned" beyond the text of the page that defines it).

The backward pass (``selective_scan_bwd``) is pinned by central finite differences of the forward
oracle and by torch's fp64 CPU autograd through an independent step-by-step formulation.

The upstream stages (``block_upstream``: causal depthwise convolution + SiLU, x projection, dt
projection, each output rounded once to bf16) are pinned against torch's fp64 ``conv1d`` and
numpy's ``convolve`` and ``matmul``, an impulse-response hand case, and their bf16 rounding
against torch's own fp32 -> bf16 conversion and hand-made ties.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "scan_oracle.c")
BLOCK_SOURCE = os.path.join(_HERE, "block_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, source=None, out: str = _LIB) -> str:
    """Compile the oracle with plain gcc: -O2, no fast-math, host libm. ``source``: one file or a
    list of files (default: both oracle sources)."""
    sources = [SOURCE, BLOCK_SOURCE] if source is None else (
        [source] if isinstance(source, str) else list(source))
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, *sources, "-lm"],
            check=True,
        )
        os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    f = lib.oracle_selective_scan
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] + [P] * 5 + [P] * 4 + [ctypes.c_int] + [
        P, ctypes.c_int64, P, P, ctypes.c_int]
    g = lib.oracle_selective_scan_ex
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] + [P] * 5 + [P] * 4 + [ctypes.c_int] * 2 + [
        P, ctypes.c_int64, P, P, ctypes.c_int]
    return lib


def _bind_bwd(lib):
    f = lib.oracle_selective_scan_bwd
    f.restype = ctypes.c_int
    P = ctypes.c_void_p
    f.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] + [P] * 5 + [P] * 4 + [ctypes.c_int] + [
        P] * 11 + [ctypes.c_int]
    g = lib.oracle_selective_scan_bwd_ex
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int] + [P] * 5 + [P] * 4 + [ctypes.c_int] * 2 + [
        P] * 11 + [ctypes.c_int]
    return lib


def _bind_block(lib):
    P = ctypes.c_void_p
    f = lib.oracle_block_upstream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int64] * 6 + [P] * 5 + [P] * 6 + [ctypes.c_int]
    g = lib.oracle_round_bf16
    g.restype = None
    g.argtypes = [P, P, ctypes.c_int64]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind_block(_bind_bwd(_bind(_LIB)))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _as(arr, kind):
    if arr is None:
        return None
    if kind == "in":
        a = np.ascontiguousarray(arr)
        if a.dtype not in (np.float32, np.uint16):
            raise TypeError(f"oracle inputs are fp32 or bf16 bit patterns (uint16), got {a.dtype}")
        return a
    a = np.ascontiguousarray(arr, dtype=np.float32)
    return a


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   h0=None, rows=None, nthreads=None, lib_path=None, zoh_b=False):
    """Reference scan in fp64. ``zoh_b``: B discretised by zero-order hold, (e^{dt A} - 1) / A * B
    (dt * B where A = 0), instead of the selective scan's dt * B.

    u, delta, z: (batch, dim, L); B, C: (batch, N, L), all fp32 or all bf16 bit patterns
    (numpy uint16). A: (dim, N) fp32; D, delta_bias: (dim,) fp32; h0: (batch, dim, N), widened to fp64.
    rows: optional flat row indices b*dim + d to compute (default: all, in order).
    Returns (y, last_state) as fp64 arrays of shape (nrows, L) and (nrows, N), reshaped to
    (batch, dim, L) / (batch, dim, N) when all rows are computed.
    """
    lib = _bind(lib_path) if lib_path else _load()
    u, delta, B, C = (_as(x, "in") for x in (u, delta, B, C))
    z = _as(z, "in")
    kinds = {x.dtype for x in (u, delta, B, C) + ((z,) if z is not None else ())}
    if len(kinds) != 1:
        raise TypeError("u, delta, z, B, C must share one storage dtype")
    in_dtype = 1 if kinds.pop() == np.uint16 else 0
    batch, dim, L = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta, z shapes differ")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L):
        raise ValueError("B, C must be (batch, N, L)")
    A = _as(A, "p")
    D = _as(D, "p")
    delta_bias = _as(delta_bias, "p")
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    if rows is None:
        nrows, rows_arr = batch * dim, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    y = np.empty((nrows, L), dtype=np.float64)
    ls = np.empty((nrows, N), dtype=np.float64)

    def ptr(a):
        return None if a is None else a.ctypes.data

    rc = lib.oracle_selective_scan_ex(
        batch, dim, L, N, in_dtype, ptr(u), ptr(delta), ptr(z), ptr(B), ptr(C), ptr(A), ptr(D),
        ptr(delta_bias), ptr(h0), int(bool(delta_softplus)), int(bool(zoh_b)), ptr(rows_arr), nrows,
        ptr(y), ptr(ls), int(nthreads or default_threads()),
    )
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan failed with {rc}")
    if rows is None:
        return y.reshape(batch, dim, L), ls.reshape(batch, dim, N)
    return y, ls


def selective_scan_bwd(u, delta, A, B, C, gy, D=None, z=None, delta_bias=None,
                       delta_softplus=False, h0=None, glast=None, nthreads=None, lib_path=None,
                       zoh_b=False):
    """Gradients of a loss with dLoss/dy = gy (batch, dim, L) and dLoss/dlast_state = glast
    (batch, dim, N) or None, in fp64. Inputs as for ``selective_scan`` (``zoh_b``: of the scan
    whose B is discretised by zero-order hold).

    Returns a dict: u, delta, z (batch, dim, L; z only when given), B, C (batch, N, L), A (dim, N),
    D, delta_bias (dim,) and h0 (batch, dim, N), all fp64.
    """
    lib = _bind_bwd(_bind(lib_path)) if lib_path else _load()
    u, delta, B, C = (_as(x, "in") for x in (u, delta, B, C))
    z = _as(z, "in")
    kinds = {x.dtype for x in (u, delta, B, C) + ((z,) if z is not None else ())}
    if len(kinds) != 1:
        raise TypeError("u, delta, z, B, C must share one storage dtype")
    in_dtype = 1 if kinds.pop() == np.uint16 else 0
    batch, dim, L = u.shape
    N = A.shape[1]
    A = _as(A, "p")
    D = _as(D, "p")
    delta_bias = _as(delta_bias, "p")
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    gy = np.ascontiguousarray(gy, dtype=np.float64)
    glast = None if glast is None else np.ascontiguousarray(glast, dtype=np.float64)
    if gy.shape != (batch, dim, L) or (glast is not None and glast.shape != (batch, dim, N)):
        raise ValueError("gy must be (batch, dim, L) and glast (batch, dim, N)")
    out = {k: np.zeros(shape, dtype=np.float64) for k, shape in (
        ("u", (batch, dim, L)), ("delta", (batch, dim, L)), ("z", (batch, dim, L)),
        ("B", (batch, N, L)), ("C", (batch, N, L)), ("A", (dim, N)), ("D", (dim,)),
        ("delta_bias", (dim,)), ("h0", (batch, dim, N)))}

    def ptr(a):
        return None if a is None else a.ctypes.data

    rc = lib.oracle_selective_scan_bwd_ex(
        batch, dim, L, N, in_dtype, ptr(u), ptr(delta), ptr(z), ptr(B), ptr(C), ptr(A), ptr(D),
        ptr(delta_bias), ptr(h0), int(bool(delta_softplus)), int(bool(zoh_b)), ptr(gy), ptr(glast),
        ptr(out["u"]), ptr(out["delta"]), ptr(out["z"]), ptr(out["B"]), ptr(out["C"]),
        ptr(out["A"]), ptr(out["D"]), ptr(out["delta_bias"]), ptr(out["h0"]),
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_selective_scan_bwd failed with {rc}")
    if z is None:
        del out["z"]
    return out


def round_bf16(values, lib_path=None) -> np.ndarray:
    """The oracle's rounding of fp64 values to bf16 (nearest, ties to even), as uint16 bits."""
    lib = _bind_block(ctypes.CDLL(lib_path)) if lib_path else _load()
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_round_bf16(v.ctypes.data, out.ctypes.data, v.size)
    return out


def block_upstream(x, conv_w, conv_b, w_x, w_dt, dstate, dt_rank, want_pre=False, nthreads=None,
                   lib_path=None):
    """The stages in front of the scan, in fp64 with bf16 storage between them.

    x: (batch, dim, L) bf16 bits (uint16); conv_w: (dim, d_conv) fp32; conv_b: (dim,) fp32 or None;
    w_x: (dt_rank + 2 dstate, dim) bf16 bits; w_dt: (dim, dt_rank) bf16 bits.
    Returns a dict with u (batch, dim, L), xdbl (batch, dt_rank + 2 dstate, L) and delta
    (batch, dim, L) as bf16 bits; with ``want_pre`` also u_pre, xdbl_pre, delta_pre: the fp64
    values before each rounding. The scan's B and C are ``xdbl[:, dt_rank:dt_rank + dstate]`` and
    ``xdbl[:, dt_rank + dstate:]``.
    """
    lib = _bind_block(ctypes.CDLL(lib_path)) if lib_path else _load()
    x = np.ascontiguousarray(x)
    w_x = np.ascontiguousarray(w_x)
    w_dt = np.ascontiguousarray(w_dt)
    for name, a in (("x", x), ("w_x", w_x), ("w_dt", w_dt)):
        if a.dtype != np.uint16:
            raise TypeError(f"{name} must hold bf16 bit patterns (uint16)")
    batch, dim, L = x.shape
    conv_w = np.ascontiguousarray(conv_w, dtype=np.float32)
    conv_b = None if conv_b is None else np.ascontiguousarray(conv_b, dtype=np.float32)
    d_conv = conv_w.shape[1]
    J = dt_rank + 2 * dstate
    if conv_w.shape[0] != dim or w_x.shape != (J, dim) or w_dt.shape != (dim, dt_rank):
        raise ValueError("weight shapes do not match x, dstate and dt_rank")
    out = {"u": np.empty((batch, dim, L), np.uint16), "xdbl": np.empty((batch, J, L), np.uint16),
           "delta": np.empty((batch, dim, L), np.uint16)}
    if want_pre:
        out.update({k + "_pre": np.empty(out[k].shape, np.float64) for k in ("u", "xdbl", "delta")})

    def ptr(a):
        return None if a is None else a.ctypes.data

    rc = lib.oracle_block_upstream(
        batch, dim, L, dstate, dt_rank, d_conv, ptr(x), ptr(conv_w), ptr(conv_b), ptr(w_x),
        ptr(w_dt), ptr(out["u"]), ptr(out["xdbl"]), ptr(out["delta"]), ptr(out.get("u_pre")),
        ptr(out.get("xdbl_pre")), ptr(out.get("delta_pre")), int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_block_upstream failed with {rc}")
    return out
