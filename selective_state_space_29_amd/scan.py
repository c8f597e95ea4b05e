"""Python binding of the selective-scan C ABI (argument marshalling only).

Every step of the scan runs in ``libmamba_scan.so``; this module only turns torch tensors into
device pointers, strides and flags, allocates the outputs with torch, and calls
``mamba_scan_fwd`` on torch's current HIP stream. There is no CPU fallback: without the built
library, or without a GPU, calls raise.

Signature and defaults follow ``selective_scan_ref(u, delta, A, B, C, D=None, delta_bias=None,
delta_softplus=False, return_last_state=False)`` of "Mamba代码实战…" §6, with the gate ``z`` of
§3.3 and an initial state ``h0`` (the state argument of the scan in "手把手用PyTorch实现Mamba的SSM层…"
§3.1). Inputs whose last stride is not 1 are made contiguous first (§4.1).
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmamba_scan.so")

F32, BF16 = 0, 1
DELTA_SOFTPLUS = 1 << 0
RETURN_LAST_STATE = 1 << 1
ZOH_B = 1 << 2
SAVE_CHECKPOINTS = 1 << 3
FORCE_GENERIC = 1 << 8
FORCE_TILED = 1 << 9
FORCE_LANES = 1 << 10
FORCE_CHUNKED = 1 << 11
FORCE_STEP = 1 << 12

_I64 = ctypes.c_int64
_P = ctypes.c_void_p


class Ptrs(ctypes.Structure):
    _fields_ = [("u", _P), ("delta", _P), ("z", _P), ("B", _P), ("C", _P), ("A", _P), ("D", _P),
                ("delta_bias", _P), ("h0", _P), ("y", _P), ("last_state", _P),
                ("workspace", _P), ("workspace_bytes", _I64)]


class Shape(ctypes.Structure):
    _fields_ = [("batch", _I64), ("dim", _I64), ("len", _I64), ("dstate", _I64)]


class Strides(ctypes.Structure):
    _fields_ = [("u", _I64 * 3), ("delta", _I64 * 3), ("z", _I64 * 3), ("B", _I64 * 3),
                ("C", _I64 * 3), ("y", _I64 * 3), ("h0", _I64 * 3), ("last_state", _I64 * 3),
                ("A", _I64 * 2), ("D", _I64), ("delta_bias", _I64)]


class BwdPtrs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias", "h0", "dy",
                                  "dlast_state", "du", "ddelta", "dz", "dB", "dC", "dA", "dD",
                                  "ddelta_bias", "dh0", "workspace")] + [("workspace_bytes", _I64),
                                                                          ("checkpoints", _P)]


class UpPtrs(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("x", "conv_w", "conv_b", "w_x", "w_dt", "u", "xdbl", "delta")]


class UpShape(ctypes.Structure):
    _fields_ = [(n, _I64) for n in ("batch", "dim", "len", "dstate", "dt_rank", "d_conv")]


class MambaScanError(RuntimeError):
    def __init__(self, code: int, msg: str, entry: str = "mamba_scan_fwd"):
        super().__init__(f"{entry} failed ({code}): {msg}")
        self.code = code
        self.entry = entry


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: the HIP extension is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.mamba_scan_fwd.restype = ctypes.c_int
    lib.mamba_scan_fwd.argtypes = [ctypes.POINTER(Ptrs), ctypes.POINTER(Shape),
                                   ctypes.POINTER(Strides), ctypes.c_int, ctypes.c_uint32, _P]
    lib.mamba_scan_fwd_kernel.restype = ctypes.c_int
    lib.mamba_scan_fwd_kernel.argtypes = [ctypes.POINTER(Ptrs), ctypes.POINTER(Shape),
                                          ctypes.POINTER(Strides), ctypes.c_int, ctypes.c_uint32]
    lib.mamba_scan_workspace_bytes.restype = _I64
    lib.mamba_scan_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, ctypes.c_uint32]
    lib.mamba_scan_strerror.restype = ctypes.c_char_p
    lib.mamba_scan_strerror.argtypes = [ctypes.c_int]
    lib.mamba_scan_abi_version.restype = ctypes.c_int
    lib.mamba_scan_abi_version.argtypes = []
    lib.mamba_scan_bwd.restype = ctypes.c_int
    lib.mamba_scan_bwd.argtypes = [ctypes.POINTER(BwdPtrs), ctypes.POINTER(Shape), ctypes.c_int,
                                   ctypes.c_uint32, _P]
    lib.mamba_scan_bwd_static.restype = ctypes.c_int
    lib.mamba_scan_bwd_static.argtypes = [ctypes.POINTER(BwdPtrs), ctypes.POINTER(Shape), ctypes.c_int,
                                          ctypes.c_uint32, _P]
    lib.mamba_scan_bwd_workspace_bytes.restype = _I64
    lib.mamba_scan_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Shape), ctypes.c_int, ctypes.c_uint32]
    lib.mamba_block_upstream.restype = ctypes.c_int
    lib.mamba_block_upstream.argtypes = [ctypes.POINTER(UpPtrs), ctypes.POINTER(UpShape), ctypes.c_int, _P]
    if path == LIB_PATH:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().mamba_scan_strerror(code).decode()


def _inner_contig(x):
    if x is not None and x.stride(-1) != 1:
        x = x.contiguous()
    return x


def _ptr(x):
    return None if x is None else x.data_ptr()


def _strides(x):
    """Element strides. A size-1 dimension's stride is never used and torch reports arbitrary
    values for it: report 1 for the innermost dimension and 0 for the others."""
    nd = len(x.shape)
    return [(1 if i == nd - 1 else 0) if n == 1 else s
            for i, (n, s) in enumerate(zip(x.shape, x.stride()))]


def _s3(x, fallback=(0, 0, 1)):
    return (_I64 * 3)(*(_strides(x) if x is not None else fallback))


KERNEL_NAMES = {0: "none", 1: "generic", 2: "tiled", 3: "lanes", 4: "chunked", 5: "step"}


def _fwd_args(u, delta, A, B, C, D, z, delta_bias, delta_softplus, return_last_state, h0, kernel, out,
              last_state_out, zoh_b, checkpoints_out, allocate=True):
    """Validate and marshal the forward's arguments: (ptrs, shape, strides, dtype, flags, y, ls, ws).
    With allocate=False no output or workspace is allocated (their pointers stay NULL unless
    given), for the kernel query."""
    lib = load_library()
    if u.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"u must be float32 or bfloat16, got {u.dtype}")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selective_scan_fn runs on the GPU only: inputs must be device tensors")
    for name, x in (("delta", delta), ("z", z), ("B", B), ("C", C)):
        if x is not None and (x.dtype != u.dtype or x.device != dev):
            raise TypeError(f"{name} must have u's dtype and device")
    for name, x in (("A", A), ("D", D), ("delta_bias", delta_bias), ("h0", h0)):
        if x is not None and x.device != dev:
            raise TypeError(f"{name} must be on u's device")
    u, delta, z, B, C = (_inner_contig(x) for x in (u, delta, z, B, C))
    A = _inner_contig(A.float())
    D = None if D is None else D.float()
    delta_bias = None if delta_bias is None else delta_bias.float()
    h0 = None if h0 is None else _inner_contig(h0.float())
    batch, dim, L = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape):
        raise ValueError("u, delta and z must have the same shape")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L):
        raise ValueError(f"B and C must be (batch, N, L) = {(batch, N, L)}")
    if A.shape != (dim, N):
        raise ValueError(f"A must be (dim, N) = {(dim, N)}")
    for name, x in (("D", D), ("delta_bias", delta_bias)):
        if x is not None and x.shape != (dim,):
            raise ValueError(f"{name} must be (dim,)")
    if h0 is not None and h0.shape != (batch, dim, N):
        raise ValueError("h0 must be (batch, dim, N)")

    y = out
    if y is None and allocate:
        y = torch.empty((batch, dim, L), dtype=torch.float32, device=dev)
    ls = None
    flags = (DELTA_SOFTPLUS if delta_softplus else 0) | (ZOH_B if zoh_b else 0)
    if return_last_state:
        ls = last_state_out
        if ls is None and allocate:
            ls = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
        flags |= RETURN_LAST_STATE
    forced = {None: 0, "generic": FORCE_GENERIC, "tiled": FORCE_TILED, "lanes": FORCE_LANES,
              "chunked": FORCE_CHUNKED, "step": FORCE_STEP}
    if kernel not in forced:
        raise ValueError("kernel must be None, 'generic', 'tiled', 'lanes', 'chunked' or 'step'")
    flags |= forced[kernel]

    shape = Shape(batch, dim, L, N)
    dtype = BF16 if u.dtype == torch.bfloat16 else F32
    if checkpoints_out is not None:
        _check_checkpoints(checkpoints_out, batch, dim, L, N, dev)
        flags |= SAVE_CHECKPOINTS
        ws, ws_bytes = checkpoints_out, checkpoints_out.numel() * 4
    else:
        ws_bytes = lib.mamba_scan_workspace_bytes(ctypes.byref(shape), dtype, flags)
        if ws_bytes < 0:
            _raise(int(ws_bytes), "mamba_scan_workspace_bytes")
        ws = torch.empty(int(ws_bytes), dtype=torch.uint8, device=dev) if (ws_bytes > 0 and allocate) else None

    st = Strides()
    st.u, st.delta, st.z = _s3(u), _s3(delta), _s3(z)
    st.B, st.C = _s3(B), _s3(C)
    st.y = _s3(y) if y is not None else (_I64 * 3)(dim * L, L, 1)
    st.h0, st.last_state = _s3(h0), _s3(ls)
    st.A = (_I64 * 2)(*_strides(A))
    st.D = _strides(D)[0] if D is not None else 1
    st.delta_bias = _strides(delta_bias)[0] if delta_bias is not None else 1
    ptrs = Ptrs(_ptr(u), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D),
                _ptr(delta_bias), _ptr(h0), _ptr(y), _ptr(ls), _ptr(ws), int(ws_bytes))
    keep = (u, delta, z, B, C, A, D, delta_bias, h0)  # the converted tensors must outlive the call
    return ptrs, shape, st, dtype, flags, y, ls, ws, keep


def _raise(rc, entry="mamba_scan_fwd"):
    """A library error code as an exception: ValueError (with the MambaScanError as its cause)
    for the codes that reject the arguments, MambaScanError itself for a refused launch."""
    err = MambaScanError(rc, strerror(rc), entry)
    if rc in (-1, -2, -3, -4, -5, -6, -8, -9, -10):
        raise ValueError(str(err)) from err
    raise err


def selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                      return_last_state=False, h0=None, *, kernel=None, out=None,
                      last_state_out=None, zoh_b=False, checkpoints_out=None):
    """y = selective_scan(...), fp32 (batch, dim, L); with ``return_last_state`` also the final
    state (batch, dim, N) fp32. ``zoh_b``: B discretised by zero-order hold,
    (e^{dt A} - 1) / A * B, instead of dt * B (forward only).

    u, delta, z: (batch, dim, L); B, C: (batch, N, L); one storage dtype for all five
    (torch.float32 or torch.bfloat16). A: (dim, N); D, delta_bias: (dim,); h0: (batch, dim, N);
    these are taken in fp32. ``kernel``: None (library picks), "generic", "tiled", "lanes" (a
    16-lane row per channel: one state per lane at 16 states, 2 or 4 at 32 or 64), "chunked"
    (parallel along the sequence: a wave per channel scanning 4 runs of each 64-step chunk; 16
    states) or "step" (short calls such as decode, at most 64 steps; 16 states).
    ``checkpoints_out``: a contiguous fp32 (batch, dim, ceil(L/16), N) tensor that receives the
    state before every 16-step segment, for ``selective_scan_bwd(checkpoints=...)``
    (lane-per-state and chunked kernels only).
    """
    lib = load_library()
    ptrs, shape, st, dtype, flags, y, ls, ws, keep = _fwd_args(
        u, delta, A, B, C, D, z, delta_bias, delta_softplus, return_last_state, h0, kernel, out,
        last_state_out, zoh_b, checkpoints_out)
    dev = u.device
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.mamba_scan_fwd(ctypes.byref(ptrs), ctypes.byref(shape), ctypes.byref(st),
                                dtype, flags, stream)
    del keep
    if rc != 0:
        _raise(rc)
    if ws is not None and checkpoints_out is None:
        ws.record_stream(torch.cuda.current_stream(dev))
    return (y, ls) if return_last_state else y


def forward_kernel(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   return_last_state=False, h0=None, *, kernel=None, out=None, last_state_out=None,
                   zoh_b=False, checkpoints_out=None):
    """Name of the kernel ``selective_scan_fn`` would run with these arguments ("generic",
    "tiled", "lanes", "chunked" or "step"), from the library's own choice (``mamba_scan_fwd_kernel``);
    raises as the call would for arguments it rejects. Launches nothing."""
    lib = load_library()
    ptrs, shape, st, dtype, flags, _, _, _, keep = _fwd_args(
        u, delta, A, B, C, D, z, delta_bias, delta_softplus, return_last_state, h0, kernel, out,
        last_state_out, zoh_b, checkpoints_out, allocate=False)
    if ptrs.y is None:
        ptrs.y = 1 << 62  # any non-NULL address outside the inputs: compared, never dereferenced
    if return_last_state and ptrs.last_state is None:
        ptrs.last_state = (1 << 62) + (1 << 50)
    with torch.cuda.device(u.device):
        rc = lib.mamba_scan_fwd_kernel(ctypes.byref(ptrs), ctypes.byref(shape), ctypes.byref(st), dtype, flags)
    del keep
    if rc < 0:
        _raise(rc, "mamba_scan_fwd_kernel")
    return KERNEL_NAMES[rc]


def checkpoint_shape(batch, dim, L, N):
    """Shape of the saved segment states: (batch, dim, ceil(L/16), N)."""
    return (batch, dim, (L + 15) // 16, N)


def _check_checkpoints(ck, batch, dim, L, N, dev):
    if (ck.dtype != torch.float32 or ck.device != dev or tuple(ck.shape) != checkpoint_shape(batch, dim, L, N)
            or not ck.is_contiguous()):
        raise ValueError(f"checkpoints must be a contiguous float32 tensor of shape "
                         f"{checkpoint_shape(batch, dim, L, N)} on u's device")


def selective_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, delta_softplus=False,
                       h0=None, dlast_state=None, want_dh0=True, checkpoints=None, static_scratch=False,
                       kernel=None, zoh_b=False):
    """Gradients of the scan (``mamba_scan_bwd``) for incoming gradients dy (batch, dim, L) and,
    optionally, dlast_state (batch, dim, N). Inputs as for ``selective_scan_fn``; all tensors are
    made contiguous first. Returns a dict of fp32 gradients: u, delta, B, C, A, and z, D,
    delta_bias when given, h0 when ``want_dh0`` (the gradient of the initial state, which is zero
    when h0 is None). ``checkpoints``: the segment states that ``selective_scan_fn(checkpoints_out=)``
    saved for the same inputs; the backward then does not recompute them. ``static_scratch``: call
    ``mamba_scan_bwd_static``, whose workspace is the library's own static per-device buffer (no
    workspace is allocated here; calls overlapping in time on one GPU must not be made).
    ``kernel``: None (the library's choice: the lane-per-state kernel at 16, 32 and 64 states,
    else the segment-tiled one), "lanes" or "tiled" (forced; an error where it cannot run).
    ``zoh_b``: the gradients of the forward with B discretised by zero-order hold (either
    kernel; ``checkpoints`` then come from a zero-order-hold forward).
    """
    lib = load_library()
    if u.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"u must be float32 or bfloat16, got {u.dtype}")
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("selective_scan_bwd runs on the GPU only: inputs must be device tensors")
    for name, x in (("delta", delta), ("z", z), ("B", B), ("C", C)):
        if x is not None and (x.dtype != u.dtype or x.device != dev):
            raise TypeError(f"{name} must have u's dtype and device")
    u, delta, z, B, C = (None if x is None else x.contiguous() for x in (u, delta, z, B, C))
    A = A.float().contiguous()
    D = None if D is None else D.float().contiguous()
    delta_bias = None if delta_bias is None else delta_bias.float().contiguous()
    h0 = None if h0 is None else h0.float().contiguous()
    dy = dy.float().contiguous()
    dlast_state = None if dlast_state is None else dlast_state.float().contiguous()
    batch, dim, L = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or (z is not None and z.shape != u.shape) or dy.shape != u.shape:
        raise ValueError("u, delta, z and dy must have the same shape")
    if B.shape != (batch, N, L) or C.shape != (batch, N, L) or A.shape != (dim, N):
        raise ValueError("B, C must be (batch, N, L) and A (dim, N)")
    for name, x, shape in (("D", D, (dim,)), ("delta_bias", delta_bias, (dim,)),
                           ("h0", h0, (batch, dim, N)), ("dlast_state", dlast_state, (batch, dim, N))):
        if x is not None and tuple(x.shape) != shape:
            raise ValueError(f"{name} must be {shape}")

    f32 = dict(dtype=torch.float32, device=dev)
    g = {"u": torch.empty((batch, dim, L), **f32), "delta": torch.empty((batch, dim, L), **f32),
         "B": torch.empty((batch, N, L), **f32), "C": torch.empty((batch, N, L), **f32),
         "A": torch.empty((dim, N), **f32)}
    if z is not None:
        g["z"] = torch.empty((batch, dim, L), **f32)
    if D is not None:
        g["D"] = torch.empty((dim,), **f32)
    if delta_bias is not None:
        g["delta_bias"] = torch.empty((dim,), **f32)
    if want_dh0:
        g["h0"] = torch.empty((batch, dim, N), **f32)
    shape = Shape(batch, dim, L, N)
    dtype = BF16 if u.dtype == torch.bfloat16 else F32
    flags = (DELTA_SOFTPLUS if delta_softplus else 0) | (ZOH_B if zoh_b else 0)
    if kernel not in (None, "lanes", "tiled"):
        raise ValueError(f"unknown backward kernel {kernel!r}: None, 'lanes' or 'tiled'")
    flags |= {None: 0, "lanes": FORCE_LANES, "tiled": FORCE_TILED}[kernel]
    if static_scratch:
        ws, ws_bytes = None, 0
    else:
        ws_bytes = lib.mamba_scan_bwd_workspace_bytes(
            ctypes.byref(shape), dtype, flags | (SAVE_CHECKPOINTS if checkpoints is not None else 0))
        if ws_bytes < 0:
            _raise(int(ws_bytes), "mamba_scan_bwd_workspace_bytes")
        ws = torch.empty(int(ws_bytes), dtype=torch.uint8, device=dev)
    ptrs = BwdPtrs(_ptr(u), _ptr(delta), _ptr(z), _ptr(B), _ptr(C), _ptr(A), _ptr(D), _ptr(delta_bias),
                   _ptr(h0), _ptr(dy), _ptr(dlast_state), _ptr(g["u"]), _ptr(g["delta"]), _ptr(g.get("z")),
                   _ptr(g["B"]), _ptr(g["C"]), _ptr(g["A"]), _ptr(g.get("D")), _ptr(g.get("delta_bias")),
                   _ptr(g.get("h0")), _ptr(ws), int(ws_bytes))
    if checkpoints is not None:
        _check_checkpoints(checkpoints, batch, dim, L, N, dev)
        ptrs.checkpoints = _ptr(checkpoints)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        entry = lib.mamba_scan_bwd_static if static_scratch else lib.mamba_scan_bwd
        rc = entry(ctypes.byref(ptrs), ctypes.byref(shape), dtype, flags, stream)
    if rc != 0:
        _raise(rc, "mamba_scan_bwd_static" if static_scratch else "mamba_scan_bwd")
    if ws is not None:
        ws.record_stream(torch.cuda.current_stream(dev))
    return g


class SelectiveScan(torch.autograd.Function):
    """y (and last_state) = selective_scan(...) with a backward pass through ``mamba_scan_bwd``.

    The inputs are saved, and, where the lane-per-state or chunked forward runs (16, 32 or 64
    states), the state before every 16-step segment; the backward recomputes the states inside each segment
    from there ("手把手用PyTorch实现Mamba的SSM层…" §4.2), or from the start without them.
    Gradients come back in each input's dtype.
    """

    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, zoh_b):
        kw = dict(D=D, z=z, delta_bias=delta_bias, delta_softplus=delta_softplus, return_last_state=True, h0=h0,
                  zoh_b=zoh_b)
        ck = None
        if A.shape[1] in (16, 32, 64) and u.dtype in (torch.float32, torch.bfloat16):
            ck = torch.empty(checkpoint_shape(*u.shape, A.shape[1]), dtype=torch.float32, device=u.device)
            try:
                y, ls = selective_scan_fn(u, delta, A, B, C, checkpoints_out=ck, **kw)
            except ValueError as e:
                if not isinstance(e.__cause__, MambaScanError) or e.__cause__.code != -8:
                    raise
                ck = None  # shape outside the lane-per-state kernels: no saved states
        if ck is None:
            y, ls = selective_scan_fn(u, delta, A, B, C, **kw)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0, ck)
        ctx.delta_softplus = delta_softplus
        ctx.zoh_b = zoh_b
        return y, ls

    @staticmethod
    def backward(ctx, gy, gls):
        u, delta, A, B, C, D, z, delta_bias, h0, ck = ctx.saved_tensors
        if gy is None:
            gy = torch.zeros(u.shape, dtype=torch.float32, device=u.device)
        g = selective_scan_bwd(u, delta, A, B, C, gy, D=D, z=z, delta_bias=delta_bias,
                               delta_softplus=ctx.delta_softplus, h0=h0, dlast_state=gls,
                               want_dh0=h0 is not None and ctx.needs_input_grad[8], checkpoints=ck,
                               zoh_b=ctx.zoh_b)

        def cast(name, like):
            return None if like is None or name not in g else g[name].to(like.dtype)

        return (cast("u", u), cast("delta", delta), cast("A", A), cast("B", B), cast("C", C),
                cast("D", D), cast("z", z), cast("delta_bias", delta_bias), cast("h0", h0), None, None)


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                   return_last_state=False, h0=None, zoh_b=False):
    """Differentiable form of ``selective_scan_fn`` (torch autograd through the HIP backward).
    When no gradient can flow (grad mode off, or no input requires one) it is the plain forward:
    no states are saved for a backward that will not run."""
    inputs = (u, delta, A, B, C, D, z, delta_bias, h0)
    if not (torch.is_grad_enabled() and any(t is not None and t.requires_grad for t in inputs)):
        return selective_scan_fn(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias,
                                 delta_softplus=delta_softplus, return_last_state=return_last_state,
                                 h0=h0, zoh_b=zoh_b)
    y, ls = SelectiveScan.apply(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, zoh_b)
    return (y, ls) if return_last_state else y


def block_upstream(x, conv_w, conv_b, w_x, w_dt, dstate, dt_rank, out=None):
    """The stages in front of the scan (``mamba_block_upstream``): causal depthwise conv1d + SiLU,
    x_proj, dt_proj, each output rounded to bf16.

    x: (batch, dim, L) bf16; conv_w: (dim, d_conv) fp32 (a Conv1d weight (dim, 1, d_conv) may be
    passed); conv_b: (dim,) fp32 or None; w_x: (dt_rank + 2 dstate, dim) bf16; w_dt: (dim, dt_rank)
    bf16. Returns (u, xdbl, delta), bf16; the scan's B and C are views of xdbl (see
    :func:`split_xdbl`). ``out`` = optional preallocated (u, xdbl, delta).
    """
    lib = load_library()
    if conv_w.dim() == 3:
        conv_w = conv_w.reshape(conv_w.shape[0], conv_w.shape[2])
    x, conv_w, w_x, w_dt = (t.contiguous() for t in (x, conv_w, w_x, w_dt))
    conv_b = None if conv_b is None else conv_b.contiguous()
    for name, t, dt in (("x", x, torch.bfloat16), ("w_x", w_x, torch.bfloat16), ("w_dt", w_dt, torch.bfloat16),
                        ("conv_w", conv_w, torch.float32)) + ((("conv_b", conv_b, torch.float32),) if conv_b is not None else ()):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if t.device != x.device or not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU of x")
    batch, dim, L = x.shape
    J = dt_rank + 2 * dstate
    if out is None:
        u = torch.empty_like(x)
        xdbl = torch.empty((batch, J, L), dtype=torch.bfloat16, device=x.device)
        delta = torch.empty_like(x)
    else:
        u, xdbl, delta = out
    ptrs = UpPtrs(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(w_x), _ptr(w_dt), _ptr(u), _ptr(xdbl), _ptr(delta))
    shape = UpShape(batch, dim, L, dstate, dt_rank, conv_w.shape[1])
    with torch.cuda.device(x.device):
        rc = lib.mamba_block_upstream(ctypes.byref(ptrs), ctypes.byref(shape), BF16,
                                      torch.cuda.current_stream(x.device).cuda_stream)
    if rc != 0:
        _raise(rc, "mamba_block_upstream")
    return u, xdbl, delta


def split_xdbl(xdbl, dt_rank, dstate):
    """(dt rows, B, C) as views of x_dbl, in the split order dt_rank, dstate, dstate."""
    return xdbl[:, :dt_rank], xdbl[:, dt_rank:dt_rank + dstate], xdbl[:, dt_rank + dstate:]


def block_ssm(x, conv_w, conv_b, w_x, w_dt, dt_bias, A, D=None, z=None, return_last_state=False, h0=None):
    """The selective-SSM part of a Mamba block: :func:`block_upstream` then the scan with
    delta_bias = dt_proj's bias and softplus on, B and C read in place from x_dbl."""
    dstate = A.shape[1]
    dt_rank = w_dt.shape[1]
    u, xdbl, delta = block_upstream(x, conv_w, conv_b, w_x, w_dt, dstate, dt_rank)
    _, B, C = split_xdbl(xdbl, dt_rank, dstate)
    return selective_scan_fn(u, delta, A, B, C, D=D, z=z, delta_bias=dt_bias, delta_softplus=True,
                             return_last_state=return_last_state, h0=h0)
