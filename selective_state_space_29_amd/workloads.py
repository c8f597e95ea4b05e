"""The five synthetic selective-scan workloads and their seeded inputs.

Each workload fixes shapes, storage dtype, value distributions and flags; inputs come from the
counter-based generator in :mod:`selective_state_space_29_amd.gen` with seed ``29000 + id`` and one
stream per tensor (u=1, delta=2, z=3, B=4, C=5, D=6, delta_bias=7). ``A[d, n] = -(n + 1)`` is
written exactly (the mamba-minimal initialisation ``A_log = log(1..N)``, ``A = -exp(A_log)``, from
the page "告别'炼丹'：从Mamba-minimal入手…", section 1.1, without the rounding of exp(log)).

No workload stands for a dataset: the pages' DNA and text inputs are replaced by N(0,1) tensors of
the same shapes. This module holds no scan arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import gen

STREAM = {"u": 1, "delta": 2, "z": 3, "B": 4, "C": 5, "D": 6, "delta_bias": 7,
          "x": 8, "conv_w": 9, "conv_b": 10, "w_x": 11, "w_dt": 12}


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    dtype: str  # storage dtype of u, delta, z, B, C: "f32" or "bf16"
    has_z: bool
    bias_dist: str  # "normal" or "u41" (U(-4,-1))
    d_dist: str  # "normal" or "ones"
    softplus: bool = True
    last_state: bool = True
    note: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 29000 + self.wid

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen * self.dstate

    @property
    def rows(self) -> int:
        return self.batch * self.dim

    def algorithmic_bytes(self) -> int:
        """Bytes the path must move at least once: inputs read once, outputs written once."""
        es = 2 if self.dtype == "bf16" else 4
        b, d, n, l = self.batch, self.dim, self.dstate, self.seqlen
        rd = (2 + int(self.has_z)) * b * d * l * es  # u, delta, z
        rd += 2 * b * n * l * es  # B, C
        rd += d * n * 4 + 2 * d * 4  # A, D, delta_bias (fp32)
        wr = b * d * l * 4 + (b * d * n * 4 if self.last_state else 0)  # y, last_state (fp32)
        return rd + wr


WORKLOADS = {
    1: Workload(1, "tiny-fp32", 4, 16, 32, 64, "f32", False, "normal", "normal",
                note="the page 'Mamba代码实战…' section 2.1 parameter set"),
    2: Workload(2, "mamba-minimal-fp32", 32, 128, 16, 256, "f32", True, "u41", "normal",
                note="(32, 256, 128) toy with d_state 16, the mamba-minimal benchmark shape"),
    3: Workload(3, "mamba130m-layer-bf16", 8, 1536, 16, 2048, "bf16", True, "u41", "ones",
                note="Mamba-130m mixer: d_model 768, expand 2, d_state 16, L 2048"),
    4: Workload(4, "genomic-100k-bf16", 4, 1024, 16, 100000, "bf16", True, "u41", "ones",
                note="d_model 512, expand 2, L = 100000 DNA-length sequences"),
    5: Workload(5, "wide-state-bf16", 4, 4096, 64, 16384, "bf16", True, "u41", "normal",
                note="d_model 2048, expand 2, d_state 64, L 16384"),
}


def a_matrix(dim: int, dstate: int) -> np.ndarray:
    """A[d, n] = -(n + 1), fp32, exactly."""
    return np.tile(-(np.arange(dstate, dtype=np.float32) + 1.0), (dim, 1))  # C-contiguous


def _vec(w: Workload, which: str, dist: str) -> np.ndarray:
    if dist == "normal":
        return gen.normal(w.seed, STREAM[which], (w.dim,), "f32")
    if dist == "u41":
        return gen.uniform(w.seed, STREAM[which], (w.dim,), -4.0, -1.0, "f32")
    if dist == "ones":
        return np.ones(w.dim, dtype=np.float32)
    raise ValueError(dist)


def make_params(w: Workload) -> dict:
    """The per-channel parameters A (D,N), D (D), delta_bias (D), all fp32."""
    return {
        "A": a_matrix(w.dim, w.dstate),
        "D": _vec(w, "D", w.d_dist),
        "delta_bias": _vec(w, "delta_bias", w.bias_dist),
    }


def make_bc(w: Workload, batches=None) -> dict:
    """B and C, (batch, N, L) in the workload's storage dtype; optionally only some batches."""
    out = {}
    nl = w.dstate * w.seqlen
    for key in ("B", "C"):
        if batches is None:
            out[key] = gen.normal(w.seed, STREAM[key], (w.batch, w.dstate, w.seqlen), w.dtype)
        else:
            out[key] = np.stack(
                [gen.normal(w.seed, STREAM[key], (w.dstate, w.seqlen), w.dtype, offset=b * nl)
                 for b in batches]
            )
    return out


def make_inputs(w: Workload) -> dict:
    """Every input tensor of the workload, full size, contiguous, as numpy arrays."""
    shp = (w.batch, w.dim, w.seqlen)
    out = {
        "u": gen.normal(w.seed, STREAM["u"], shp, w.dtype),
        "delta": gen.normal(w.seed, STREAM["delta"], shp, w.dtype),
        "z": gen.normal(w.seed, STREAM["z"], shp, w.dtype) if w.has_z else None,
    }
    out.update(make_bc(w))
    out.update(make_params(w))
    return out


def make_row_inputs(w: Workload, rows) -> dict:
    """Inputs restricted to the listed flat rows ``b * dim + d``, one independent single-channel
    problem per row: entry ``i`` of u/delta/z (nrows, 1, L), of B/C (nrows, N, L) and of
    A (nrows, N), D and delta_bias (nrows,) is row ``rows[i]``'s data. The slices are
    bit-identical to the same rows of :func:`make_inputs` (the generator is counter-based)."""
    rows = [int(r) for r in rows]
    L = w.seqlen
    full = make_params(w)
    res = {"u": [], "delta": [], "z": [] if w.has_z else None}
    for r in rows:
        for key in ("u", "delta") + (("z",) if w.has_z else ()):
            res[key].append(gen.normal(w.seed, STREAM[key], (1, L), w.dtype, offset=r * L))
    for key in ("u", "delta") + (("z",) if w.has_z else ()):
        res[key] = np.stack(res[key])
    bc = make_bc(w, batches=[r // w.dim for r in rows])
    res.update(bc)
    ds = [r % w.dim for r in rows]
    res["A"] = np.ascontiguousarray(full["A"][ds])
    res["D"] = np.ascontiguousarray(full["D"][ds])
    res["delta_bias"] = np.ascontiguousarray(full["delta_bias"][ds])
    return res


# ---------------------------------------------------------------------------------------------
# The stages in front of the scan (convolution + SiLU, x projection, dt projection).


@dataclass(frozen=True)
class UpstreamWorkload:
    """Shapes of the block's upstream stages: x (batch, dim, L) bf16 in; u, delta (batch, dim, L)
    and x_dbl (batch, dt_rank + 2 dstate, L) bf16 out. Seed ``29100 + id``."""

    wid: int
    name: str
    batch: int
    dim: int
    dstate: int
    dt_rank: int
    seqlen: int
    d_conv: int = 4
    note: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 29100 + self.wid

    @property
    def proj_rows(self) -> int:
        return self.dt_rank + 2 * self.dstate

    def algorithmic_bytes(self) -> int:
        """x read once; u, x_dbl, delta written once; the weights read once."""
        b, d, l, j = self.batch, self.dim, self.seqlen, self.proj_rows
        rd = b * d * l * 2 + d * self.d_conv * 4 + d * 4 + j * d * 2 + d * self.dt_rank * 2
        wr = 2 * b * d * l * 2 + b * j * l * 2
        return rd + wr

    def flops(self) -> int:
        """Multiply-adds of the two projections, as 2 flops each (the convolution is not counted)."""
        b, d, l = self.batch, self.dim, self.seqlen
        return 2 * b * l * d * (self.proj_rows + self.dt_rank)


UPSTREAM = {
    1: UpstreamWorkload(1, "upstream-small", 2, 192, 16, 8, 200,
                        note="ragged: 192 channels, 200 steps, dt_rank 8"),
    2: UpstreamWorkload(2, "mamba130m-upstream", 8, 1536, 16, 48, 2048,
                        note="Mamba-130m: d_inner 1536, d_state 16, dt_rank 48 = 768 / 16, "
                             "d_conv 4, L 2048; produces the scan inputs of the layer workload"),
}


def make_upstream_inputs(w: UpstreamWorkload) -> dict:
    """x ~ N(0, 1) in bf16, and weights drawn as PyTorch initialises the layers the pages build:
    Conv1d(dim, dim, d_conv, groups=dim) weight and bias U(-1/sqrt(d_conv), 1/sqrt(d_conv)) (fp32),
    Linear(dim, dt_rank + 2 dstate) weight U(-1/sqrt(dim), 1/sqrt(dim)) and Linear(dt_rank, dim)
    weight U(-1/sqrt(dt_rank), 1/sqrt(dt_rank)) (bf16)."""
    kc = 1.0 / np.sqrt(w.d_conv)
    kx = 1.0 / np.sqrt(w.dim)
    kt = 1.0 / np.sqrt(w.dt_rank)
    return {
        "x": gen.normal(w.seed, STREAM["x"], (w.batch, w.dim, w.seqlen), "bf16"),
        "conv_w": gen.uniform(w.seed, STREAM["conv_w"], (w.dim, w.d_conv), -kc, kc, "f32"),
        "conv_b": gen.uniform(w.seed, STREAM["conv_b"], (w.dim,), -kc, kc, "f32"),
        "w_x": gen.uniform(w.seed, STREAM["w_x"], (w.proj_rows, w.dim), -kx, kx, "bf16"),
        "w_dt": gen.uniform(w.seed, STREAM["w_dt"], (w.dim, w.dt_rank), -kt, kt, "bf16"),
    }


def make_upstream_case(seed: int, batch: int, dim: int, dstate: int, dt_rank: int, seqlen: int,
                       d_conv: int = 4, bias: bool = True) -> dict:
    """An ad-hoc upstream case with the same distributions (for tests of odd shapes)."""
    w = UpstreamWorkload(seed - 29100, "case", batch, dim, dstate, dt_rank, seqlen, d_conv)
    x = make_upstream_inputs(w)
    if not bias:
        x["conv_b"] = None
    return x
