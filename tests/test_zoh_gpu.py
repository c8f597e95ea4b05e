"""GPU parity of the zero-order-hold B discretisation (MAMBA_SCAN_ZOH_B) against the fp64 oracle
with ``zoh_b=True``, for the lane-per-state (16, 32, 64 states), chunked, tiled and generic
kernels. Bars as
for the Euler scan: max|g - r| / (1 + |r|) <= 1e-4 for fp32 inputs, <= 2e-3 for bf16 inputs (the
GPU's coefficient (e^{dt A} - 1) / A is within 2^-20 relative of the exact one, see zoh_coef_f
and zoh_coef2_f)."""

import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
from selective_state_space_29_amd import scan, workloads

pytestmark = pytest.mark.gpu


def _run(x, kernel=None, softplus=True, h0=None, zoh=True):
    g = {k: gu.to_dev(v) if isinstance(v, np.ndarray) else v for k, v in x.items()}
    y, ls = scan.selective_scan_fn(g["u"], g["delta"], g["A"], g["B"], g["C"], D=g.get("D"), z=g.get("z"),
                                   delta_bias=g.get("delta_bias"), delta_softplus=softplus,
                                   return_last_state=True, kernel=kernel, zoh_b=zoh,
                                   h0=None if h0 is None else gu.to_dev(h0.astype(np.float32)))
    torch.cuda.synchronize()
    return y.cpu().numpy(), ls.cpu().numpy()


def _check(x, tol, kernel=None, softplus=True, h0=None):
    yg, lg = _run(x, kernel, softplus, h0)
    yr, lr = oracle.selective_scan(x["u"], x["delta"], x["A"], x["B"], x["C"], D=x.get("D"), z=x.get("z"),
                                   delta_bias=x.get("delta_bias"), delta_softplus=softplus, zoh_b=True,
                                   h0=None if h0 is None else h0.astype(np.float32).astype(np.float64))
    ey, el = gu.rel_err(yg, yr), gu.rel_err(lg, lr)
    print(f"  y {ey:.2e} last_state {el:.2e}", flush=True)
    assert np.all(np.isfinite(yg))
    assert ey <= tol and el <= tol, (ey, el)


@pytest.mark.parametrize("wid,kernel", [(1, None), (2, None), (3, None), (3, "tiled")])
def test_zoh_workload_parity(wid, kernel):
    """Default: the lane-per-state kernels (32 states in workload 1, 16 in 2 and 3)."""
    w = workloads.WORKLOADS[wid]
    print(f"zoh parity, workload {wid}: {w.name}, kernel {kernel}", flush=True)
    _check(workloads.make_inputs(w), 1e-4 if w.dtype == "f32" else 2e-3, kernel=kernel)


EDGE = [
    # (batch, dim, N, L, dtype, a_kind, kernel, h0)
    (2, 64, 16, 64, "f32", "mamba", "tiled", False),
    (2, 80, 16, 36, "bf16", "rand", "tiled", True),
    (1, 70, 4, 40, "f32", "zeros_mixed", "tiled", False),
    (2, 64, 12, 100, "f32", "tiny", "tiled", False),
    (1, 64, 32, 64, "bf16", "mamba", "tiled", False),
    (1, 64, 64, 32, "f32", "rand", "tiled", True),
    (2, 33, 16, 17, "f32", "zeros_mixed", "generic", True),
    (1, 40, 100, 23, "f32", "rand", "generic", False),
    # the lane-per-state kernels: ragged chunks (32 steps at 16 states, 16 at 32 and 64), partly
    # filled waves and workgroups, both sides of the series threshold in one chunk
    (2, 64, 16, 64, "f32", "mamba", "lanes", False),
    (2, 37, 16, 45, "bf16", "rand", "lanes", True),
    (1, 70, 16, 40, "f32", "zeros_mixed", "lanes", False),
    (2, 64, 16, 100, "f32", "tiny", "lanes", True),
    (1, 50, 32, 33, "bf16", "mamba", "lanes", False),
    (2, 19, 32, 70, "f32", "zeros_mixed", "lanes", True),
    (1, 64, 64, 31, "f32", "rand", "lanes", True),
    (1, 33, 64, 50, "bf16", "tiny", "lanes", False),
    # the chunked kernel: the default for few rows of >= 1024 steps, forced below that; ragged
    # last chunks, both sides of the series threshold within a run
    (1, 8, 16, 1100, "f32", "zeros_mixed", None, True),
    (2, 5, 16, 200, "bf16", "tiny", "chunked", False),
    (1, 6, 16, 77, "f32", "rand", "chunked", True),
    (2, 64, 16, 130, "f32", "mamba", "chunked", False),
]


def _a(kind, dim, N, rng):
    if kind == "zeros_mixed":  # every third state has A = 0 (pure integration)
        A = (-rng.uniform(0.05, 4.0, (dim, N))).astype(np.float32)
        A[:, ::3] = 0.0
        return A
    if kind == "tiny":  # |dt A| far below the series threshold
        return (-rng.uniform(1e-5, 1e-3, (dim, N))).astype(np.float32)
    return None


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_zoh_edge_cases(idx):
    batch, dim, N, L, dtype, a_kind, kernel, with_h0 = EDGE[idx]
    print(f"zoh edge case {EDGE[idx]}", flush=True)
    rng = np.random.default_rng(700 + idx)
    x = gu.case(700 + idx, batch, dim, N, L, dtype=dtype, a_kind="rand" if a_kind != "mamba" else "mamba")
    A = _a(a_kind, dim, N, rng)
    if A is not None:
        x["A"] = A
    h0 = rng.standard_normal((batch, dim, N)) if with_h0 else None
    _check(x, 1e-4 if dtype == "f32" else 2e-3, kernel=kernel, h0=h0)


@pytest.mark.parametrize("kernel,N", [("tiled", 16), ("generic", 16), ("lanes", 16), ("lanes", 64), ("chunked", 16)])
def test_zoh_with_zero_A_is_euler_bit_for_bit(kernel, N):
    """At A = 0 the zero-order-hold coefficient is dt exactly: the same bits as the Euler scan."""
    x = gu.case(720, 2, 64, N, 64, dtype="bf16")
    x["A"] = np.zeros_like(x["A"])
    ye, le = _run(x, kernel, zoh=False)
    yz, lz = _run(x, kernel, zoh=True)
    assert np.array_equal(ye, yz) and np.array_equal(le, lz)



@pytest.mark.parametrize("L", [1, 3, 64])
def test_zoh_short_calls_keep_the_lane_kernel_states(L):
    """The short-call kernel with the zero-order hold (the default for calls of at most 4 steps):
    its states are the lane-per-state kernel's bits, y agrees to rounding (the 16 states' terms
    are added in another order), and both match the oracle."""
    x = gu.case(740 + L, 2, 96, 16, L, dtype="bf16", a_kind="rand")
    rng = np.random.default_rng(L)
    h0 = rng.standard_normal((2, 96, 16)).astype(np.float32)
    ys, ls = _run(x, "step", h0=h0)
    yl, ll = _run(x, "lanes", h0=h0)
    assert np.array_equal(ls, ll)
    assert gu.rel_err(ys, yl) <= 1e-6
    _check(x, 2e-3, kernel="step", h0=h0)
