"""GPU parity of the lane-per-state forward kernels (MAMBA_SCAN_FORCE_LANES: 16, 32 and 64
states) against the fp64 oracle, on the shapes their decomposition makes special: channel counts
that leave a wave or a workgroup partly empty, lengths that end inside a chunk (16- or 32-step
chunks), B / C rows that are not 4-element aligned (element-wise staging instead of vector
loads), exp mode, no z / D / bias, an initial state, strided views, and an all-NaN-free check of
the padded steps. Bar: max|g - r| / (1 + |r|) <= 1e-4 (fp32 inputs) or 2e-3 (bf16 inputs).
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from selective_state_space_29_amd import scan

pytestmark = pytest.mark.gpu


def tol(dtype):
    return gu.FP32_TOL if dtype == "f32" else gu.BF16_TOL


CASES = [
    # (batch, dim, N, L, dtype, options)
    (1, 1, 16, 1, "f32", {}),                       # one lane row used, one step
    (2, 5, 16, 31, "bf16", {}),                     # 5 channels: a wave and a half; L odd (element staging)
    (1, 17, 16, 64, "f32", {"h0": True}),           # one channel past a workgroup; exact chunks
    (3, 40, 16, 97, "bf16", {"softplus": False}),   # exp mode; L = 3 chunks + 1
    (2, 12, 16, 40, "f32", {"z": False, "D": False, "bias": False}),
    (1, 3, 32, 1, "bf16", {}),                      # 32 states: half a wave empty
    (2, 9, 32, 47, "f32", {"h0": True}),            # 9 channels over workgroups of 8; ragged
    (1, 20, 32, 128, "bf16", {"softplus": False, "z": False}),
    (2, 6, 64, 15, "bf16", {}),                     # 64 states: one 16-step chunk, ragged
    (1, 5, 64, 33, "f32", {"h0": True, "D": False}),
    (3, 7, 64, 80, "bf16", {"bias": False}),
]


@pytest.mark.parametrize("idx", range(len(CASES)),
                         ids=[f"b{c[0]}d{c[1]}n{c[2]}l{c[3]}{c[4]}" for c in CASES])
def test_lane_kernels_against_the_oracle(idx):
    batch, dim, N, L, dtype, opt = CASES[idx]
    print(f"lanes case {CASES[idx]}", flush=True)
    x = gu.case(7000 + idx, batch, dim, N, L, dtype=dtype, z=opt.get("z", True), D=opt.get("D", True),
                bias=opt.get("bias", True))
    sp = opt.get("softplus", True)
    if not sp:
        x["delta_bias"] = None if x["delta_bias"] is None else (x["delta_bias"] * 0.5).astype(np.float32)
    h0 = np.random.default_rng(idx).standard_normal((batch, dim, N)).astype(np.float32) if opt.get("h0") else None
    y, ls = gu.gpu_scan(x, softplus=sp, kernel="lanes", h0=h0)
    yr, lr = gu.oracle_scan(x, softplus=sp, h0=h0)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(ls))
    ey, el = gu.rel_err(y, yr), gu.rel_err(ls, lr)
    print(f"   y {ey:.2e} last_state {el:.2e}", flush=True)
    assert ey <= tol(dtype) and el <= tol(dtype)


@pytest.mark.parametrize("N", [16, 32, 64])
def test_lanes_equal_across_split_points(N):
    """scan(0..L) == scan(0..L1) then scan(L1..L, h0): bit-identical for split points inside and
    at the end of a chunk (the per-step arithmetic does not depend on where a chunk starts)."""
    x = gu.case(7100 + N, 2, 24, N, 150, dtype="bf16")
    y, ls = gu.gpu_scan(x, kernel="lanes")
    for L1 in (16, 37, 64, 149):
        a = {k: (np.ascontiguousarray(v[..., :L1]) if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
        b = {k: (np.ascontiguousarray(v[..., L1:]) if k in ("u", "delta", "z", "B", "C") else v) for k, v in x.items()}
        ya, la = gu.gpu_scan(a, kernel="lanes")
        yb, lb = gu.gpu_scan(b, kernel="lanes", h0=la)
        assert np.array_equal(np.concatenate([ya, yb], -1), y), f"N={N} split at {L1}"
        assert np.array_equal(lb, ls), f"N={N} split at {L1}"


@pytest.mark.parametrize("N", [16, 32, 64])
def test_lanes_aligned_and_unaligned_staging_agree(N):
    """B / C handed over as 4-element-aligned rows (vector staging) or as a view whose rows are
    not (element-wise staging): the same inputs give the same bits."""
    x = gu.case(7200 + N, 2, 20, N, 96, dtype="bf16")
    g = {k: gu.to_dev(v) for k, v in x.items() if v is not None}
    base = dict(D=g["D"], z=g["z"], delta_bias=g["delta_bias"], delta_softplus=True, return_last_state=True,
                kernel="lanes")
    y1, l1 = scan.selective_scan_fn(g["u"], g["delta"], g["A"], g["B"], g["C"], **base)
    # the same values at an odd element offset inside a larger buffer: rows lose 8-byte alignment
    Bbig = torch.zeros((2, N, 97), dtype=torch.bfloat16, device="cuda:0")
    Cbig = torch.zeros((2, N, 97), dtype=torch.bfloat16, device="cuda:0")
    Bbig[..., 1:] = g["B"]
    Cbig[..., 1:] = g["C"]
    y2, l2 = scan.selective_scan_fn(g["u"], g["delta"], g["A"], Bbig[..., 1:], Cbig[..., 1:], **base)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(l1, l2)


def test_lanes_reject_other_state_counts():
    x = gu.case(7300, 1, 8, 24, 20)
    with pytest.raises(ValueError, match=r"\(-8\)"):
        gu.gpu_scan(x, kernel="lanes")
