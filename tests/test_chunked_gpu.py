"""The chunked kernel (parallel along the sequence) on the GPU, through the C ABI.

A wave holds one channel; its four 16-lane rows scan four consecutive 16-step runs of every
64-step chunk from a zero state, the runs' (decay product, end state) pairs are combined with the
associative operator of the parallel scan ("手把手用PyTorch实现Mamba的SSM层…" §3.2) and every run
is re-scanned from the state entering it. What that decomposition makes special is tested here,
against the fp64 oracle (max|g - r| / (1 + |r|) <= 1e-4 for fp32 inputs, 2e-3 for bf16 inputs):
lengths ending anywhere in a run or a chunk, partly filled workgroups (4 channels each), slowly
decaying states carried over many chunks, growing states (A > 0), unaligned B / C rows, exp mode,
an initial state, no z / D / bias; a sequence split at a multiple of 64 steps and resumed from
last_state is bit-identical to one call, split elsewhere it meets the bar; and the library picks
it by itself for the genomic shape (4 x 1024 channels, L = 100 000).
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
from selective_state_space_29_amd import scan

pytestmark = pytest.mark.gpu

SEQ = ("u", "delta", "z", "B", "C")


def tol(dtype):
    return gu.FP32_TOL if dtype == "f32" else gu.BF16_TOL


CASES = [
    # batch, dim, L, dtype, options
    (1, 1, 1, "f32", {}),
    (1, 3, 15, "bf16", {}),
    (2, 4, 16, "f32", {}),
    (1, 5, 17, "bf16", {}),
    (2, 6, 63, "f32", {}),
    (1, 7, 64, "bf16", {}),
    (2, 9, 65, "f32", {}),
    (1, 4, 127, "bf16", {}),
    (2, 3, 128, "f32", {}),
    (1, 8, 129, "bf16", {}),
    (3, 10, 1000, "bf16", {}),
    (2, 6, 777, "f32", dict(z=False, D=False, bias=False)),
    (1, 12, 300, "bf16", dict(a_kind="random")),
    (2, 8, 4104, "bf16", {}),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[f"b{c[0]}d{c[1]}l{c[2]}{c[3]}" for c in CASES])
def test_shapes_against_the_oracle(idx):
    b, d, L, dt, opt = CASES[idx]
    print(f"[chunked] case {CASES[idx]}", flush=True)
    x = gu.case(7000 + idx, b, d, 16, L, dtype=dt, **opt)
    y, ls = gu.gpu_scan(x, kernel="chunked")
    yr, lr = gu.oracle_scan(x)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(ls))
    assert gu.rel_err(y, yr) <= tol(dt) and gu.rel_err(ls, lr) <= tol(dt)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_exp_mode_and_initial_state(dt):
    x = gu.case(7100, 2, 13, 16, 333, dtype=dt)
    x["delta_bias"] = (x["delta_bias"] * 0.5).astype(np.float32)
    h0 = np.random.default_rng(7101).standard_normal((2, 13, 16)).astype(np.float32)
    for sp in (False, True):
        y, ls = gu.gpu_scan(x, softplus=sp, h0=h0, kernel="chunked")
        yr, lr = gu.oracle_scan(x, softplus=sp, h0=h0)
        assert gu.rel_err(y, yr) <= tol(dt) and gu.rel_err(ls, lr) <= tol(dt)


def test_slow_decay_carries_across_many_chunks():
    """A close to 0 (decay per step ~ 1 - 1e-4): the state entering a chunk dominates its outputs
    for thousands of steps, so any slip in the carry or the combine shows."""
    x = gu.case(7200, 2, 8, 16, 5000, dtype="f32")
    x["A"] = (-np.linspace(1e-4, 3e-3, 16, dtype=np.float32))[None, :].repeat(8, 0).copy()
    h0 = np.random.default_rng(7201).standard_normal((2, 8, 16)).astype(np.float32)
    y, ls = gu.gpu_scan(x, h0=h0, kernel="chunked")
    yr, lr = gu.oracle_scan(x, h0=h0)
    assert gu.rel_err(y, yr) <= gu.FP32_TOL and gu.rel_err(ls, lr) <= gu.FP32_TOL


def test_growing_states_and_zero_input_prefix():
    """A > 0 (the state grows) with no input for the first 200 steps: the zero state stays zero
    through the combine (decay products are kept finite), then grows like the oracle's."""
    x = gu.case(7300, 1, 4, 16, 600, dtype="f32")
    x["A"] = np.full((4, 16), 0.05, dtype=np.float32)
    x["delta_bias"] = np.full(4, -3.0, dtype=np.float32)
    x["u"] = x["u"].copy()
    x["u"][..., :200] = 0.0
    y, ls = gu.gpu_scan(x, kernel="chunked")
    yr, lr = gu.oracle_scan(x)
    assert np.all(np.isfinite(y)) and np.all(y[..., :200] == 0.0) and np.all(yr[..., :200] == 0.0)
    assert gu.rel_err(y, yr) <= gu.FP32_TOL and gu.rel_err(ls, lr) <= gu.FP32_TOL


def test_unaligned_bc_rows():
    """B / C rows that are not 4-element aligned are staged element by element: same bits as the
    aligned staging of the same values."""
    x = gu.case(7400, 2, 6, 16, 250, dtype="bf16")
    g = {k: gu.to_dev(v) if isinstance(v, np.ndarray) else v for k, v in x.items()}
    big = {k: torch.zeros((2, 16, 251), dtype=g[k].dtype, device="cuda:0") for k in ("B", "C")}
    for k in big:
        big[k][..., 1:] = g[k]
    Bv, Cv = big["B"][..., 1:], big["C"][..., 1:]
    kw = dict(D=g["D"], z=g["z"], delta_bias=g["delta_bias"], delta_softplus=True, return_last_state=True,
              kernel="chunked")
    y1, l1 = scan.selective_scan_fn(g["u"], g["delta"], g["A"], g["B"], g["C"], **kw)
    y2, l2 = scan.selective_scan_fn(g["u"], g["delta"], g["A"], Bv, Cv, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
    yr, lr = gu.oracle_scan(x)
    assert gu.rel_err(y2.cpu().numpy(), yr) <= gu.BF16_TOL


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_continuation(dt):
    x = gu.case(7500, 2, 7, 16, 700, dtype=dt)
    y, ls = gu.gpu_scan(x, kernel="chunked")
    for L1 in (64, 320, 100, 333):
        a = {k: (np.ascontiguousarray(v[..., :L1]) if k in SEQ else v) for k, v in x.items()}
        b = {k: (np.ascontiguousarray(v[..., L1:]) if k in SEQ else v) for k, v in x.items()}
        ya, la = gu.gpu_scan(a, kernel="chunked")
        yb, lb = gu.gpu_scan(b, kernel="chunked", h0=la)
        ys = np.concatenate([ya, yb], -1)
        if L1 % 64 == 0:
            assert np.array_equal(ys, y) and np.array_equal(lb, ls), f"split at {L1}"
        else:
            assert gu.rel_err(ys, y) <= tol(dt) and gu.rel_err(lb, ls) <= tol(dt), f"split at {L1}"


def test_library_picks_it_for_the_genomic_shape():
    """The default choice: chunked for 4 x 1024 channels of 100 000 steps (a quarter of the SIMDs'
    worth of lane-per-state waves), the lane-per-state kernel for the Mamba-130m layer (8 x 1536,
    2048 steps) and for short calls."""
    dev = "cuda:0"

    def shaped(batch, dim, L, N=16):
        buf = torch.zeros(L, dtype=torch.bfloat16, device=dev)
        seq = buf.as_strided((batch, dim, L), (0, 0, 1))
        bc = buf.as_strided((batch, N, L), (0, 0, 1))
        A = -torch.ones((dim, N), device=dev)
        return dict(u=seq, delta=seq, z=seq, B=bc, C=bc, A=A, D=torch.ones(dim, device=dev),
                    delta_bias=torch.zeros(dim, device=dev))

    def pick(batch, dim, L, N=16):
        t = shaped(batch, dim, L, N)
        return scan.forward_kernel(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                   delta_bias=t["delta_bias"], delta_softplus=True, return_last_state=True)

    assert pick(4, 1024, 100000) == "chunked"
    assert pick(8, 1536, 2048) == "lanes"
    assert pick(4, 1024, 1000) == "lanes"
    assert pick(4, 4096, 16384, N=64) == "lanes"
    assert pick(4, 1024, 100000, N=24) == "tiled"
