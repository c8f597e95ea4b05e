"""GPU parity of the backward pass (``mamba_scan_bwd`` through the C ABI) against the fp64 backward
oracle on identical inputs.

Bar: max|g - r| / (1 + |r|) over every gradient, the forward's bars: <= 1e-4 when u, delta, z,
B, C are fp32 and <= 2e-3 when they are bf16 (the same bits on both sides in either case). The
GPU accumulates in fp32 (the reverse recurrence over up to L steps, sums over channels for dB, dC
and over batch x steps for dA, dD, dbias, all in a fixed order) and the oracle in fp64; the
inputs' storage precision does not enter the difference, so the fp32 bar is the forward's fp32
bar, not the bf16 one.
"""

import numpy as np
import pytest
import torch

import gpu_util as gu
import oracle
from selective_state_space_29_amd import scan, workloads

pytestmark = pytest.mark.gpu

TOL = 2e-3        # bf16 storage
TOL_F32 = 1e-4    # fp32 storage


def tol_of(x):
    return TOL_F32 if x["u"].dtype == np.float32 else TOL
NAMES = ("u", "delta", "z", "B", "C", "A", "D", "delta_bias", "h0")


def _grads_gpu(x, dy, dlast, softplus, h0=None, kernel=None):
    g = {k: gu.to_dev(v) if isinstance(v, np.ndarray) else v for k, v in x.items()}
    out = scan.selective_scan_bwd(
        g["u"], g["delta"], g["A"], g["B"], g["C"], gu.to_dev(dy.astype(np.float32)), D=g.get("D"),
        z=g.get("z"), delta_bias=g.get("delta_bias"), delta_softplus=softplus,
        h0=None if h0 is None else gu.to_dev(h0.astype(np.float32)),
        dlast_state=None if dlast is None else gu.to_dev(dlast.astype(np.float32)), want_dh0=True,
        kernel=kernel)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _grads_oracle(x, dy, dlast, softplus, h0=None):
    return oracle.selective_scan_bwd(
        x["u"], x["delta"], x["A"], x["B"], x["C"], dy.astype(np.float32).astype(np.float64),
        D=x.get("D"), z=x.get("z"), delta_bias=x.get("delta_bias"), delta_softplus=softplus,
        h0=None if h0 is None else h0.astype(np.float32).astype(np.float64),
        glast=None if dlast is None else dlast.astype(np.float32).astype(np.float64))


def _check(x, softplus=True, with_h0=False, with_dlast=True, seed=0, tol=None, kernel=None):
    tol = tol_of(x) if tol is None else tol
    batch, dim, L = x["u"].shape
    N = x["A"].shape[1]
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((batch, dim, L)).astype(np.float32)
    dlast = rng.standard_normal((batch, dim, N)).astype(np.float32) if with_dlast else None
    h0 = rng.standard_normal((batch, dim, N)).astype(np.float32) if with_h0 else None
    gg = _grads_gpu(x, dy, dlast, softplus, h0, kernel)
    gr = _grads_oracle(x, dy, dlast, softplus, h0)
    for k in NAMES:
        if k not in gr or (k != "h0" and x.get(k) is None):
            continue
        assert np.all(np.isfinite(gg[k])), k
        err = gu.rel_err(gg[k], gr[k])
        print(f"  d{k}: max rel err {err:.3e} (bar {tol:g})", flush=True)
        assert err <= tol, f"d{k}: max rel err {err:.3g}"
    return gg


@pytest.mark.parametrize("wid,kernel", [(1, None), (1, "tiled"), (2, None), (2, "tiled"), (3, None), (3, "tiled")])
def test_workload_backward_parity(wid, kernel):
    """Default: the lane-per-state kernel (16 states in workloads 2, 3; 32 in workload 1, two
    blocks of 16); the segment-tiled kernel forced as well."""
    w = workloads.WORKLOADS[wid]
    x = workloads.make_inputs(w)
    print(f"backward parity, workload {wid}: {w.name}, kernel {kernel or 'default'}", flush=True)
    _check(x, softplus=w.softplus, with_dlast=w.last_state, seed=wid, kernel=kernel)


EDGE = [
    # (batch, dim, N, L, dtype, flags)
    (1, 1, 1, 1, "f32", {}),
    (2, 64, 16, 16, "f32", {}),
    (2, 80, 16, 17, "bf16", {}),
    (3, 130, 16, 100, "f32", {"h0": True}),
    (1, 64, 8, 33, "bf16", {"softplus": False}),
    (2, 70, 4, 40, "f32", {"z": False, "D": False, "bias": False}),
    (2, 65, 12, 31, "f32", {"dlast": False}),
    (1, 128, 10, 48, "bf16", {"h0": True, "dlast": False}),
    (2, 96, 16, 7, "f32", {"a_kind": "rand"}),
    (1, 192, 16, 257, "bf16", {"h0": True}),
    # more than 16 states: one launch per block of states, sums carried across the blocks
    (2, 70, 24, 40, "f32", {"h0": True}),            # blocks 16 + 8
    (1, 64, 32, 33, "bf16", {}),                     # 16 + 16
    (2, 100, 40, 50, "f32", {"softplus": False}),    # 16 + 16 + 8
    (1, 130, 64, 70, "bf16", {"h0": True}),          # 4 x 16
    (2, 64, 11, 20, "f32", {}),                      # odd in (8, 16]: 8 + 3
    (1, 65, 27, 17, "f32", {"z": False}),            # 16 + 8 + 3
    (1, 66, 46, 24, "bf16", {"D": False, "bias": False, "dlast": False}),  # 16 + 16 + 14
    (1, 40, 256, 19, "f32", {}),                     # the largest dstate
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_backward_edge_cases(idx):
    batch, dim, N, L, dtype, fl = EDGE[idx]
    print(f"backward edge case {EDGE[idx]}", flush=True)
    x = gu.case(500 + idx, batch, dim, N, L, dtype=dtype, z=fl.get("z", True), D=fl.get("D", True),
                bias=fl.get("bias", True), a_kind=fl.get("a_kind", "mamba"))
    _check(x, softplus=fl.get("softplus", True), with_h0=fl.get("h0", False),
           with_dlast=fl.get("dlast", True), seed=idx)


# The lane-per-state kernel forced: ragged lengths (segments of 16 steps), channel counts that
# leave workgroups (16 channels) and waves (4) partly empty, every optional input on and off; 32
# and 64 states (blocks of 16 carried through du, ddelta, dz) with and without the gate; few
# channels over long sequences, which split the segments into parts of at least 32 segments and
# 4 pre-pass sub-parts each (63 at (1, 4, 16, 32770), whose last part is 3 segments: one short and
# three empty sub-parts; 5 at (1, 8, 16, 3000), 4 at (2, 20, 32, 2047), 2 at (1, 3, 64, 1500)),
# with and without dlast
EDGE_LANES = [
    # (batch, dim, N, L, dtype, flags)
    (1, 1, 16, 1, "f32", {}),
    (1, 3, 16, 2, "bf16", {"h0": True}),
    (2, 16, 16, 15, "f32", {}),
    (1, 17, 16, 16, "bf16", {"dlast": False}),
    (3, 20, 16, 17, "f32", {"h0": True}),
    (2, 33, 16, 31, "bf16", {"softplus": False}),
    (1, 64, 16, 33, "f32", {"z": False, "D": False, "bias": False}),
    (2, 48, 16, 100, "bf16", {"a_kind": "rand", "h0": True}),
    (1, 130, 16, 257, "f32", {"z": False}),
    (2, 96, 16, 64, "bf16", {"D": False, "dlast": False}),
    (1, 40, 16, 1000, "f32", {"softplus": False, "h0": True}),
    (2, 70, 32, 40, "f32", {"h0": True}),
    (1, 33, 32, 17, "bf16", {"z": False}),
    (1, 130, 64, 70, "bf16", {"h0": True}),
    (2, 20, 64, 33, "f32", {"softplus": False, "dlast": False}),
    (1, 50, 64, 300, "bf16", {"D": False, "bias": False, "a_kind": "rand"}),
    (1, 8, 16, 3000, "f32", {"h0": True}),
    (2, 20, 32, 2047, "bf16", {"a_kind": "rand", "dlast": False}),
    (1, 3, 64, 1500, "f32", {"softplus": False}),
    (1, 4, 16, 32770, "f32", {"dlast": False}),
]


@pytest.mark.parametrize("idx", range(len(EDGE_LANES)))
def test_lane_backward_edge_cases(idx):
    batch, dim, N, L, dtype, fl = EDGE_LANES[idx]
    print(f"lane-per-state backward edge case {EDGE_LANES[idx]}", flush=True)
    x = gu.case(700 + idx, batch, dim, N, L, dtype=dtype, z=fl.get("z", True), D=fl.get("D", True),
                bias=fl.get("bias", True), a_kind=fl.get("a_kind", "mamba"))
    _check(x, softplus=fl.get("softplus", True), with_h0=fl.get("h0", False),
           with_dlast=fl.get("dlast", True), seed=idx, kernel="lanes")


@pytest.mark.parametrize("kernel,shape", [("tiled", (2, 96, 90)), ("lanes", (2, 96, 90)), ("lanes", (4, 2048, 1024))])
def test_state_blocks_are_independent(kernel, shape):
    """dB, dC, dA and dh0 of a state depend on no other state, so with 32 states the first 16
    states' gradients are the bits of a 16-state run on those states alone (the same first block
    of 16 states, with either kernel; (4, 2048, 1024) splits the sequence into 2 parts, by a rule
    that does not depend on the state count, and recomputes the states with the lane-per-state
    forward at both state counts: a shape whose 16-state forward is the chunked kernel would not
    give the 32-state run's bits)."""
    batch, dim, L = shape
    x = gu.case(73, batch, dim, 32, L, dtype="bf16")
    rng = np.random.default_rng(4)
    dy = rng.standard_normal((batch, dim, L)).astype(np.float32)
    dlast = rng.standard_normal((batch, dim, 32)).astype(np.float32)
    h0 = rng.standard_normal((batch, dim, 32)).astype(np.float32)
    full = _grads_gpu(x, dy, dlast, True, h0, kernel=kernel)
    half = dict(x, A=np.ascontiguousarray(x["A"][:, :16]), B=np.ascontiguousarray(x["B"][:, :16]),
                C=np.ascontiguousarray(x["C"][:, :16]))
    part = _grads_gpu(half, dy, np.ascontiguousarray(dlast[..., :16]), True, np.ascontiguousarray(h0[..., :16]),
                      kernel=kernel)
    for k in ("B", "C"):
        assert np.array_equal(full[k][:, :16], part[k]), k
    assert np.array_equal(full["A"][:, :16], part["A"])
    assert np.array_equal(full["h0"][..., :16], part["h0"])


def test_genomic_workload_every_channel():
    """Full-size backward of the genomic workload (batch 4, 1024 channels, L = 100 000, split into
    3 sequence parts) against the fp64 backward oracle on every channel: the oracle runs over
    blocks of 64 channels (all batches), each block's du, ddelta, dz, dh0 rows and dA, dD, dbias
    compared on arrival, its dB and dC partial sums over the block's channels added up in fp64 and
    compared at the end."""
    w = workloads.WORKLOADS[4]
    print(f"backward parity, workload 4: {w.name} (every channel)", flush=True)
    x = workloads.make_inputs(w)
    g = {k: gu.to_dev(v) if isinstance(v, np.ndarray) else v for k, v in x.items()}
    rng = np.random.default_rng(29504)
    dy = rng.standard_normal((w.batch, w.dim, w.seqlen)).astype(np.float32)
    dlast = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
    out = scan.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], gu.to_dev(dy), D=g["D"],
                                  z=g["z"], delta_bias=g["delta_bias"], delta_softplus=True,
                                  dlast_state=gu.to_dev(dlast), want_dh0=True)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(v).all()) for v in out.values())
    got = {k: v.cpu().numpy() for k, v in out.items()}
    del out, g
    err = {k: 0.0 for k in ("u", "delta", "z", "h0", "A", "D", "delta_bias")}
    acc = {"B": 0.0, "C": 0.0}
    for c0 in range(0, w.dim, 64):
        blk = slice(c0, min(c0 + 64, w.dim))
        r = oracle.selective_scan_bwd(
            x["u"][:, blk], x["delta"][:, blk], x["A"][blk], x["B"], x["C"], dy[:, blk].astype(np.float64),
            D=x["D"][blk], z=x["z"][:, blk], delta_bias=x["delta_bias"][blk], delta_softplus=True,
            glast=dlast[:, blk].astype(np.float64))
        for k in ("u", "delta", "z", "h0"):
            err[k] = max(err[k], gu.rel_err(got[k][:, blk], r[k]))
        for k in ("A", "D", "delta_bias"):
            err[k] = max(err[k], gu.rel_err(got[k][blk], r[k]))
        for k in acc:
            acc[k] = acc[k] + r[k]
        print(f"  channels {blk.start}..{blk.stop - 1}: " + ", ".join(f"d{k} {v:.2e}" for k, v in err.items()),
              flush=True)
    for k in acc:
        err[k] = gu.rel_err(got[k], acc[k])
    for k, v in err.items():
        print(f"  d{k}: {v:.3e} (bar {TOL:g})", flush=True)
        assert v <= TOL, f"d{k}: {v:.3g}"


@pytest.mark.parametrize("wid", [5])
def test_large_workload_sampled_channels(wid):
    """Full-size backward of the 64-state workload (one launch per block of 16 states; the genomic
    one is checked on every channel above); the oracle checks every channel-local gradient of
    sampled channels:
    du, ddelta, dz and dh0 of each (batch, channel) row, and dA, dD, dbias of the channel (summed
    over the batch). dB and dC sum over all channels and are checked at the smaller sizes above."""
    w = workloads.WORKLOADS[wid]
    print(f"backward parity, workload {wid}: {w.name} (sampled channels)", flush=True)
    x = workloads.make_inputs(w)
    g = {k: gu.to_dev(v) if isinstance(v, np.ndarray) else v for k, v in x.items()}
    del x
    gen = torch.Generator(device="cuda:0").manual_seed(29500 + wid)
    dy = torch.randn((w.batch, w.dim, w.seqlen), device="cuda:0", generator=gen)
    dlast = torch.randn((w.batch, w.dim, w.dstate), device="cuda:0", generator=gen)
    out = scan.selective_scan_bwd(g["u"], g["delta"], g["A"], g["B"], g["C"], dy, D=g["D"], z=g["z"],
                                  delta_bias=g["delta_bias"], delta_softplus=True, dlast_state=dlast,
                                  want_dh0=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    chans = sorted({0, 1, 63, 64, w.dim - 1} | {int(c) for c in rng.integers(0, w.dim, 5)})
    rows = [b * w.dim + d for b in range(w.batch) for d in chans]
    idx = torch.tensor(rows, device="cuda:0")
    got = {k: out[k].reshape(w.batch * w.dim, -1).index_select(0, idx).cpu().numpy()
           for k in ("u", "delta", "z", "h0")}
    cidx = torch.tensor(chans, device="cuda:0")
    got_c = {k: out[k].index_select(0, cidx).cpu().numpy() for k in ("A", "D", "delta_bias")}
    dy_r = dy.reshape(w.batch * w.dim, -1).index_select(0, idx).cpu().numpy()
    dl_r = dlast.reshape(w.batch * w.dim, -1).index_select(0, idx).cpu().numpy()
    assert all(bool(torch.isfinite(v).all()) for v in out.values())
    del out, g, dy, dlast
    xr = workloads.make_row_inputs(w, rows)

    from concurrent.futures import ThreadPoolExecutor

    def one(i):
        s = slice(i, i + 1)
        return oracle.selective_scan_bwd(
            xr["u"][s], xr["delta"][s], xr["A"][s], xr["B"][s], xr["C"][s],
            dy_r[s].reshape(1, 1, -1).astype(np.float64), D=xr["D"][s], z=xr["z"][s],
            delta_bias=xr["delta_bias"][s], delta_softplus=True,
            glast=dl_r[s].reshape(1, 1, -1).astype(np.float64), nthreads=1)

    with ThreadPoolExecutor(max_workers=min(16, oracle.default_threads())) as ex:
        res = list(ex.map(one, range(len(rows))))
    ref = {k: np.stack([r[k].reshape(-1) for r in res]) for k in ("u", "delta", "z", "h0")}
    nc = len(chans)
    ref_c = {k: sum(np.stack([res[b * nc + j][k].reshape(-1) for j in range(nc)]) for b in range(w.batch))
             for k in ("A", "D", "delta_bias")}
    for k in ref:
        err = gu.rel_err(got[k], ref[k])
        print(f"  d{k}: {err:.3e} over {len(rows)} rows", flush=True)
        assert err <= TOL, k
    for k in ref_c:
        err = gu.rel_err(got_c[k].reshape(nc, -1), ref_c[k].reshape(nc, -1))
        print(f"  d{k}: {err:.3e} over {nc} channels", flush=True)
        assert err <= TOL, k


@pytest.mark.parametrize("kernel,shape", [("lanes", (2, 150, 200)), ("tiled", (2, 150, 200)), ("lanes", (1, 30, 2500))])
def test_backward_is_deterministic(kernel, shape):
    """Two calls, the same bits ((1, 30, 2500): 4 sequence parts)."""
    batch, dim, L = shape
    x = gu.case(71, batch, dim, 16, L, dtype="bf16")
    rng = np.random.default_rng(1)
    dy = rng.standard_normal((batch, dim, L)).astype(np.float32)
    a = _grads_gpu(x, dy, None, True, kernel=kernel)
    b = _grads_gpu(x, dy, None, True, kernel=kernel)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_autograd_function_matches_the_oracle():
    """torch autograd through the SelectiveScan function: gradients of
    sum(W * y) + sum(V * last_state) for every differentiable input."""
    x = gu.case(72, 2, 96, 16, 64, dtype="f32")
    rng = np.random.default_rng(2)
    h0 = rng.standard_normal((2, 96, 16)).astype(np.float32)
    W = rng.standard_normal((2, 96, 64)).astype(np.float32)
    V = rng.standard_normal((2, 96, 16)).astype(np.float32)
    t = {k: gu.to_dev(v).requires_grad_(True) for k, v in x.items() if v is not None}
    th0 = gu.to_dev(h0).requires_grad_(True)
    y, ls = scan.selective_scan(t["u"], t["delta"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                                delta_bias=t["delta_bias"], delta_softplus=True,
                                return_last_state=True, h0=th0)
    loss = (y * gu.to_dev(W)).sum() + (ls * gu.to_dev(V)).sum()
    loss.backward()
    gr = _grads_oracle(x, W, V, True, h0)
    for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias"):
        assert gu.rel_err(t[k].grad.cpu().numpy(), gr[k]) <= TOL_F32, k
    assert gu.rel_err(th0.grad.cpu().numpy(), gr["h0"]) <= TOL_F32
