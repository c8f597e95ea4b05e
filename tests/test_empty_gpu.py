"""Empty calls through the C ABI: no (batch, channel) row, or no step. The scan of no steps leaves
its initial state (last_state = h0, or zeros); the gradients are sums over nothing (zeros), except
that of the initial state over no steps, which is the final state's. Every kernel choice is
accepted and none is used; outputs around the results are not touched."""

import numpy as np
import pytest
import torch

from selective_state_space_29_amd import scan

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KERNELS = (None, "generic", "tiled", "lanes", "chunked", "step")


def inputs(batch, dim, L, N, dtype=torch.bfloat16, seed=0, z=True, D=True, bias=True):
    g = torch.Generator(device="cpu").manual_seed(seed)

    def r(*shape, dt=torch.float32):
        return torch.randn(*shape, generator=g).to(dt).to(DEV)

    return dict(u=r(batch, dim, L, dt=dtype), delta=r(batch, dim, L, dt=dtype),
                A=-torch.rand(dim, N, generator=g).to(DEV) - 0.1, B=r(batch, N, L, dt=dtype),
                C=r(batch, N, L, dt=dtype), D=r(dim) if D else None, z=r(batch, dim, L, dt=dtype) if z else None,
                delta_bias=r(dim) if bias else None)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("N", (16, 64, 5))
def test_no_steps_leaves_the_initial_state(kernel, N):
    x = inputs(3, 40, 0, N)
    h0 = torch.randn(3, 40, N, device=DEV)
    y, ls = scan.selective_scan_fn(**x, delta_softplus=True, return_last_state=True, h0=h0, kernel=kernel)
    torch.cuda.synchronize()
    assert y.shape == (3, 40, 0)
    assert torch.equal(ls, h0)
    # without h0: zeros, written over whatever the buffer held
    out = torch.full((3, 40, N), float("nan"), device=DEV)
    y, ls = scan.selective_scan_fn(**x, delta_softplus=True, return_last_state=True, last_state_out=out, kernel=kernel)
    torch.cuda.synchronize()
    assert ls.data_ptr() == out.data_ptr() and torch.equal(ls, torch.zeros_like(ls))
    q = dict(x, delta_softplus=True, return_last_state=True, kernel=kernel)
    assert scan.forward_kernel(**q) == "generic"
    assert scan.forward_kernel(**dict(q, return_last_state=False)) == "none"


@pytest.mark.parametrize("shape", [(0, 40, 100, 16), (3, 0, 100, 16), (0, 0, 0, 64), (2, 0, 0, 32)])
def test_no_rows(shape):
    b, d, L, N = shape
    x = inputs(b, d, L, N)
    for kernel in KERNELS:
        y, ls = scan.selective_scan_fn(**x, delta_softplus=True, return_last_state=True, kernel=kernel)
        assert y.shape == (b, d, L) and ls.shape == (b, d, N)
        assert scan.forward_kernel(**x, delta_softplus=True, return_last_state=True, kernel=kernel) == "none"
    torch.cuda.synchronize()


def test_empty_slice_of_a_sequence_writes_nothing_around_it():
    """A length-0 view into real buffers: y's storage keeps its bits, last_state gets h0."""
    x = inputs(2, 24, 64, 16)
    xs = {k: (v[..., :0] if (v is not None and v.dim() == 3 and k != "A") else v) for k, v in x.items()}
    y_buf = torch.full((2, 24, 64), 7.0, device=DEV)
    h0 = torch.randn(2, 24, 16, device=DEV)
    y, ls = scan.selective_scan_fn(**xs, delta_softplus=True, return_last_state=True, h0=h0, out=y_buf[..., :0])
    torch.cuda.synchronize()
    assert torch.equal(y_buf, torch.full_like(y_buf, 7.0)) and torch.equal(ls, h0)


def test_checkpoints_of_an_empty_call():
    x = inputs(2, 8, 0, 16)
    ck = torch.empty(scan.checkpoint_shape(2, 8, 0, 16), device=DEV)
    y, ls = scan.selective_scan_fn(**x, delta_softplus=True, return_last_state=True, checkpoints_out=ck)
    torch.cuda.synchronize()
    assert ck.numel() == 0 and torch.equal(ls, torch.zeros_like(ls))


@pytest.mark.parametrize("static", (False, True))
@pytest.mark.parametrize("kernel", (None, "lanes", "tiled"))
def test_backward_over_no_steps(kernel, static):
    b, d, N = 3, 20, 16
    x = inputs(b, d, 0, N)
    dy = torch.empty(b, d, 0, device=DEV)
    dlast = torch.randn(b, d, N, device=DEV)
    h0 = torch.randn(b, d, N, device=DEV)
    g = scan.selective_scan_bwd(**x, dy=dy, delta_softplus=True, h0=h0, dlast_state=dlast, kernel=kernel,
                                static_scratch=static)
    torch.cuda.synchronize()
    assert torch.equal(g["h0"], dlast)  # the initial state of no steps is the final state
    for k in ("A", "D", "delta_bias"):
        assert torch.equal(g[k], torch.zeros_like(g[k])), k
    for k in ("u", "delta", "z", "B", "C"):
        assert g[k].numel() == 0, k
    g = scan.selective_scan_bwd(**x, dy=dy, delta_softplus=True, kernel=kernel, static_scratch=static)
    torch.cuda.synchronize()
    assert torch.equal(g["h0"], torch.zeros_like(g["h0"]))


@pytest.mark.parametrize("shape", [(2, 0, 50, 16), (0, 6, 50, 32), (0, 0, 10, 8)])
def test_backward_without_rows(shape):
    b, d, L, N = shape
    x = inputs(b, d, L, N)
    g = scan.selective_scan_bwd(**x, dy=torch.empty(b, d, L, device=DEV), delta_softplus=True,
                                dlast_state=torch.empty(b, d, N, device=DEV))
    torch.cuda.synchronize()
    # dB, dC: (batch, N, L) sums over no channel; dA, dD, dbias: sums over no (batch, step)
    for k in ("B", "C", "A", "D", "delta_bias"):
        assert torch.equal(g[k], torch.zeros_like(g[k])), k
    assert g["B"].shape == (b, N, L) and g["A"].shape == (d, N)


def test_autograd_through_an_empty_sequence():
    x = inputs(2, 12, 0, 16, dtype=torch.float32)
    leaves = {k: v.clone().requires_grad_(True) for k, v in x.items() if v is not None}
    h0 = torch.randn(2, 12, 16, device=DEV, requires_grad=True)
    y, ls = scan.selective_scan(**leaves, delta_softplus=True, return_last_state=True, h0=h0)
    (ls * 3.0).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(h0.grad, torch.full_like(h0, 3.0))
    assert torch.equal(leaves["A"].grad, torch.zeros_like(leaves["A"]))
    assert torch.equal(leaves["D"].grad, torch.zeros_like(leaves["D"]))
