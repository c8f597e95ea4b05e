"""The fp64 oracle against its pins (see pins.py), plus the pages' own einsum loop."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(oracle_mod, pin):
    pin(oracle_mod.selective_scan)


def pages_einsum_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False,
                      h0=None):
    """The pages' formulation run in torch fp64 on the CPU: bias + softplus|exp on delta
    ('Mamba代码实战…' §2.2), dA/dB as (B, D, L, N) einsums (§3.1), the per-step state loop (§3.2),
    the output contraction with the subscripts of 'Mamba-minimal项目解析…' ('b d_in n, b n -> b d_in'),
    then the skip and the silu gate (§3.3)."""
    t = lambda x: None if x is None else torch.as_tensor(np.asarray(x, dtype=np.float64))
    u, delta, A, B, C, D, z, bias = map(t, (u, delta, A, B, C, D, z, delta_bias))
    if bias is not None:
        delta = delta + bias.view(1, -1, 1)
    delta = F.softplus(delta, beta=1.0, threshold=1e9) if delta_softplus else delta.exp()
    dA = torch.einsum("bdl,dn->bdln", delta, A).exp()
    dB = torch.einsum("bdl,bnl->bdln", delta, B)
    state = torch.zeros(u.shape[0], u.shape[1], A.shape[1], dtype=torch.float64)
    if h0 is not None:
        state = t(h0).clone()
    ys = []
    for i in range(u.shape[2]):
        state = dA[:, :, i] * state + dB[:, :, i] * u[:, :, i].unsqueeze(-1)
        ys.append(torch.einsum("bdn,bn->bd", state, C[:, :, i]))
    y = torch.stack(ys, dim=-1)
    if D is not None:
        y = y + u * D.view(1, -1, 1)
    if z is not None:
        y = y * F.silu(z)
    return y.numpy(), state.numpy()


@pytest.mark.parametrize("seed,shape,kw", [
    (101, (2, 4, 6, 50), {}),
    (102, (1, 3, 16, 64), dict(h0=True)),
    (103, (3, 2, 2, 20), dict(z=False, softplus=False, bias_scale=0.2)),
])
def test_oracle_matches_pages_einsum_loop(oracle_mod, seed, shape, kw):
    c = pins.rand_case(seed, *shape, **kw)
    y, ls = oracle_mod.selective_scan(**c)
    yp, lp = pages_einsum_scan(**c)
    assert np.max(np.abs(y - yp) / (1 + np.abs(yp))) <= 1e-13
    assert np.max(np.abs(ls - lp) / (1 + np.abs(lp))) <= 1e-13


def test_cumprod_parallel_scan_of_the_page_is_not_the_recurrence(oracle_mod):
    """'Mamba代码实战…' §4.2/§6 offer cumsum(dB * cumprod(dA)) * u as a parallel scan. It is not
    the recurrence: already at L = 1 it scales the input term by dA. The oracle follows the
    sequential loop of §3.2; this documents the disagreement on the L=1 hand case."""
    f = np.float32
    c = dict(u=np.array([[[2.0]]], f), delta=np.array([[[0.0]]], f),
             A=np.array([[-1.0, -2.0]], f), B=np.array([[[1.0], [2.0]]], f),
             C=np.array([[[3.0], [-1.0]]], f), delta_softplus=True)
    _, ls = oracle_mod.selective_scan(**c)
    dt = np.log(2.0)
    dA = np.exp(dt * np.array([-1.0, -2.0]))
    dB = dt * np.array([1.0, 2.0])
    wrong = np.cumsum(dB * np.cumprod(dA)) * 2.0  # one step: dB * dA * u
    assert np.allclose(ls[0, 0], dB * 2.0, rtol=0, atol=1e-15)
    assert not np.allclose(wrong, dB * 2.0)


def test_oracle_row_subset_matches_full(oracle_mod):
    c = pins.rand_case(111, 3, 5, 4, 21, h0=True)
    y, ls = oracle_mod.selective_scan(**c)
    rows = [14, 0, 7, 7, 3]
    yr, lr = oracle_mod.selective_scan(**c, rows=rows)
    assert np.array_equal(yr, y.reshape(15, -1)[rows])
    assert np.array_equal(lr, ls.reshape(15, -1)[rows])


def test_oracle_threads_do_not_change_results(oracle_mod):
    c = pins.rand_case(121, 2, 7, 3, 40)
    y1, l1 = oracle_mod.selective_scan(**c, nthreads=1)
    y8, l8 = oracle_mod.selective_scan(**c, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(l1, l8)


def test_oracle_rejects_bad_shapes(oracle_mod):
    c = pins.rand_case(131, 1, 2, 3, 8)
    c["B"] = c["B"][:, :2]
    with pytest.raises(ValueError):
        oracle_mod.selective_scan(**c)
