"""Pins of the backward oracle, each against something other than the backward code itself.

* ``fd``: central finite differences of the forward oracle (itself pinned by ``pins.py``) for a
  loss sum(W * y) + sum(V * last_state), at entries of every input.
* ``autograd``: torch's fp64 CPU autograd through a separate step-by-step formulation of the
  forward recurrence (torch ops only; it shares nothing with the C oracle).
Both take ``zoh=True`` for the scan whose B is discretised by zero-order hold (the input term's
coefficient (e^{dt A} - 1) / A of "手把手用PyTorch实现Mamba的SSM层…" §2.1 in place of dt).

Each pin takes the backward oracle as a callable ``bwd(**kw)`` (and the forward as ``fwd``), so
that mutant copies of the oracle can be checked against the same pins.
"""

from __future__ import annotations

import numpy as np
import torch

SEQ = ("u", "delta", "z", "B", "C")


def make_case(seed, batch=2, dim=3, N=4, L=9, z=True, D=True, bias=True, h0=True, bf16=False,
              a_scale=1.0, a_zero=False):
    rng = np.random.default_rng(seed)

    def t(shape, scale=1.0):
        v = (scale * rng.standard_normal(shape)).astype(np.float32)
        if bf16:
            return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return v

    x = dict(u=t((batch, dim, L)), delta=t((batch, dim, L)), z=t((batch, dim, L)) if z else None,
             B=t((batch, N, L)), C=t((batch, N, L)),
             A=(-a_scale * rng.uniform(0.2, 2.5, (dim, N))).astype(np.float32),
             D=rng.standard_normal(dim).astype(np.float32) if D else None,
             delta_bias=rng.uniform(-1.5, 0.5, dim).astype(np.float32) if bias else None,
             h0=rng.standard_normal((batch, dim, N)) if h0 else None)
    if a_zero:  # a zero state in every channel: the hold's coefficient at its limit dt
        x["A"][:, 0] = 0.0
    W = rng.standard_normal((batch, dim, L))
    V = rng.standard_normal((batch, dim, N))
    return x, W, V


def _widen(a):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _loss(fwd, x, W, V, softplus, zoh=False):
    kw = dict(zoh_b=True) if zoh else {}
    y, ls = fwd(u=x["u"], delta=x["delta"], A=x["A"], B=x["B"], C=x["C"], D=x["D"], z=x["z"],
                delta_bias=x["delta_bias"], delta_softplus=softplus, h0=x["h0"], **kw)
    return float(np.sum(W * y) + np.sum(V * ls))


def fd(bwd, fwd, softplus=True, seed=5, zoh=False, **case_kw):
    """Central differences at 4 entries of each fp32 input (perturbed in fp32, divided by the
    exact difference of the two perturbed values) and of h0 (fp64); with ``a_zero`` every
    channel's zero state is among the A entries perturbed."""
    x, W, V = make_case(seed, **case_kw)
    kw = dict(zoh_b=True) if zoh else {}
    g = bwd(u=x["u"], delta=x["delta"], A=x["A"], B=x["B"], C=x["C"], gy=W, D=x["D"], z=x["z"],
            delta_bias=x["delta_bias"], delta_softplus=softplus, h0=x["h0"], glast=V, **kw)
    rng = np.random.default_rng(seed + 1)
    for k in ("u", "delta", "z", "B", "C", "A", "D", "delta_bias", "h0"):
        if x[k] is None:
            continue
        picks = [tuple(int(rng.integers(0, s)) for s in x[k].shape) for _ in range(4)]
        if k == "A" and case_kw.get("a_zero"):
            picks += [(d, 0) for d in range(x["A"].shape[0])]
        for idx in picks:
            xp = {kk: (None if v is None else v.copy()) for kk, v in x.items()}
            xm = {kk: (None if v is None else v.copy()) for kk, v in x.items()}
            v0 = float(x[k][idx])
            if k == "h0":
                step = 1e-6
                xp[k][idx] = v0 + step
                xm[k][idx] = v0 - step
                denom = 2 * step
            else:
                step = np.float32(2.0 ** -10)
                xp[k][idx] = np.float32(v0) + step
                xm[k][idx] = np.float32(v0) - step
                denom = float(xp[k][idx]) - float(xm[k][idx])
            est = (_loss(fwd, xp, W, V, softplus, zoh) - _loss(fwd, xm, W, V, softplus, zoh)) / denom
            got = float(g[k][idx])
            assert abs(est - got) <= 2e-5 * (1 + abs(got)), f"d loss / d {k}{idx}: fd {est} vs {got}"


def torch_grads(x, W, V, softplus, zoh=False):
    """The forward recurrence step by step in torch fp64 on the CPU, differentiated by autograd
    (with ``zoh``, the input coefficient as torch's expm1(dt A) / A: no zero A)."""
    T = {k: (None if x[k] is None else torch.tensor(_widen(x[k]) if k in SEQ else np.asarray(x[k], np.float64),
                                                      dtype=torch.float64, requires_grad=True))
         for k in x}
    u, delta, z, B, C, A = T["u"], T["delta"], T["z"], T["B"], T["C"], T["A"]
    batch, dim, L = u.shape
    N = A.shape[1]
    xb = delta + (T["delta_bias"][None, :, None] if T["delta_bias"] is not None else 0.0)
    dt = torch.nn.functional.softplus(xb, beta=1.0, threshold=1e9) if softplus else torch.exp(xb)
    h = T["h0"] if T["h0"] is not None else torch.zeros(batch, dim, N, dtype=torch.float64)
    ys = []
    for t in range(L):
        a = torch.exp(dt[:, :, t, None] * A[None])                       # (b, d, n)
        if zoh:
            cf = torch.expm1(dt[:, :, t, None] * A[None]) / A[None]
        else:
            cf = dt[:, :, t, None]
        h = a * h + cf * B[:, None, :, t] * u[:, :, t, None]
        y = (h * C[:, None, :, t]).sum(-1)
        if T["D"] is not None:
            y = y + T["D"][None, :] * u[:, :, t]
        if z is not None:
            y = y * torch.nn.functional.silu(z[:, :, t])
        ys.append(y)
    yy = torch.stack(ys, -1)
    loss = (yy * torch.tensor(W)).sum() + (h * torch.tensor(V)).sum()
    loss.backward()
    return {k: T[k].grad.numpy() for k in T if T[k] is not None}


def autograd(bwd, softplus=True, seed=7, zoh=False, **case_kw):
    x, W, V = make_case(seed, **case_kw)
    kw = dict(zoh_b=True) if zoh else {}
    g = bwd(u=x["u"], delta=x["delta"], A=x["A"], B=x["B"], C=x["C"], gy=W, D=x["D"], z=x["z"],
            delta_bias=x["delta_bias"], delta_softplus=softplus, h0=x["h0"], glast=V, **kw)
    ref = torch_grads(x, W, V, softplus, zoh)
    for k, r in ref.items():
        err = np.max(np.abs(g[k] - r) / (1 + np.abs(r)))
        assert err <= 1e-11, f"d loss / d {k}: max rel err {err}"


CASES = [
    dict(softplus=True),
    dict(softplus=False),
    dict(softplus=True, z=False, D=False, bias=False, h0=False),
    dict(softplus=True, bf16=True, N=5, L=11),
    dict(softplus=True, batch=1, dim=2, N=1, L=1),
]

# zero-order hold: the cases above, one with |dt A| below 1/64 (the series branch of dc/dA) and,
# for finite differences only (torch's expm1(x)/A has no value at A = 0), zero A states
ZOH_CASES = CASES + [dict(softplus=True, a_scale=1e-3, L=12)]
ZOH_FD_ONLY = [dict(softplus=True, a_zero=True), dict(softplus=False, a_zero=True, z=False)]
