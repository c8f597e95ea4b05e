"""Pins of the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes a ``scan`` callable with the signature of
``oracle.selective_scan`` and raises AssertionError when the scan disagrees with:

* ``pin_brute``   - the non-recursive form of the same sums (O(L^2 N) per row): for a diagonal A the
                    product of per-step decays is exp(A * (S_t - S_s)) with S the running sum of dt;
* ``pin_closed``  - the closed form of a geometric series for constant dt, A, B, C, u;
* ``pin_delta0``  - the delta -> 0 limit (softplus(-1e4) is exactly 0): the state never moves;
* ``pin_hand``    - hand-derived L=1 / L=2 cases (``golden/hand_cases.json``);
* ``pin_lfilter`` - N = 1 with constant dt, B, C is a first-order IIR filter (scipy.signal.lfilter);
* ``pin_cumsum``  - A = 0 makes the state a plain prefix sum (numpy.cumsum);
* ``pin_split``   - scanning 0..L equals scanning 0..L1 then L1..L from the first part's state;
* ``pin_causal``, ``pin_linear``, ``pin_permute`` - invariants of the recurrence;
* ``pin_bf16_widen`` - bf16 bit patterns give the same result as the same values stored as fp32.

The pins are written so that a plausible slip in the oracle (a dropped term, a wrong sign,
index or operand) fails at least one of them; ``test_oracle_mutants.py`` checks exactly that.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.signal import lfilter
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.json")


def rand_case(seed, batch, dim, N, L, z=True, h0=False, softplus=True, bias_scale=1.0):
    """Small random fp32 case drawn with numpy (pins need no link to the workload generator)."""
    rng = np.random.default_rng(seed)
    f = np.float32
    c = dict(
        u=rng.standard_normal((batch, dim, L)).astype(f),
        delta=rng.standard_normal((batch, dim, L)).astype(f),
        A=(-rng.uniform(0.1, 3.0, (dim, N))).astype(f),
        B=rng.standard_normal((batch, N, L)).astype(f),
        C=rng.standard_normal((batch, N, L)).astype(f),
        D=rng.standard_normal(dim).astype(f),
        delta_bias=(bias_scale * rng.standard_normal(dim)).astype(f),
        z=rng.standard_normal((batch, dim, L)).astype(f) if z else None,
        h0=rng.standard_normal((batch, dim, N)) if h0 else None,
        delta_softplus=softplus,
    )
    return c


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def brute_force(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=False, h0=None):
    """y and last state as explicit sums, no recurrence (fp64)."""
    u, delta, A, B, C, D, z, bias, h0 = map(_f64, (u, delta, A, B, C, D, z, delta_bias, h0))
    batch, dim, L = u.shape
    N = A.shape[1]
    x = delta + (bias[None, :, None] if bias is not None else 0.0)
    dt = np.logaddexp(0.0, x) if delta_softplus else np.exp(x)  # ln(1 + e^x) | e^x
    S = np.cumsum(dt, axis=-1)
    y = np.zeros((batch, dim, L))
    last = np.zeros((batch, dim, N))
    tri = np.tril(np.ones((L, L), dtype=bool))  # [t, s]: s <= t
    for b in range(batch):
        for d in range(dim):
            gap = S[b, d][:, None] - S[b, d][None, :]  # S_t - S_s
            drive = dt[b, d] * u[b, d]  # dt_s * u_s
            hist = np.zeros((L, N))  # h_t[n]
            for n in range(N):
                w = np.where(tri, np.exp(A[d, n] * np.where(tri, gap, 0.0)), 0.0)
                hist[:, n] = w @ (drive * B[b, n])
                if h0 is not None:
                    hist[:, n] += np.exp(A[d, n] * S[b, d]) * h0[b, d, n]
            yy = np.einsum("tn,nt->t", hist, C[b])
            if D is not None:
                yy = yy + D[d] * u[b, d]
            if z is not None:
                yy = yy * z[b, d] * expit(z[b, d])
            y[b, d] = yy
            last[b, d] = hist[-1]
    return y, last


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


def pin_brute(scan):
    for seed, shp, kw in [
        (1, (2, 3, 5, 33), {}),
        (2, (1, 2, 4, 17), dict(h0=True)),
        (3, (2, 2, 3, 9), dict(z=False, softplus=False, bias_scale=0.3)),
        (4, (1, 3, 5, 1), dict(h0=True)),
    ]:
        c = rand_case(seed, *shp, **kw)
        y, ls = scan(**c)
        yb, lb = brute_force(**c)
        _close(y, yb, 1e-12, f"brute y {shp} {kw}")
        _close(ls, lb, 1e-12, f"brute last_state {shp} {kw}")


def pin_closed(scan):
    batch, dim, N, L = 1, 2, 3, 40
    dt_x = 0.3  # delta value; dt = softplus(0.3)
    A = np.array([[-0.5, -1.0, 0.0], [-2.0, -0.25, -1.5]], dtype=np.float32)
    Bv = np.array([0.7, -1.2, 0.4], dtype=np.float32)
    Cv = np.array([1.5, 0.5, -2.0], dtype=np.float32)
    uv, Dv = np.float32(0.9), np.array([0.25, -0.75], dtype=np.float32)
    c = dict(
        u=np.full((batch, dim, L), uv, np.float32),
        delta=np.full((batch, dim, L), dt_x, np.float32),
        A=A,
        B=np.repeat(Bv[None, :, None], L, axis=2).astype(np.float32),
        C=np.repeat(Cv[None, :, None], L, axis=2).astype(np.float32),
        D=Dv,
        delta_softplus=True,
    )
    y, ls = scan(**c)
    dt = math.log1p(math.exp(float(np.float32(dt_x))))
    t = np.arange(L)
    for d in range(dim):
        h = np.zeros((L, N))
        for n in range(N):
            a = math.exp(dt * float(A[d, n]))
            drive = dt * float(Bv[n]) * float(uv)
            h[:, n] = (t + 1) * drive if a == 1.0 else drive * (1 - a ** (t + 1)) / (1 - a)
        ref = h @ Cv.astype(np.float64) + float(Dv[d]) * float(uv)
        _close(y[0, d], ref, 1e-13, f"closed form y d={d}")
        _close(ls[0, d], h[-1], 1e-13, f"closed form last_state d={d}")


def pin_delta0(scan):
    c = rand_case(11, 2, 3, 4, 20, z=True, h0=False)
    c["delta"] = np.full_like(c["delta"], -1e4)
    c["delta_bias"] = np.zeros_like(c["delta_bias"])
    y, ls = scan(**c)
    u, z, D = (x.astype(np.float64) for x in (c["u"], c["z"], c["D"]))
    ref = (D[None, :, None] * u) * (z / (1.0 + np.exp(-z)))
    _close(y, ref, 1e-15, "delta->0: y = D*u*silu(z)")
    assert np.array_equal(ls, np.zeros_like(ls)), "delta->0: last_state must stay exactly 0"
    c2 = rand_case(12, 1, 2, 3, 15, z=False, h0=True)
    c2["delta"] = np.full_like(c2["delta"], -1e4)
    c2["delta_bias"] = np.zeros_like(c2["delta_bias"])
    y2, ls2 = scan(**c2)
    assert np.array_equal(ls2, c2["h0"]), "delta->0 with h0: the state must stay h0"
    ref2 = np.einsum("bdn,bnl->bdl", c2["h0"], c2["C"].astype(np.float64)) + (
        c2["D"].astype(np.float64)[None, :, None] * c2["u"].astype(np.float64))
    _close(y2, ref2, 1e-15, "delta->0 with h0: y = C.h0 + D*u")


_SAFE = {"log": math.log, "exp": math.exp, "sqrt": math.sqrt}


def _expr(e):
    return float(eval(e, {"__builtins__": {}}, _SAFE)) if isinstance(e, str) else float(e)


def pin_hand(scan):
    cases = json.load(open(GOLDEN, encoding="utf-8"))["cases"]
    for c in cases:
        f = np.float32
        args = dict(
            u=np.array(c["u"], f), delta=np.array(c["delta"], f),
            z=None if c["z"] is None else np.array(c["z"], f),
            B=np.array(c["B"], f), C=np.array(c["C"], f), A=np.array(c["A"], f),
            D=np.array(c["D"], f), delta_bias=np.array(c["delta_bias"], f),
            delta_softplus=c["softplus"],
        )
        y, ls = scan(**args)
        ey = np.array([[_expr(e) for e in row] for row in c["y"]])
        el = np.array([[_expr(e) for e in row] for row in c["last_state"]])
        _close(y[0], ey, 1e-15, f"hand case {c['name']} y")
        _close(ls[0], el, 1e-15, f"hand case {c['name']} last_state")


def pin_lfilter(scan):
    L = 300
    rng = np.random.default_rng(21)
    for a_val, dx in [(-0.7, 0.2), (-3.0, -1.5), (0.0, 0.0)]:
        u = rng.standard_normal((1, 1, L)).astype(np.float32)
        c = dict(
            u=u, delta=np.full((1, 1, L), dx, np.float32), A=np.array([[a_val]], np.float32),
            B=np.full((1, 1, L), 1.3, np.float32), C=np.full((1, 1, L), -0.6, np.float32),
            D=np.array([0.4], np.float32), delta_softplus=True,
        )
        y, ls = scan(**c)
        dt = math.log1p(math.exp(float(np.float32(dx))))
        pole = math.exp(dt * float(np.float32(a_val)))
        h = lfilter([dt * float(np.float32(1.3))], [1.0, -pole], u[0, 0].astype(np.float64))
        ref = float(np.float32(-0.6)) * h + float(np.float32(0.4)) * u[0, 0].astype(np.float64)
        _close(y[0, 0], ref, 1e-12, f"lfilter A={a_val}")
        _close(ls[0, 0], h[-1:], 1e-12, f"lfilter last A={a_val}")


def pin_cumsum(scan):
    c = rand_case(31, 2, 2, 3, 50, z=False)
    c["A"] = np.zeros_like(c["A"])
    c["D"] = None
    y, ls = scan(**c)
    dt = np.logaddexp(0.0, c["delta"].astype(np.float64) + c["delta_bias"].astype(np.float64)[None, :, None])
    drive = dt * c["u"].astype(np.float64)
    for b in range(2):
        for d in range(2):
            h = np.stack([np.cumsum(drive[b, d] * c["B"][b, n].astype(np.float64)) for n in range(3)], 1)
            _close(y[b, d], np.einsum("tn,nt->t", h, c["C"][b].astype(np.float64)), 1e-12, "cumsum y")
            _close(ls[b, d], h[-1], 1e-12, "cumsum last_state")


def _cut(c, lo, hi):
    out = dict(c)
    for k in ("u", "delta", "z", "B", "C"):
        if out.get(k) is not None:
            out[k] = np.ascontiguousarray(out[k][..., lo:hi])
    return out


def pin_split(scan):
    c = rand_case(41, 2, 3, 4, 37, z=True, h0=True)
    y, ls = scan(**c)
    for L1 in (1, 13, 36):
        a = _cut(c, 0, L1)
        ya, la = scan(**a)
        b = _cut(c, L1, 37)
        b["h0"] = la
        yb, lb = scan(**b)
        assert np.array_equal(np.concatenate([ya, yb], -1), y), f"split at {L1}: y differs"
        assert np.array_equal(lb, ls), f"split at {L1}: last_state differs"


def pin_causal(scan):
    c = rand_case(51, 1, 2, 3, 40)
    y, _ = scan(**c)
    for key, t0 in (("u", 17), ("delta", 5), ("B", 30), ("C", 22), ("z", 9)):
        c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c.items()}
        c2[key][..., t0] += 1.5
        y2, _ = scan(**c2)
        assert np.array_equal(y2[..., :t0], y[..., :t0]), f"causality: {key}@{t0} changed earlier y"
        assert not np.array_equal(y2[..., t0:], y[..., t0:]), f"causality: {key}@{t0} changed nothing"


def pin_linear(scan):
    c = rand_case(61, 2, 2, 3, 30, z=False)
    c["D"] = None
    rng = np.random.default_rng(62)
    # multiples of 1/64 below 8 in size: al*u1 + be*u2 is then exact in fp32
    u1 = (np.round(c["u"] * 64) / 64).astype(np.float32)
    u2 = (np.round(rng.standard_normal(c["u"].shape) * 64) / 64).astype(np.float32)
    al, be = 0.5, -2.0
    y1, _ = scan(**dict(c, u=u1))
    y2, _ = scan(**dict(c, u=u2))
    y12, _ = scan(**dict(c, u=(al * u1 + be * u2).astype(np.float32)))
    _close(y12, al * y1 + be * y2, 1e-12, "linearity in u")


def pin_permute(scan):
    c = rand_case(71, 2, 5, 3, 12, h0=True)
    y, ls = scan(**c)
    perm = np.array([3, 0, 4, 2, 1])
    p = dict(c)
    for k in ("u", "delta", "z", "h0"):
        p[k] = np.ascontiguousarray(c[k][:, perm])
    for k in ("A", "D", "delta_bias"):
        p[k] = np.ascontiguousarray(c[k][perm])
    yp, lp = scan(**p)
    assert np.array_equal(yp, y[:, perm]) and np.array_equal(lp, ls[:, perm]), "row permutation"
    q = dict(c)
    for k in ("u", "delta", "z", "h0", "B", "C"):
        q[k] = np.ascontiguousarray(c[k][::-1])
    yq, lq = scan(**q)
    assert np.array_equal(yq, y[::-1]) and np.array_equal(lq, ls[::-1]), "batch independence"


def pin_bf16_widen(scan):
    c = rand_case(81, 2, 3, 4, 25)
    bits = {}
    for k in ("u", "delta", "z", "B", "C"):
        b32 = c[k].view(np.uint32)
        bits[k] = (b32 >> 16).astype(np.uint16)  # truncated patterns: any bf16 value will do
        c[k] = (bits[k].astype(np.uint32) << 16).view(np.float32)
    y32, l32 = scan(**c)
    y16, l16 = scan(**dict(c, **bits))
    assert np.array_equal(y32, y16) and np.array_equal(l32, l16), "bf16 widening"


ALL_PINS = [pin_brute, pin_closed, pin_delta0, pin_hand, pin_lfilter, pin_cumsum, pin_split,
            pin_causal, pin_linear, pin_permute, pin_bf16_widen]
