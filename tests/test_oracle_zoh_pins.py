"""Pins of the oracle's zero-order-hold discretisation of B (``zoh_b=True``):
dB = (e^{dt A} - 1) / A * B per diagonal state, dt * B where A = 0 ("手把手用PyTorch实现Mamba的SSM层…"
§2.1, B_d = A^-1 (e^{A dt} - I) B, for a diagonal A). Each pin checks it against something other
than the oracle: scipy's ``cont2discrete(method='zoh')`` + ``dlsim``, an ODE solver integrating
dh/dt = A h + B u with the input held over each step, and the continuous-time steady state.
Copies of the oracle with one planted slip in the coefficient must fail a pin."""

import os

import numpy as np
import pytest
import scipy.integrate
import scipy.signal

import oracle
from test_oracle_mutants import mutate


def _softplus(x):
    return np.logaddexp(0.0, x)


def _scan(lib=None, **kw):
    return oracle.selective_scan(**kw, zoh_b=True, lib_path=lib)


def pin_lti_matches_scipy_zoh(lib=None):
    """Constant dt, B, C (an LTI system with three diagonal states, one of them A = 0): the scan
    equals scipy's ZOH discretisation simulated by dlsim, for a varying input u."""
    rng = np.random.default_rng(1)
    L, N = 40, 3
    A = np.array([[-0.7, -2.5, 0.0]], np.float32)
    Bv = np.array([0.8, -1.3, 0.6], np.float32)
    Cv = np.array([1.1, 0.4, -0.9], np.float32)
    x = np.float32(0.35)
    dt = float(_softplus(np.float64(x)))
    u = rng.standard_normal(L).astype(np.float32)
    y, ls = _scan(lib, u=u.reshape(1, 1, L), delta=np.full((1, 1, L), x, np.float32), A=A,
                  B=np.repeat(Bv[None, :, None], L, axis=2), C=np.repeat(Cv[None, :, None], L, axis=2),
                  D=np.array([0.3], np.float32), delta_softplus=True)
    Ac = np.diag(A[0].astype(np.float64))
    Dw = float(np.float32(0.3))  # the fp32 skip weight the scan reads
    sysd = scipy.signal.cont2discrete((Ac, Bv.astype(np.float64).reshape(N, 1), Cv.astype(np.float64).reshape(1, N),
                                       np.array([[Dw]])), dt, method="zoh")
    _, yref, xref = scipy.signal.dlsim(sysd[:4] + (dt,), u.astype(np.float64))
    # dlsim's output at t uses the state before the update; the scan's y_t uses the state after
    xnext = np.vstack([xref[1:], (sysd[0] @ xref[-1] + sysd[1][:, 0] * u[-1])])
    ynext = xnext @ Cv.astype(np.float64) + Dw * u.astype(np.float64)
    assert np.allclose(y[0, 0], ynext, rtol=1e-11, atol=1e-12)
    assert np.allclose(ls[0, 0], xnext[-1], rtol=1e-11, atol=1e-12)


def pin_ode_with_held_input(lib=None):
    """Selective (varying dt and B): each step integrates dh/dt = A h + B_t u_t exactly over dt_t."""
    rng = np.random.default_rng(2)
    L, N = 12, 2
    A = np.array([[-1.3, -0.2]], np.float32)
    delta = rng.uniform(-1.5, 1.0, (1, 1, L)).astype(np.float32)
    u = rng.standard_normal((1, 1, L)).astype(np.float32)
    B = rng.standard_normal((1, N, L)).astype(np.float32)
    C = np.zeros((1, N, L), np.float32)
    _, ls = _scan(lib, u=u, delta=delta, A=A, B=B, C=C, delta_softplus=True)
    h = np.zeros(N)
    a = A[0].astype(np.float64)
    for t in range(L):
        dt = float(_softplus(np.float64(delta[0, 0, t])))
        b = B[0, :, t].astype(np.float64) * float(u[0, 0, t])
        sol = scipy.integrate.solve_ivp(lambda _, hh: a * hh + b, (0.0, dt), h, rtol=1e-12, atol=1e-14,
                                        method="DOP853")
        h = sol.y[:, -1]
    assert np.allclose(ls[0, 0], h, rtol=1e-9, atol=1e-12)


def pin_continuous_steady_state(lib=None):
    """Constant input, A < 0: the ZOH state tends to the continuous steady state -B u / A, whatever
    dt is (Euler's dt B u / (1 - e^{dt A}) does not)."""
    L = 3000
    A = np.array([[-0.5, -3.0]], np.float32)
    for x in (-3.0, 0.5):
        _, ls = _scan(lib, u=np.full((1, 1, L), 0.75, np.float32), delta=np.full((1, 1, L), x, np.float32),
                      A=A, B=np.full((1, 2, L), 1.5, np.float32), C=np.zeros((1, 2, L), np.float32),
                      delta_softplus=True)
        assert np.allclose(ls[0, 0], -1.5 * 0.75 / A[0].astype(np.float64), rtol=1e-12), x


def pin_zero_A_is_the_limit(lib=None):
    """A = 0 gives dt B (integration); a tiny A gives nearly the same."""
    rng = np.random.default_rng(4)
    L = 9
    kw = dict(u=rng.standard_normal((1, 1, L)).astype(np.float32),
              delta=rng.standard_normal((1, 1, L)).astype(np.float32),
              B=rng.standard_normal((1, 1, L)).astype(np.float32),
              C=rng.standard_normal((1, 1, L)).astype(np.float32), delta_softplus=True)
    y0, _ = _scan(lib, A=np.zeros((1, 1), np.float32), **kw)
    y1, _ = _scan(lib, A=np.full((1, 1), -1e-7, np.float32), **kw)
    dt = _softplus(kw["delta"][0, 0].astype(np.float64))
    hh = np.cumsum(dt * kw["B"][0, 0] * kw["u"][0, 0])
    assert np.allclose(y0[0, 0], kw["C"][0, 0] * hh, rtol=1e-13, atol=1e-14)
    assert np.allclose(y1[0, 0], y0[0, 0], rtol=1e-5, atol=1e-9)


ALL_PINS = [pin_lti_matches_scipy_zoh, pin_ode_with_held_input, pin_continuous_steady_state,
            pin_zero_A_is_the_limit]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_zoh_pin(pin):
    pin()


def test_euler_is_the_default():
    """Without the flag the scan keeps dt * B: the ZOH result differs."""
    rng = np.random.default_rng(5)
    kw = dict(u=rng.standard_normal((1, 2, 8)).astype(np.float32),
              delta=rng.standard_normal((1, 2, 8)).astype(np.float32),
              A=-rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32),
              B=rng.standard_normal((1, 3, 8)).astype(np.float32),
              C=rng.standard_normal((1, 3, 8)).astype(np.float32), delta_softplus=True)
    ye, _ = oracle.selective_scan(**kw)
    yz, _ = oracle.selective_scan(**kw, zoh_b=True)
    assert not np.allclose(ye, yz, rtol=1e-3)


ZOH_MUTANTS = {
    "missing_minus_one": ("expm1(dt * An) / An", "exp(dt * An) / An"),
    "extra_dt": ("expm1(dt * An) / An", "dt * expm1(dt * An) / An"),
    "zero_A_dropped": ("An == 0.0 ? dt :", "An == 0.0 ? 0.0 :"),
    "divided_by_dt": ("expm1(dt * An) / An", "expm1(dt * An) / dt"),
}


@pytest.mark.parametrize("name", sorted(ZOH_MUTANTS))
def test_zoh_mutant_fails_a_pin(tmp_path, name):
    old, new = ZOH_MUTANTS[name]
    src = open(oracle.SOURCE).read()
    mutant_c = os.path.join(tmp_path, f"{name}.c")
    with open(mutant_c, "w") as f:
        f.write(mutate(src, "static double zoh_coef(", old, new, name))
    lib = oracle.build(force=True, source=mutant_c, out=os.path.join(tmp_path, f"{name}.so"))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"ZOH mutant {name} passed every pin"
