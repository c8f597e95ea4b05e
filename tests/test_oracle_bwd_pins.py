"""The fp64 backward oracle against finite differences of the forward oracle and against torch
fp64 autograd of an independent formulation; plus planted slips that these pins must catch."""

import os

import pytest

import oracle
import pins_bwd
from test_oracle_mutants import mutate


@pytest.mark.parametrize("i", range(len(pins_bwd.CASES)))
def test_backward_matches_finite_differences(i):
    if pins_bwd.CASES[i].get("bf16"):
        pytest.skip("inputs held as bf16 bit patterns are not perturbed by finite differences "
                    "(the autograd pin covers this case)")
    pins_bwd.fd(oracle.selective_scan_bwd, oracle.selective_scan, seed=100 + i, **pins_bwd.CASES[i])


@pytest.mark.parametrize("i", range(len(pins_bwd.CASES)))
def test_backward_matches_torch_autograd(i):
    pins_bwd.autograd(oracle.selective_scan_bwd, seed=200 + i, **pins_bwd.CASES[i])


def test_backward_threads_do_not_change_the_result_beyond_rounding():
    import numpy as np

    x, W, V = pins_bwd.make_case(3, batch=3, dim=5, N=4, L=20)
    kw = dict(u=x["u"], delta=x["delta"], A=x["A"], B=x["B"], C=x["C"], gy=W, D=x["D"], z=x["z"],
              delta_bias=x["delta_bias"], delta_softplus=True, h0=x["h0"], glast=V)
    one = oracle.selective_scan_bwd(**kw, nthreads=1)
    many = oracle.selective_scan_bwd(**kw, nthreads=7)
    for k in one:
        assert np.allclose(one[k], many[k], rtol=1e-13, atol=1e-13), k


BWD_MUTANTS = {
    "carry_without_decay": ("lam[n] *= an;", "lam[n] *= 1.0;"),
    "gate_derivative_missing_term": ("(sg + zt * sg * (1.0 - sg))", "(sg)"),
    "gB_without_u": ("j->pB[bc_off + n * L + t] += lam[n] * cf * ut;", "j->pB[bc_off + n * L + t] += lam[n] * cf;"),
    "gdt_without_input_term": ("gdt += lam[n] * (an * hprev[n] * An + cf_dt * Bt * ut);", "gdt += lam[n] * (an * hprev[n] * An);"),
    "gA_with_current_state": ("j->pA[d * N + n] += lam[n] * an * hprev[n] * dt;", "j->pA[d * N + n] += lam[n] * an * h[n] * dt;"),
    "softplus_derivative_as_exp": ("gdt * sigmoid(x) : gdt * dt", "gdt * dt : gdt * dt"),
    "output_grad_added_after_carry": ("lam[n] += gp * Ct;", "lam[n] += 0.0;"),
    "skip_grad_missing": ("double gu = gp * dskip, gdt = 0.0;", "double gu = 0.0, gdt = 0.0;"),
}


@pytest.mark.parametrize("i", range(len(pins_bwd.ZOH_CASES) + len(pins_bwd.ZOH_FD_ONLY)))
def test_zoh_backward_matches_finite_differences(i):
    case = (pins_bwd.ZOH_CASES + pins_bwd.ZOH_FD_ONLY)[i]
    if case.get("bf16"):
        pytest.skip("inputs held as bf16 bit patterns are not perturbed by finite differences "
                    "(the autograd pin covers this case)")
    pins_bwd.fd(oracle.selective_scan_bwd, oracle.selective_scan, seed=400 + i, zoh=True, **case)


@pytest.mark.parametrize("i", range(len(pins_bwd.ZOH_CASES)))
def test_zoh_backward_matches_torch_autograd(i):
    pins_bwd.autograd(oracle.selective_scan_bwd, seed=500 + i, zoh=True, **pins_bwd.ZOH_CASES[i])


def test_zoh_backward_at_zero_A_is_the_euler_one_except_for_A():
    """At A = 0 the hold's coefficient is dt and its derivative in dt is e^0 = 1, so every gradient
    but dA is the Euler one bit for bit; dA keeps the coefficient's derivative in A, dt^2 / 2
    at A = 0 (pinned by finite differences above)."""
    import numpy as np

    x, W, V = pins_bwd.make_case(9, N=3, L=10)
    x["A"][:] = 0.0
    kw = dict(u=x["u"], delta=x["delta"], A=x["A"], B=x["B"], C=x["C"], gy=W, D=x["D"], z=x["z"],
              delta_bias=x["delta_bias"], delta_softplus=True, h0=x["h0"], glast=V, nthreads=1)
    e = oracle.selective_scan_bwd(**kw)
    h = oracle.selective_scan_bwd(**kw, zoh_b=True)
    for k in e:
        if k != "A":
            assert np.array_equal(e[k], h[k]), k
    assert not np.allclose(e["A"], h["A"])


ZOH_MUTANTS = {
    "zoh_gdt_coefficient_derivative_one": ("const double cf_dt = a->zoh_b ? an : 1.0;", "const double cf_dt = 1.0;"),
    "zoh_gA_without_coefficient_term": (
        "if (a->zoh_b) j->pA[d * N + n] += lam[n] * Bt * ut * zoh_coef_dA(dt, An);", ""),
    "zoh_gB_with_dt": ("j->pB[bc_off + n * L + t] += lam[n] * cf * ut;", "j->pB[bc_off + n * L + t] += lam[n] * dt * ut;"),
    "zoh_gu_with_dt": ("gu += lam[n] * cf * Bt;", "gu += lam[n] * dt * Bt;"),
}
ZOH_HELPER_MUTANTS = {
    "zoh_coef_dA_sign": ("return (dt * exp(x) - expm1(x) / An) / An;", "return (dt * exp(x) + expm1(x) / An) / An;"),
    "zoh_coef_dA_series_term": ("x * (1.0 / 3.0 + x", "x * (1.0 / 2.0 + x"),
}


@pytest.mark.parametrize("name", sorted(ZOH_MUTANTS) + sorted(ZOH_HELPER_MUTANTS))
def test_zoh_backward_mutant_fails_a_pin(tmp_path, name):
    old, new = ZOH_MUTANTS.get(name) or ZOH_HELPER_MUTANTS[name]
    src = open(oracle.SOURCE).read()
    head = "static void bwd_row(" if name in ZOH_MUTANTS else "static double zoh_coef_dA("
    mutant_c = os.path.join(tmp_path, f"{name}.c")
    with open(mutant_c, "w") as f:
        f.write(mutate(src, head, old, new, name))
    lib = oracle.build(force=True, source=mutant_c, out=os.path.join(tmp_path, f"{name}.so"))

    def bwd(**kw):
        return oracle.selective_scan_bwd(**kw, lib_path=lib)

    def fwd(**kw):
        return oracle.selective_scan(**kw, lib_path=lib)

    failed = 0
    for i, case in enumerate(pins_bwd.ZOH_CASES[:3] + pins_bwd.ZOH_CASES[-1:]):
        try:
            pins_bwd.autograd(bwd, seed=600 + i, zoh=True, **case)
        except AssertionError:
            failed += 1
    for i, case in enumerate(pins_bwd.ZOH_FD_ONLY):
        try:
            pins_bwd.fd(bwd, fwd, seed=700 + i, zoh=True, **case)
        except AssertionError:
            failed += 1
    assert failed, f"zero-order-hold backward mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_fails_a_pin(tmp_path, name):
    old, new = BWD_MUTANTS[name]
    src = open(oracle.SOURCE).read()
    mutant_c = os.path.join(tmp_path, f"{name}.c")
    with open(mutant_c, "w") as f:
        f.write(mutate(src, "static void bwd_row(", old, new, name))
    lib = oracle.build(force=True, source=mutant_c, out=os.path.join(tmp_path, f"{name}.so"))

    def bwd(**kw):
        return oracle.selective_scan_bwd(**kw, lib_path=lib)

    failed = 0
    for i, case in enumerate(pins_bwd.CASES[:3]):
        try:
            pins_bwd.autograd(bwd, seed=300 + i, **case)
        except AssertionError:
            failed += 1
    assert failed, f"backward mutant {name} passed every pin"
