"""The upstream oracle (convolution + SiLU, x projection, dt projection) against its pins, and
copies of it with one planted slip each, which must fail at least one pin."""

import os

import pytest

import oracle
import pins_upstream
from test_oracle_mutants import mutate


@pytest.mark.parametrize("pin", pins_upstream.ALL_PINS, ids=lambda p: p.__name__)
def test_upstream_pin(pin):
    pin()


UPSTREAM_MUTANTS = {
    # (function, old, new)
    "kernel_reversed": ("static void conv_row(", "a->conv_w[d * K + k]", "a->conv_w[d * K + (K - 1 - k)]"),
    "one_step_late": ("static void conv_row(", "const int64_t s = t + k - (K - 1);", "const int64_t s = t + k - K;"),
    "conv_bias_dropped": ("static void conv_row(", "a->conv_b ? (double)a->conv_b[d] : 0.0", "0.0"),
    "silu_dropped": ("static void conv_row(", "const double v = silu(acc);", "const double v = acc;"),
    "silu_as_sigmoid": ("static double silu(", "return v / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(-v));"),
    "x_proj_transposed": ("static void xproj_row(", "a->w_x[j * D + d]", "a->w_x[d * J + j]"),
    "dt_rows_from_B": ("static void dtproj_row(", "a->xdbl + (b * J + r) * L", "a->xdbl + (b * J + a->dstate + r) * L"),
    "dt_proj_transposed": ("static void dtproj_row(", "a->w_dt[d * R + r]", "a->w_dt[r * a->dim + d]"),
    "round_toward_zero": ("static uint16_t round_bf16(", "nearbyint(ldexp(v, -q))", "trunc(ldexp(v, -q))"),
    "rounding_one_bit_short": ("static uint16_t round_bf16(", "int q = e - 8;", "int q = e - 7;"),
}


@pytest.mark.parametrize("name", sorted(UPSTREAM_MUTANTS))
def test_upstream_mutant_fails_a_pin(tmp_path, name):
    func, old, new = UPSTREAM_MUTANTS[name]
    src = open(oracle.BLOCK_SOURCE).read()
    mutant_c = os.path.join(tmp_path, f"{name}.c")
    with open(mutant_c, "w") as f:
        f.write(mutate(src, func, old, new, name))
    lib = oracle.build(force=True, source=mutant_c, out=os.path.join(tmp_path, f"{name}.so"))
    failed = []
    for pin in pins_upstream.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"upstream mutant {name} passed every pin"
