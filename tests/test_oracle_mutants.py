"""The pins are sharp: copies of the oracle with one planted slip each must fail a pin.

Each mutant is a textual edit of a copy of ``oracle/scan_oracle.c`` compiled into a temporary
library on the CPU; the oracle itself is never modified. Forward mutants edit the forward row
function only (the backward repeats some of its expressions).
"""

import os

import pytest

import pins

MUTANTS = {
    "drop_skip": ("double v = acc + dskip * ut;", "double v = acc;"),
    "sign_of_decay": ("exp(dt * An)", "exp(-dt * An)"),
    "B_for_C": ("acc += Ct * h[n];", "acc += Bt * h[n];"),
    "C_one_step_late": ("widen(a->C, a->in_dtype, bc_off + n * L + t)",
                        "widen(a->C, a->in_dtype, bc_off + n * L + (t > 0 ? t - 1 : t))"),
    "A_transposed": ("a->A[d * N + n]", "a->A[n * D + d]"),
    "gate_sigmoid_only": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "softplus_exp_swapped": ("a->delta_softplus ? softplus(x) : exp(x)",
                             "a->delta_softplus ? exp(x) : softplus(x)"),
    "bias_dropped": ("widen(a->delta, a->in_dtype, row_off + t) + bias;",
                     "widen(a->delta, a->in_dtype, row_off + t);"),
    "dt_missing_from_input": ("a->zoh_b ? zoh_coef(dt, An) : dt;", "a->zoh_b ? zoh_coef(dt, An) : 1.0;"),
    "output_before_update": ("h[n] = dA * h[n] + dB * Bt * ut;\n            acc += Ct * h[n];",
                             "acc += Ct * h[n];\n            h[n] = dA * h[n] + dB * Bt * ut;"),
    "h0_ignored": ("h[n] = a->h0 ? a->h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    "gate_on_u": ("if (a->z) v *= silu(widen(a->z,", "if (a->z) v *= silu(widen(a->u,"),
    "bf16_widen_shift": ("(uint32_t)((const uint16_t*)p)[i] << 16", "(uint32_t)((const uint16_t*)p)[i] << 15"),
    "softplus_no_log1p": ("fmax(x, 0.0) + log1p(exp(-fabs(x)))", "fmax(x, 0.0) + exp(-fabs(x))"),
    "B_batch_stride_missing": ("const int64_t bc_off = b * N * L;", "const int64_t bc_off = 0;"),
}


# mutants of the shared helpers are scoped to the helper itself
HELPER_SCOPE = {
    "gate_sigmoid_only": "static double silu(",
    "bf16_widen_shift": "static double widen(",
    "softplus_no_log1p": "static double softplus(",
}


def mutate(src, func_head, old, new, name):
    """Replace `old` by `new` inside the body of the function starting at `func_head` (the site
    must occur there exactly once)."""
    a = src.index(func_head)
    b = src.index("\n}\n", a) + 3
    body = src[a:b]
    assert body.count(old) == 1, f"mutation site for {name} not found exactly once"
    return src[:a] + body.replace(old, new) + src[b:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_some_pin(oracle_mod, tmp_path, name):
    old, new = MUTANTS[name]
    src = open(oracle_mod.SOURCE).read()
    mutant_c = os.path.join(tmp_path, f"{name}.c")
    with open(mutant_c, "w") as f:
        f.write(mutate(src, HELPER_SCOPE.get(name, "static void scan_row("), old, new, name))
    lib = oracle_mod.build(force=True, source=mutant_c, out=os.path.join(tmp_path, f"{name}.so"))

    def scan(**kw):
        return oracle_mod.selective_scan(**kw, lib_path=lib)

    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(scan)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
