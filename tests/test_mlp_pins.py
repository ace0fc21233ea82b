"""CPU tests: the MLP oracle against its pins, and planted mistakes caught by them."""

import os
import types

import numpy as np
import pytest

import oracle.mlp as mlp_oracle
from tests import mlp_pins as pins

SRC = mlp_oracle.__file__

MUTATIONS = {
    "silu_is_sigmoid": ("    a = g * s\n", "    a = s\n"),
    "sigmoid_sign": ("out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))", "out[pos] = 1.0 / (1.0 + np.exp(g[pos]))"),
    "gate_up_swapped": ("_, u, _, a = _block(x64[r0:r1], Wg64, Wu64)", "_, u, _, a = _block(x64[r0:r1], Wu64, Wg64)"),
    "dsilu_missing_term": ("dg = dp * u * s * (1.0 + g * (1.0 - s))", "dg = dp * u * s"),
    "du_uses_gate": ("du = dp * a\n", "du = dp * g\n"),
    "dx_missing_up_term": ("dx[r0:r1] = dg @ Wg64 + du @ Wu64", "dx[r0:r1] = dg @ Wg64"),
    "dWd_overwritten_per_block": ("dWd += dyb.T @ (a * u)", "dWd = dyb.T @ (a * u)"),
    "dWg_from_up": ("dWg += dg.T @ xb", "dWg += du.T @ xb"),
    "dp_transposed_weight": ("dp = dyb @ Wd64\n", "dp = dyb @ Wd64[:, ::-1]\n"),
    "cols_dsilu_missing_term": ("dgc = dpc * uc * s * (1.0 + gc * (1.0 - s))", "dgc = dpc * uc * s"),
    "cols_du_uses_gate": ("duc = dpc * a\n", "duc = dpc * gc\n"),
    "cols_dWd_first_block_only": ("dWdc += dyb.T @ (a * uc)", "dWdc += dyb.T @ (a * uc) if r0 == 0 else 0.0"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"mlp_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("pin", pins.ALL_MLP_PINS, ids=lambda f: f.__name__)
def test_mlp_pin(pin):
    pin(mlp_oracle)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mlp_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in pins.ALL_MLP_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
