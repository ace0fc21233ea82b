"""CPU tests: the oracle against its pins, and planted mistakes caught by them."""

import os
import types

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.py")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)


# Plausible mistakes, planted in a private copy of the oracle's source.  Each
# must make at least one pin fail; otherwise the pins would not have caught it.
MUTATIONS = {
    "lse_drops_max": ("return m + np.log(np.exp(z - m[:, None]).sum(axis=1))",
                      "return np.log(np.exp(z - m[:, None]).sum(axis=1))"),
    "onehot_sign": ("P[rows[v], y[r0:r1][v]] -= 1.0", "P[rows[v], y[r0:r1][v]] += 1.0"),
    "mean_over_all_rows": ("scale = float(grad) / n_valid", "scale = float(grad) / L"),
    "label_off_by_one": ("z_label[r0:r1][v] = z[rows[v], y[r0:r1][v]]",
                         "z_label[r0:r1][v] = z[rows[v], (y[r0:r1][v] + 1) % V]"),
    "ignored_rows_not_masked": ("P[~v, :] = 0.0\n        G = P * scale", "G = P * scale"),
    "dh_uses_transposed_softmax_scale": ("dh[r0:r1] = G @ W64", "dh[r0:r1] = (G * (1.0 + 1.0 / (1 + np.arange(G.shape[1])))) @ W64"),
    "dW_missing_block": ("dW += G.T @ h64[r0:r1]", "dW = G.T @ h64[r0:r1]"),
    "grad_ignored": ("scale = float(grad) / n_valid", "scale = 1.0 / n_valid"),
    "label_range_drops_negative": ("bad = valid & ((y < 0) | (y >= V))", "bad = valid & (y >= V)"),
    "label_range_off_by_one_at_V": ("bad = valid & ((y < 0) | (y >= V))", "bad = valid & ((y < 0) | (y > V))"),
    "label_range_check_removed": ("    if np.any(bad):\n", "    if False:\n"),
    "cols_dW_grad_ignored": ("scale = float(grad) / float(n_valid)", "scale = 1.0 / float(n_valid)"),
    "cols_dW_onehot_dropped": ("        Gc -= (y[r0:r1, None] == cols[None, :])\n", ""),
    "cols_dW_ignored_rows_kept": ("        Gc[~valid[r0:r1], :] = 0.0\n", ""),
    "cols_dW_first_block_only": ("        dW += (Gc * scale).T @ h64\n", "        dW += (Gc * scale).T @ h64 if r0 == 0 else 0.0\n"),
}


def _mutant(name):
    old, new = MUTATIONS[name]
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, f"mutation {name} does not apply"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(name)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
