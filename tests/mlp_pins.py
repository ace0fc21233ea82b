"""Checks that pin the MLP oracle (oracle/mlp.py) to facts other than itself.

Each ``pin_*`` takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when it disagrees with what the
mathematics fixes.  ``test_mlp_pins.py`` runs them on the real oracle and
checks that each planted mistake is caught by at least one pin.

Sources of truth, none of which is the oracle's own code path:
  * closed forms where one weight is zero (Wg = 0: silu(0) = 0 and
    silu'(0) = 1/2; Wu = 0; Wd = 0);
  * PyTorch's linear and silu with autograd, in float64 (library routines);
  * a 50-digit decimal brute force on tiny shapes;
  * central finite differences of <dy, y>;
  * known values of silu(v) = v / (1 + e^-v) and of its derivative;
  * independence from the row block (the sequence tiling itself).
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import torch


def _case(L, H, I, seed, scale_x=1.0, w_std=0.2, bf16=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((L, H)) * scale_x
    Wg = rng.standard_normal((I, H)) * w_std
    Wu = rng.standard_normal((I, H)) * w_std
    Wd = rng.standard_normal((H, I)) * w_std
    dy = rng.standard_normal((L, H))
    out = []
    for a in (x, Wg, Wu, Wd, dy):
        a = a.astype(np.float32)
        if bf16:
            a = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
        out.append(a)
    return out


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(1e-300, np.linalg.norm(b)))


def _silu_t(t):
    return torch.nn.functional.silu(t)


# ------------------------------------------------------------------ closed forms
def pin_mlp_zero_weights(orc):
    """Wg = 0: y = 0, dx = 0, dWu = 0, dWd = 0, dWg = 1/2 ((dy Wd) * (x Wu^T))^T x.
    Wu = 0: y = 0, dx = 0, dWg = 0, dWd = 0, dWu = ((dy Wd) * silu(x Wg^T))^T x.
    Wd = 0: y = 0, dx = dWg = dWu = 0, dWd = dy^T (silu(x Wg^T) * x Wu^T)."""
    x, Wg, Wu, Wd, dy = (a.astype(np.float64) for a in _case(9, 8, 12, seed=1))
    xt, Wgt, Wut, Wdt, dyt = (torch.from_numpy(a) for a in (x, Wg, Wu, Wd, dy))
    Z = np.zeros_like
    o = orc.mlp_fwd_bwd(x, Z(Wg), Wu, Wd, dy)
    assert np.all(o["y"] == 0) and np.all(o["dx"] == 0) and np.all(o["dWu"] == 0) and np.all(o["dWd"] == 0)
    expect = 0.5 * ((dy @ Wd) * (x @ Wu.T)).T @ x
    assert _rel(o["dWg"], expect) <= 1e-13, "dWg at Wg = 0"
    o = orc.mlp_fwd_bwd(x, Wg, Z(Wu), Wd, dy)
    assert np.all(o["y"] == 0) and np.all(o["dx"] == 0) and np.all(o["dWg"] == 0) and np.all(o["dWd"] == 0)
    expect = ((dy @ Wd) * _silu_t(xt @ Wgt.T).numpy()).T @ x
    assert _rel(o["dWu"], expect) <= 1e-13, "dWu at Wu = 0"
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Z(Wd), dy)
    assert np.all(o["y"] == 0) and np.all(o["dx"] == 0) and np.all(o["dWg"] == 0) and np.all(o["dWu"] == 0)
    expect = dy.T @ (_silu_t(xt @ Wgt.T).numpy() * (x @ Wu.T))
    assert _rel(o["dWd"], expect) <= 1e-13, "dWd at Wd = 0"


def pin_mlp_silu_values(orc):
    """With H = 2, x = [v, 1], Wg = [[1, 0]], Wu = [[0, 1]], Wd = [[1], [0]]:
    y[:, 0] = silu(v); with dy = [1, 0], dx[:, 0] = silu'(v).  Known values:
    sigmoid(1) = 0.7310585786300049, sigmoid(2) = 0.8807970779778823,
    silu'(v) = sigmoid(v) (1 + v (1 - sigmoid(v))), silu'(0) = 1/2."""
    v = np.array([0.0, 1.0, -1.0, 2.0, -30.0, 40.0])
    x = np.stack([v, np.ones_like(v)], axis=1)
    Wg = np.array([[1.0, 0.0]])
    Wu = np.array([[0.0, 1.0]])
    Wd = np.array([[1.0], [0.0]])
    dy = np.stack([np.ones_like(v), np.zeros_like(v)], axis=1)
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy)
    s1, s2 = 0.7310585786300049, 0.8807970779778823
    silu = [0.0, s1, -(1 - s1), 2 * s2, -30.0 / (1.0 + math.exp(30.0)), 40.0]
    dsilu = [0.5, s1 * (1 + (1 - s1)), (1 - s1) * (1 - (1 - (1 - s1))), s2 * (1 + 2 * (1 - s2)), None, 1.0]
    for i in range(len(v)):
        assert abs(o["y"][i, 0] - silu[i]) <= 1e-15 * max(1.0, abs(silu[i])), (v[i], o["y"][i, 0])
        if dsilu[i] is not None:
            assert abs(o["dx"][i, 0] - dsilu[i]) <= 1e-12, (v[i], o["dx"][i, 0])
    assert abs(o["dx"][4, 0]) < 1e-11  # silu' is tiny far to the left


# ------------------------------------------------------------------ library
def pin_mlp_torch_autograd(orc):
    """torch.nn.functional.linear / silu with autograd in float64."""
    for (L, H, I, seed) in [(7, 16, 24, 2), (40, 32, 64, 3)]:
        x, Wg, Wu, Wd, dy = _case(L, H, I, seed)
        o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy, block_rows=5)
        t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, Wg, Wu, Wd)]
        F = torch.nn.functional
        y = F.linear(F.silu(F.linear(t[0], t[1])) * F.linear(t[0], t[2]), t[3])
        g = torch.autograd.grad(y, t, torch.tensor(dy, dtype=torch.float64))
        assert _rel(o["y"], y.detach().numpy()) <= 1e-13, "y vs torch"
        for name, ref in zip(("dx", "dWg", "dWu", "dWd"), g):
            assert _rel(o[name], ref.numpy()) <= 1e-13, f"{name} vs torch autograd"


# ------------------------------------------------------------------ brute force
def pin_mlp_decimal(orc):
    """Every output against a 50-digit decimal evaluation of the definition."""
    getcontext().prec = 50
    L, H, I = 3, 4, 5
    x, Wg, Wu, Wd, dy = _case(L, H, I, seed=4, w_std=0.8)
    D = lambda a: [[Decimal(float(v)) for v in row] for row in a]
    xd, Wgd, Wud, Wdd, dyd = D(x), D(Wg), D(Wu), D(Wd), D(dy)
    one = Decimal(1)
    g = [[sum(xd[r][k] * Wgd[i][k] for k in range(H)) for i in range(I)] for r in range(L)]
    u = [[sum(xd[r][k] * Wud[i][k] for k in range(H)) for i in range(I)] for r in range(L)]
    s = [[one / (one + (-g[r][i]).exp()) for i in range(I)] for r in range(L)]
    p = [[g[r][i] * s[r][i] * u[r][i] for i in range(I)] for r in range(L)]
    y = [[sum(p[r][i] * Wdd[h][i] for i in range(I)) for h in range(H)] for r in range(L)]
    dp = [[sum(dyd[r][h] * Wdd[h][i] for h in range(H)) for i in range(I)] for r in range(L)]
    du = [[dp[r][i] * g[r][i] * s[r][i] for i in range(I)] for r in range(L)]
    dg = [[dp[r][i] * u[r][i] * s[r][i] * (one + g[r][i] * (one - s[r][i])) for i in range(I)] for r in range(L)]
    dx = [[sum(dg[r][i] * Wgd[i][k] + du[r][i] * Wud[i][k] for i in range(I)) for k in range(H)] for r in range(L)]
    dWg = [[sum(dg[r][i] * xd[r][k] for r in range(L)) for k in range(H)] for i in range(I)]
    dWu = [[sum(du[r][i] * xd[r][k] for r in range(L)) for k in range(H)] for i in range(I)]
    dWd = [[sum(dyd[r][h] * p[r][i] for r in range(L)) for i in range(I)] for h in range(H)]
    f = lambda a: np.array([[float(v) for v in row] for row in a])
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy)
    for name, ref in (("y", y), ("dx", dx), ("dWg", dWg), ("dWu", dWu), ("dWd", dWd)):
        assert np.max(np.abs(o[name] - f(ref))) <= 1e-12, f"{name} vs decimal brute force"


# ------------------------------------------------------------------ finite differences
def pin_mlp_finite_differences(orc):
    """Central differences (eps = 1e-6) of f = <dy, y> for every input."""
    L, H, I = 3, 4, 5
    x, Wg, Wu, Wd, dy = (a.astype(np.float64) for a in _case(L, H, I, seed=5, bf16=False))
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy)
    f = lambda args: float((dy * orc.mlp_forward(*args)).sum())
    args = [x, Wg, Wu, Wd]
    eps = 1e-6
    for k, name in enumerate(("dx", "dWg", "dWu", "dWd")):
        fd = np.zeros_like(args[k])
        for idx in np.ndindex(*args[k].shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[k][idx] += eps
            am[k][idx] -= eps
            fd[idx] = (f(ap) - f(am)) / (2 * eps)
        assert _rel(o[name], fd) <= 1e-7, f"{name} vs finite differences: {_rel(o[name], fd)}"


# ------------------------------------------------------------------ tiling
def pin_mlp_row_blocks(orc):
    """Any row block gives the untiled result (the sequence tiling)."""
    x, Wg, Wu, Wd, dy = _case(23, 8, 16, seed=6)
    ref = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy, block_rows=23)
    for b in (1, 3, 7, 1000):
        o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy, block_rows=b)
        for k in ("y", "dx", "dWg", "dWu", "dWd"):
            assert np.max(np.abs(o[k] - ref[k])) <= 1e-12 * max(1.0, np.max(np.abs(ref[k]))), (b, k)


def pin_mlp_row_helpers(orc):
    """The row-subset helpers agree with the full arrays."""
    x, Wg, Wu, Wd, dy = _case(12, 8, 16, seed=7)
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy)
    rows = np.array([0, 3, 11])
    assert np.max(np.abs(orc.mlp_rows_forward(x[rows], Wg, Wu, Wd) - o["y"][rows])) <= 1e-13
    assert np.max(np.abs(orc.mlp_rows_dx(x[rows], Wg, Wu, Wd, dy[rows]) - o["dx"][rows])) <= 1e-13


def pin_mlp_col_helper(orc):
    """The chosen-unit weight-gradient helper agrees with the full arrays, for
    the first, last and inner units and row blocks that split the rows
    unevenly."""
    x, Wg, Wu, Wd, dy = _case(29, 8, 16, seed=8)
    o = orc.mlp_fwd_bwd(x, Wg, Wu, Wd, dy)
    cols = np.array([0, 5, 6, 15])
    for b in (4, 8192):
        dWg, dWu, dWd = orc.mlp_cols_grads(x, Wg, Wu, Wd, dy, cols, block_rows=b)
        for got, ref in ((dWg, o["dWg"][cols]), (dWu, o["dWu"][cols]), (dWd, o["dWd"][:, cols])):
            assert np.max(np.abs(got - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), b


ALL_MLP_PINS = [
    pin_mlp_zero_weights,
    pin_mlp_silu_values,
    pin_mlp_torch_autograd,
    pin_mlp_decimal,
    pin_mlp_finite_differences,
    pin_mlp_row_blocks,
    pin_mlp_row_helpers,
    pin_mlp_col_helper,
]
