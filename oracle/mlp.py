"""CPU oracle for the sequence-tiled MLP block and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library and imports nothing from the ``lm_head_chunked_amd`` package.

What it computes, and where the pages define it
-----------------------------------------------
TRL docs "Training Beyond 1M Tokens", section "One GPU is not enough: split
the sequence across many": one line of the model's MLP,

    down_proj(act_fn(gate_proj(x)) * up_proj(x)),

builds four tensors at the full intermediate width (gate_proj(x), its
activation, up_proj(x) and the product), and at a million tokens on a model
whose MLP widens each token from 2560 to 9728 they take 4 x 19 GB.  TRL PR
#6845 ("Two more that are not assumptions") lists MLP sequence tiling (lever
6) as the fix: the same row-by-row splitting as the chunked loss, applied to
this line, so that those intermediates exist for one block of rows at a
time.  Rows are independent in the forward (each output row depends on its
own input row), and the weight gradients are sums over rows, so a row-tiled
evaluation reaches exactly (up to rounding order) the plain result; this
oracle is that plain definition in float64, with act_fn = SiLU (the
activation of the Qwen3 models the pages train):

  g  = x Wg^T        u = x Wu^T           (L x I; nn.Linear weights Wg, Wu: I x H)
  a  = silu(g) = g * sigmoid(g)
  p  = a * u                              (elementwise)
  y  = p Wd^T                             (L x H; Wd: H x I)

and, for an upstream gradient dy (L x H) of y:

  dWd = dy^T p                  (H x I)
  dp  = dy Wd                   (L x I)
  du  = dp * a
  dg  = dp * u * sigmoid(g) * (1 + g * (1 - sigmoid(g)))     (d silu / d g)
  dx  = dg Wg + du Wu           (L x H)
  dWg = dg^T x,  dWu = du^T x   (I x H)

Inputs are bf16 values given as float32 (or float64) arrays; widening is
exact and every product and sum is carried out in float64, with no rounding
of the intermediates.  ``block_rows`` only bounds memory; the result does not
depend on it beyond float64 rounding order (a property the tests check).

Parity pins (tests/mlp_pins.py): closed forms at Wg = 0 and Wu = 0, PyTorch's
silu/linear with autograd in float64, a 50-digit decimal brute force on tiny
shapes, central finite differences, independence from the row block, and
known values of silu.  No function in this file is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = ["mlp_forward", "mlp_backward", "mlp_fwd_bwd", "mlp_rows_forward", "mlp_rows_dx", "mlp_cols_grads"]


def _widen(a, name):
    a = np.asarray(a)
    if a.dtype not in (np.float32, np.float64):
        raise TypeError(f"{name}: expected float32/float64 holding bf16 values, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def _shapes(x, Wg, Wu, Wd):
    L, H = x.shape
    I = Wg.shape[0]
    if Wg.shape != (I, H) or Wu.shape != (I, H) or Wd.shape != (H, I):
        raise ValueError(f"shapes: x {x.shape}, Wg {Wg.shape}, Wu {Wu.shape}, Wd {Wd.shape}")
    return L, H, I


def _sigmoid(g):
    # 1 / (1 + exp(-g)), written so that exp never overflows
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def _block(x64, Wg64, Wu64):
    g = x64 @ Wg64.T
    u = x64 @ Wu64.T
    s = _sigmoid(g)
    a = g * s
    return g, u, s, a


def mlp_forward(x, Wg, Wu, Wd, block_rows=4096):
    """y = down_proj(silu(gate_proj(x)) * up_proj(x)), float64 [L, H]."""
    x64, Wg64, Wu64, Wd64 = (_widen(t, n) for t, n in ((x, "x"), (Wg, "Wg"), (Wu, "Wu"), (Wd, "Wd")))
    L, H, I = _shapes(x64, Wg64, Wu64, Wd64)
    if block_rows < 1:
        raise ValueError("block_rows must be positive")
    y = np.empty((L, H), dtype=np.float64)
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        _, u, _, a = _block(x64[r0:r1], Wg64, Wu64)
        y[r0:r1] = (a * u) @ Wd64.T
    return y


def mlp_backward(x, Wg, Wu, Wd, dy, block_rows=4096):
    """(dx [L, H], dWg [I, H], dWu [I, H], dWd [H, I]) in float64 for upstream dy [L, H]."""
    x64, Wg64, Wu64, Wd64 = (_widen(t, n) for t, n in ((x, "x"), (Wg, "Wg"), (Wu, "Wu"), (Wd, "Wd")))
    dy64 = _widen(dy, "dy")
    L, H, I = _shapes(x64, Wg64, Wu64, Wd64)
    if dy64.shape != (L, H):
        raise ValueError("dy must have the shape of y")
    dx = np.empty((L, H), dtype=np.float64)
    dWg = np.zeros((I, H), dtype=np.float64)
    dWu = np.zeros((I, H), dtype=np.float64)
    dWd = np.zeros((H, I), dtype=np.float64)
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        xb, dyb = x64[r0:r1], dy64[r0:r1]
        g, u, s, a = _block(xb, Wg64, Wu64)
        dWd += dyb.T @ (a * u)
        dp = dyb @ Wd64
        du = dp * a
        dg = dp * u * s * (1.0 + g * (1.0 - s))
        dx[r0:r1] = dg @ Wg64 + du @ Wu64
        dWg += dg.T @ xb
        dWu += du.T @ xb
    return dx, dWg, dWu, dWd


def mlp_fwd_bwd(x, Wg, Wu, Wd, dy, block_rows=4096):
    """Both: dict with y, dx, dWg, dWu, dWd."""
    y = mlp_forward(x, Wg, Wu, Wd, block_rows=block_rows)
    dx, dWg, dWu, dWd = mlp_backward(x, Wg, Wu, Wd, dy, block_rows=block_rows)
    return {"y": y, "dx": dx, "dWg": dWg, "dWu": dWu, "dWd": dWd}


def mlp_rows_forward(x_rows, Wg, Wu, Wd):
    """y for a subset of rows: each output row depends on its own input row only."""
    return mlp_forward(x_rows, Wg, Wu, Wd, block_rows=max(1, np.asarray(x_rows).shape[0]))


def mlp_rows_dx(x_rows, Wg, Wu, Wd, dy_rows):
    """dx for a subset of rows: each row of dx depends on its own x and dy rows only."""
    return mlp_backward(x_rows, Wg, Wu, Wd, dy_rows, block_rows=max(1, np.asarray(x_rows).shape[0]))[0]


def mlp_cols_grads(x, Wg, Wu, Wd, dy, cols, block_rows=8192):
    """The weight gradients of chosen intermediate units i in cols, over all rows:
    (dWg[cols] [c, H], dWu[cols] [c, H], dWd[:, cols] [H, c]) in float64.

    Unit i's gradients need only its own column of g, u and dp (g_i = x Wg_i,
    u_i = x Wu_i, dp_i = dy Wd[:, i]), so a few units can be checked where the
    whole backward would be too slow.
    """
    x64, Wg64, Wu64, Wd64 = (_widen(t, n) for t, n in ((x, "x"), (Wg, "Wg"), (Wu, "Wu"), (Wd, "Wd")))
    L, H, I = _shapes(x64, Wg64, Wu64, Wd64)
    cols = np.asarray(cols).astype(np.int64, copy=False)
    if np.any((cols < 0) | (cols >= I)):
        raise ValueError("cols must index the intermediate units")
    dy64 = _widen(dy, "dy")
    if dy64.shape != (L, H):
        raise ValueError("dy must have the shape of y")
    Wgc, Wuc, Wdc = Wg64[cols], Wu64[cols], Wd64[:, cols]
    dWgc = np.zeros((cols.shape[0], H), dtype=np.float64)
    dWuc = np.zeros((cols.shape[0], H), dtype=np.float64)
    dWdc = np.zeros((H, cols.shape[0]), dtype=np.float64)
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        xb, dyb = x64[r0:r1], dy64[r0:r1]
        gc, uc, s, a = _block(xb, Wgc, Wuc)
        dWdc += dyb.T @ (a * uc)
        dpc = dyb @ Wdc
        duc = dpc * a
        dgc = dpc * uc * s * (1.0 + gc * (1.0 - s))
        dWgc += dgc.T @ xb
        dWuc += duc.T @ xb
    return dWgc, dWuc, dWdc
