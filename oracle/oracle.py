"""CPU oracle for the LM-head + cross-entropy (NLL) loss and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
the ``lm_head_chunked_amd`` package.

What it computes, and where the pages define it
-----------------------------------------------
TRL docs "Training Beyond 1M Tokens", section "The loss is the first thing
to break": the last decoder layer gives a hidden state h of shape L x H; it is
multiplied by the language-modelling head weights to give logits of shape
L x V, and the loss is the cross entropy of those logits against the target
labels.

Same page, section "The massive logits matrix: chunk it": the loss is a sum
over rows and the softmax of one row runs over that row's vocabulary only, so
a block of rows carries everything its own loss needs and the per-block
pieces add up to the whole.  The chunked method therefore reaches exactly
(up to rounding order) the plain full-logits result, and this oracle is that
plain definition written out in float64:

  z_i     = W h_i                                  (row i of the logits)
  lse_i   = log sum_v exp(z_iv)                    (computed with a max shift)
  valid_i = [y_i != ignore_index]
  N       = sum_i valid_i
  nll_i   = lse_i - z_{i, y_i}                     (valid rows only)
  loss    = (sum_{valid i} nll_i) / N              (mean over non-ignored rows)
  G_iv    = (g / N) * valid_i * (softmax(z_i)_v - [v == y_i])
  dh      = G W          (L x H)
  dW      = G^T h        (V x H)

g is the upstream gradient of the scalar loss (1 for a plain backward).

Readings taken where the pages are silent (each one is listed in the design
notes of the repository):
  * mean over non-ignored rows, divided by the count N of those rows;
  * labels are already shifted: labels[i] is the target of row i;
  * ignored rows still get an lse value (the forward runs every row), and
    their nll, dh row and dW contribution are exactly zero;
  * N == 0 gives loss = NaN and dh = dW = 0;
  * a non-ignored label outside [0, V) is an error;
  * no bias, temperature, soft-capping, label smoothing or z-loss.

Inputs are the bf16 values of h and W given as float32 (or float64) arrays;
widening bf16 to float64 is exact, and every product and sum below is
carried out in float64.  The rows are processed ``block_rows`` at a time
only to bound memory; the result does not depend on that block size beyond
float64 rounding order (a property the tests check).

Parity pins: every function here is pinned by CPU tests against closed forms
(W = 0), a brute-force high-precision evaluation at V <= 64, PyTorch's
cross_entropy with autograd in float64, central finite differences,
invariants (column sums of dW, vocab shifts, permutations, ignored rows) and
a statistical sanity check, and the label-range check by labels outside [0, V)
that must raise.  No function in this file is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "forward",
    "backward",
    "fwd_bwd",
    "rows_forward",
    "rows_dh",
    "cols_dW",
]


def _widen(x, name):
    a = np.asarray(x)
    if a.dtype not in (np.float32, np.float64):
        raise TypeError(f"{name}: expected float32/float64 holding bf16 values, got {a.dtype}")
    return a.astype(np.float64, copy=False)


def _check_labels(labels, V, ignore_index):
    y = np.asarray(labels).astype(np.int64, copy=False)
    valid = y != ignore_index
    bad = valid & ((y < 0) | (y >= V))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"label {int(y[i])} at row {i} is outside [0, {V}) and is not ignore_index")
    return y, valid


def _block_logits(h64, W64, r0, r1):
    # z = h W^T for rows r0..r1-1, every vocabulary entry (no tiling over V).
    return h64[r0:r1] @ W64.T


def _logsumexp_rows(z):
    # lse_i = m_i + log sum_v exp(z_iv - m_i), m_i = max_v z_iv.
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def forward(h, W, labels, ignore_index=-100, block_rows=512):
    """Mean NLL loss, per-row logsumexp and per-row nll of the full logits.

    Returns a dict with ``loss`` (float, NaN when no row is valid), ``lse``
    (float64 [L], every row), ``nll`` (float64 [L], zero on ignored rows),
    ``n_valid`` (int).
    """
    h64 = _widen(h, "h")
    W64 = _widen(W, "W")
    L, H = h64.shape
    V, H2 = W64.shape
    if H != H2:
        raise ValueError("h and W disagree on the hidden size")
    y, valid = _check_labels(labels, V, ignore_index)
    if block_rows < 1:
        raise ValueError("block_rows must be positive")

    lse = np.empty(L, dtype=np.float64)
    z_label = np.zeros(L, dtype=np.float64)
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        z = _block_logits(h64, W64, r0, r1)
        lse[r0:r1] = _logsumexp_rows(z)
        rows = np.arange(r1 - r0)
        v = valid[r0:r1]
        z_label[r0:r1][v] = z[rows[v], y[r0:r1][v]]

    n_valid = int(valid.sum())
    nll = np.where(valid, lse - z_label, 0.0)
    loss = float(nll[valid].sum() / n_valid) if n_valid > 0 else float("nan")
    return {"loss": loss, "lse": lse, "nll": nll, "n_valid": n_valid}


def backward(h, W, labels, ignore_index=-100, grad=1.0, block_rows=512):
    """Gradients dh (float64 [L,H]) and dW (float64 [V,H]) of grad * loss.

    The logits are recomputed block by block (they are never kept whole);
    G = (grad / N) * valid * (softmax - onehot) is formed per block and
    multiplied into dh = G W and dW += G^T h.
    """
    h64 = _widen(h, "h")
    W64 = _widen(W, "W")
    L, H = h64.shape
    V = W64.shape[0]
    y, valid = _check_labels(labels, V, ignore_index)
    n_valid = int(valid.sum())
    dh = np.zeros((L, H), dtype=np.float64)
    dW = np.zeros((V, H), dtype=np.float64)
    if n_valid == 0:
        return dh, dW
    scale = float(grad) / n_valid
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        z = _block_logits(h64, W64, r0, r1)
        lse = _logsumexp_rows(z)
        P = np.exp(z - lse[:, None])
        rows = np.arange(r1 - r0)
        v = valid[r0:r1]
        P[rows[v], y[r0:r1][v]] -= 1.0
        P[~v, :] = 0.0
        G = P * scale
        dh[r0:r1] = G @ W64
        dW += G.T @ h64[r0:r1]
    return dh, dW


def fwd_bwd(h, W, labels, ignore_index=-100, grad=1.0, block_rows=512):
    """forward() and backward() together: dict with loss, lse, nll, n_valid, dh, dW."""
    out = forward(h, W, labels, ignore_index=ignore_index, block_rows=block_rows)
    dh, dW = backward(h, W, labels, ignore_index=ignore_index, grad=grad, block_rows=block_rows)
    out["dh"] = dh
    out["dW"] = dW
    return out


def rows_forward(h_rows, W, labels_rows, ignore_index=-100):
    """lse and nll for a subset of rows (the same definition row by row).

    Used for sampled parity at sizes where the full oracle is too slow: every
    row's lse and nll depend on that row alone.
    """
    h64 = _widen(h_rows, "h_rows")
    W64 = _widen(W, "W")
    V = W64.shape[0]
    y, valid = _check_labels(labels_rows, V, ignore_index)
    z = h64 @ W64.T
    lse = _logsumexp_rows(z)
    rows = np.arange(h64.shape[0])
    zy = np.zeros(h64.shape[0])
    zy[valid] = z[rows[valid], y[valid]]
    nll = np.where(valid, lse - zy, 0.0)
    return lse, nll


def rows_dh(h_rows, W, labels_rows, n_valid, ignore_index=-100, grad=1.0):
    """dh for a subset of rows, given the global count N of non-ignored rows.

    dh_i = (grad / N) * valid_i * (softmax(z_i) - e_{y_i}) W depends on row i
    and on N only.
    """
    h64 = _widen(h_rows, "h_rows")
    W64 = _widen(W, "W")
    V = W64.shape[0]
    y, valid = _check_labels(labels_rows, V, ignore_index)
    z = h64 @ W64.T
    P = np.exp(z - _logsumexp_rows(z)[:, None])
    rows = np.arange(h64.shape[0])
    P[rows[valid], y[valid]] -= 1.0
    P[~valid, :] = 0.0
    if n_valid <= 0:
        return np.zeros_like(h64)
    return (P * (float(grad) / n_valid)) @ W64


def cols_dW(h, W_cols, labels, cols, lse, V, ignore_index=-100, grad=1.0, block_rows=8192):
    """Rows `cols` of dW (the given vocabulary entries), from every row's lse.

    dW_v = sum_i G_iv h_i, G_iv = (grad / N) * valid_i * (exp(z_iv - lse_i) - [v == y_i]):
    column v of G needs z_iv = W_v . h_i for every row i and that row's lse
    (forward() gives it), so a few vocabulary entries can be checked where the
    whole dW would be too slow.  W_cols holds the rows of W at `cols`; V is the
    vocabulary size, for the label check.  h is widened block by block.
    """
    W64 = _widen(W_cols, "W_cols")
    cols = np.asarray(cols).astype(np.int64, copy=False)
    if W64.shape[0] != cols.shape[0] or np.any((cols < 0) | (cols >= V)):
        raise ValueError("cols must index W's rows, one per row of W_cols")
    y, valid = _check_labels(labels, V, ignore_index)
    lse = np.asarray(lse, dtype=np.float64)
    L = y.shape[0]
    n_valid = int(valid.sum())
    dW = np.zeros((cols.shape[0], W64.shape[1]), dtype=np.float64)
    if n_valid == 0:
        return dW
    scale = float(grad) / float(n_valid)
    for r0 in range(0, L, block_rows):
        r1 = min(L, r0 + block_rows)
        h64 = _widen(h[r0:r1], "h")
        Gc = np.exp(h64 @ W64.T - lse[r0:r1, None])
        Gc -= (y[r0:r1, None] == cols[None, :])
        Gc[~valid[r0:r1], :] = 0.0
        dW += (Gc * scale).T @ h64
    return dW
