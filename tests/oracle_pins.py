"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an oracle module (the real one, or a copy with
a planted mistake) and raises AssertionError when the oracle disagrees with
what the mathematics fixes.  ``test_oracle_pins.py`` runs them on the real
oracle and checks that each planted mistake is caught by at least one pin.

Sources of truth used here, none of which is the oracle's own code path:
  * closed forms (W = 0 gives a uniform softmax: lse = ln V, dh = 0 and a
    closed-form dW);
  * a brute-force evaluation in 50-digit decimal arithmetic at V <= 16;
  * PyTorch's cross_entropy / logsumexp and autograd, in float64;
  * central finite differences of the oracle's own loss;
  * invariants (sum over the vocabulary of dW is zero, a common shift of
    every W row changes lse by h.c and leaves the loss alone, permutations,
    ignored rows contribute nothing);
  * a statistical law for random W (lse ~ ln V + sigma^2 |h|^2 / 2).
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import torch

IGN = -100


def _case(L, H, V, seed, ignore=(), h_scale=1.0, w_std=0.3, bf16=True):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((L, H)).astype(np.float32) * h_scale
    W = rng.standard_normal((V, H)).astype(np.float32) * w_std
    if bf16:
        h = torch.from_numpy(h).to(torch.bfloat16).float().numpy()
        W = torch.from_numpy(W).to(torch.bfloat16).float().numpy()
    y = rng.integers(0, V, size=L).astype(np.int64)
    for i in ignore:
        y[i] = IGN
    return h, W, y


# --------------------------------------------------------------------- P1
def pin_zero_weights(orc):
    """W = 0: every logit is 0, so softmax is uniform: lse = ln V, loss = ln V,
    dh = 0 and dW[v] = (g/N) (sum_valid h_i / V - sum_{valid, y_i = v} h_i)."""
    for (L, H, V) in [(37, 16, 50), (64, 32, 4096)]:
        h, _, y = _case(L, H, V, seed=1, ignore=(0, 5, 6))
        W = np.zeros((V, H), np.float32)
        g = 0.75
        out = orc.fwd_bwd(h, W, y, grad=g)
        lnV = math.log(V)
        assert np.max(np.abs(out["lse"] - lnV)) <= 1e-12, "lse != ln V at W = 0"
        assert abs(out["loss"] - lnV) <= 1e-12, "loss != ln V at W = 0"
        assert np.all(out["dh"] == 0.0), "dh != 0 at W = 0"
        valid = y != IGN
        N = int(valid.sum())
        h64 = h.astype(np.float64)
        expect = np.tile(h64[valid].sum(0) / V, (V, 1))
        for i in np.flatnonzero(valid):
            expect[y[i]] -= h64[i]
        expect *= g / N
        err = np.max(np.abs(out["dW"] - expect)) / max(1e-300, np.max(np.abs(expect)))
        assert err <= 1e-12, f"dW closed form at W = 0: rel err {err}"


# --------------------------------------------------------------------- P2
def _dec_case_outputs(h, W, y, g):
    """Brute force in 50-digit decimal: z, lse, nll, loss, dh, dW."""
    getcontext().prec = 50
    L, H = h.shape
    V = W.shape[0]
    hd = [[Decimal(float(h[i, k])) for k in range(H)] for i in range(L)]
    Wd = [[Decimal(float(W[v, k])) for k in range(H)] for v in range(V)]
    z = [[sum(hd[i][k] * Wd[v][k] for k in range(H)) for v in range(V)] for i in range(L)]
    lse = []
    for i in range(L):
        s = sum(zz.exp() for zz in z[i])  # no max shift: exact enough at 50 digits
        lse.append(s.ln())
    valid = [int(y[i]) != IGN for i in range(L)]
    N = sum(valid)
    nll = [lse[i] - z[i][int(y[i])] if valid[i] else Decimal(0) for i in range(L)]
    loss = sum(nll) / N
    G = [[Decimal(0)] * V for _ in range(L)]
    gd = Decimal(g)
    for i in range(L):
        if not valid[i]:
            continue
        for v in range(V):
            p = (z[i][v] - lse[i]).exp()
            G[i][v] = gd / N * (p - (1 if v == int(y[i]) else 0))
    dh = [[sum(G[i][v] * Wd[v][k] for v in range(V)) for k in range(H)] for i in range(L)]
    dW = [[sum(G[i][v] * hd[i][k] for i in range(L)) for k in range(H)] for v in range(V)]
    f = lambda a: np.array([[float(x) for x in r] for r in a]) if isinstance(a[0], list) else np.array([float(x) for x in a])
    return {"lse": f(lse), "nll": f(nll), "loss": float(loss), "dh": f(dh), "dW": f(dW)}


def pin_bruteforce_decimal(orc):
    """V <= 16: every output against a 50-digit brute force."""
    for (L, H, V, ign, seed) in [(4, 3, 5, (2,), 2), (6, 8, 16, (0, 4), 3), (3, 5, 1, (), 4)]:
        h, W, y = _case(L, H, V, seed, ignore=ign, w_std=0.7)
        g = 1.25
        ref = _dec_case_outputs(h, W, y, g)
        out = orc.fwd_bwd(h, W, y, grad=g)
        assert np.max(np.abs(out["lse"] - ref["lse"])) <= 1e-12, "lse vs brute force"
        assert np.max(np.abs(out["nll"] - ref["nll"])) <= 1e-12, "nll vs brute force"
        assert abs(out["loss"] - ref["loss"]) <= 1e-12, "loss vs brute force"
        assert np.max(np.abs(out["dh"] - ref["dh"])) <= 1e-12, "dh vs brute force"
        assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-12, "dW vs brute force"


# --------------------------------------------------------------------- P3
def pin_torch_cross_entropy(orc):
    """PyTorch float64 cross_entropy + autograd, logsumexp (library routine)."""
    for (L, H, V, ign, seed) in [(33, 24, 70, (1, 7, 30), 5), (128, 64, 512, tuple(range(0, 128, 9)), 6)]:
        h, W, y = _case(L, H, V, seed, ignore=ign)
        g = 2.0
        out = orc.fwd_bwd(h, W, y, grad=g)
        ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
        Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
        z = ht @ Wt.T
        loss = torch.nn.functional.cross_entropy(z, torch.tensor(y), ignore_index=IGN, reduction="mean")
        dh, dW = torch.autograd.grad(loss * g, (ht, Wt))
        lse = torch.logsumexp(z, dim=1).detach().numpy()
        rel = lambda a, b: np.linalg.norm(a - b) / max(1e-300, np.linalg.norm(b))
        assert abs(out["loss"] - loss.item()) <= 1e-12 * abs(loss.item()), "loss vs torch"
        assert np.max(np.abs(out["lse"] - lse)) <= 1e-12, "lse vs torch"
        assert rel(out["dh"], dh.numpy()) <= 1e-12, "dh vs torch autograd"
        assert rel(out["dW"], dW.numpy()) <= 1e-12, "dW vs torch autograd"


# --------------------------------------------------------------------- P4
def pin_finite_differences(orc):
    """Central differences of the oracle's loss (float64, eps = 1e-6)."""
    L, H, V = 5, 6, 11
    h, W, y = _case(L, H, V, seed=7, ignore=(3,), bf16=False)
    h = h.astype(np.float64)
    W = W.astype(np.float64)
    g = 1.0
    out = orc.fwd_bwd(h, W, y, grad=g)
    eps = 1e-6

    def loss_at(hh, WW):
        return orc.forward(hh, WW, y)["loss"]

    fd_h = np.zeros_like(h)
    for i in range(L):
        for k in range(H):
            hp = h.copy(); hp[i, k] += eps
            hm = h.copy(); hm[i, k] -= eps
            fd_h[i, k] = (loss_at(hp, W) - loss_at(hm, W)) / (2 * eps)
    fd_W = np.zeros_like(W)
    for v in range(V):
        for k in range(H):
            Wp = W.copy(); Wp[v, k] += eps
            Wm = W.copy(); Wm[v, k] -= eps
            fd_W[v, k] = (loss_at(h, Wp) - loss_at(h, Wm)) / (2 * eps)
    rel = lambda a, b: np.linalg.norm(a - b) / max(1e-300, np.linalg.norm(b))
    assert rel(out["dh"], fd_h) <= 1e-6, f"dh vs finite differences {rel(out['dh'], fd_h)}"
    assert rel(out["dW"], fd_W) <= 1e-6, f"dW vs finite differences {rel(out['dW'], fd_W)}"
    assert np.all(out["dh"][3] == 0.0)


# --------------------------------------------------------------------- P5
def pin_chunk_independence(orc):
    """Row blocks of any size give the unchunked result (the chunked method)."""
    L, H, V = 40, 16, 97
    h, W, y = _case(L, H, V, seed=8, ignore=(2, 39))
    ref = orc.fwd_bwd(h, W, y, block_rows=L)
    for b in (1, 3, 7, 256):
        out = orc.fwd_bwd(h, W, y, block_rows=b)
        assert abs(out["loss"] - ref["loss"]) <= 1e-12
        assert np.max(np.abs(out["lse"] - ref["lse"])) <= 1e-12
        assert np.max(np.abs(out["dh"] - ref["dh"])) <= 1e-12
        assert np.max(np.abs(out["dW"] - ref["dW"])) <= 1e-12


# --------------------------------------------------------------------- P6
def pin_ignored_rows(orc):
    """Ignored rows add nothing: deleting them leaves loss and dW; their dh
    rows are exactly 0; changing their h moves only their own lse."""
    L, H, V = 30, 12, 40
    ign = (0, 4, 5, 29)
    h, W, y = _case(L, H, V, seed=9, ignore=ign)
    out = orc.fwd_bwd(h, W, y)
    keep = np.array([i not in ign for i in range(L)])
    out2 = orc.fwd_bwd(h[keep], W, y[keep])
    assert out["n_valid"] == L - len(ign)
    assert abs(out["loss"] - out2["loss"]) <= 1e-12
    assert np.max(np.abs(out["dW"] - out2["dW"])) <= 1e-12
    assert np.max(np.abs(out["dh"][keep] - out2["dh"])) <= 1e-12
    for i in ign:
        assert np.all(out["dh"][i] == 0.0)
        assert out["nll"][i] == 0.0
    h3 = h.copy()
    h3[4] = -h3[4] * 2.0
    out3 = orc.fwd_bwd(h3, W, y)
    assert out3["loss"] == out["loss"]
    assert np.all(out3["dW"] == out["dW"])
    changed = np.flatnonzero(out3["lse"] != out["lse"])
    assert list(changed) == [4]
    # no valid row: NaN loss and zero gradients
    y0 = np.full(L, IGN, np.int64)
    out0 = orc.fwd_bwd(h, W, y0)
    assert math.isnan(out0["loss"]) and out0["n_valid"] == 0
    assert np.all(out0["dh"] == 0) and np.all(out0["dW"] == 0)
    assert np.all(np.isfinite(out0["lse"]))


# --------------------------------------------------------------------- P7
def pin_invariants(orc):
    """sum_v dW[v] = 0; W_v -> W_v + c: loss unchanged, lse_i -> lse_i + h_i.c;
    row and vocabulary permutations permute the outputs."""
    L, H, V = 48, 20, 130
    h, W, y = _case(L, H, V, seed=10, ignore=(3, 17))
    out = orc.fwd_bwd(h, W, y)
    colsum = out["dW"].sum(0)
    assert np.linalg.norm(colsum) <= 1e-10 * np.linalg.norm(out["dW"]), "sum_v dW != 0"
    c = np.random.default_rng(11).standard_normal(H).astype(np.float64) * 0.5
    out_s = orc.fwd_bwd(h.astype(np.float64), W.astype(np.float64) + c[None, :], y)
    assert abs(out_s["loss"] - out["loss"]) <= 1e-10 * abs(out["loss"])
    assert np.max(np.abs(out_s["lse"] - (out["lse"] + h.astype(np.float64) @ c))) <= 1e-10
    pr = np.random.default_rng(12).permutation(L)
    out_r = orc.fwd_bwd(h[pr], W, y[pr])
    assert abs(out_r["loss"] - out["loss"]) <= 1e-12 * abs(out["loss"])
    assert np.max(np.abs(out_r["lse"] - out["lse"][pr])) <= 1e-12
    assert np.max(np.abs(out_r["dh"] - out["dh"][pr])) <= 1e-12
    assert np.max(np.abs(out_r["dW"] - out["dW"])) <= 1e-12
    pv = np.random.default_rng(13).permutation(V)
    inv = np.argsort(pv)
    y_v = np.where(y == IGN, IGN, inv[np.where(y == IGN, 0, y)])
    out_v = orc.fwd_bwd(h, W[pv], y_v)
    assert abs(out_v["loss"] - out["loss"]) <= 1e-12 * abs(out["loss"])
    assert np.max(np.abs(out_v["lse"] - out["lse"])) <= 1e-12
    assert np.max(np.abs(out_v["dh"] - out["dh"])) <= 1e-12
    assert np.max(np.abs(out_v["dW"] - out["dW"][pv])) <= 1e-12


# --------------------------------------------------------------------- P8
def pin_statistics(orc):
    """Random W ~ N(0, s^2): z_i. ~ N(0, s^2 |h_i|^2) across the vocabulary, so
    lse_i ~ ln V + s^2 |h_i|^2 / 2 and, labels being independent of z, the mean
    loss is close to the mean lse.  Sanity level only."""
    L, H, V = 64, 256, 8192
    rng = np.random.default_rng(14)
    h = torch.from_numpy(rng.standard_normal((L, H)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    W = torch.from_numpy((rng.standard_normal((V, H)) * 0.02).astype(np.float32)).to(torch.bfloat16).float().numpy()
    y = rng.integers(0, V, size=L)
    out = orc.forward(h, W, y)
    pred = math.log(V) + 0.02 ** 2 * (h.astype(np.float64) ** 2).sum(1) / 2
    assert np.max(np.abs(out["lse"] - pred)) <= 0.02, np.max(np.abs(out["lse"] - pred))
    assert abs(out["loss"] - out["lse"].mean()) <= 0.1


# --------------------------------------------------------------------- S5
def pin_label_range(orc):
    """A label that is not ignore_index must lie in [0, V): -1, any other
    negative value and V itself are errors in every entry point (they would
    otherwise index the logits of another class, e.g. column V - 1 for -1);
    ignore_index itself, 0 and V - 1 are accepted."""
    L, H, V = 6, 4, 9
    h, W, y = _case(L, H, V, seed=16, ignore=(2,))
    for bad in (-1, -7, V, V + 3):
        yb = y.copy()
        yb[4] = bad
        for call in (lambda: orc.forward(h, W, yb), lambda: orc.backward(h, W, yb),
                     lambda: orc.fwd_bwd(h, W, yb), lambda: orc.rows_forward(h, W, yb),
                     lambda: orc.rows_dh(h, W, yb, 5),
                     lambda: orc.cols_dW(h, W[:2], yb, [0, 1], np.zeros(L), V)):
            try:
                call()
            except ValueError:
                continue
            raise AssertionError(f"label {bad} outside [0, {V}) was accepted")
    # the edges of the range and a custom ignore_index are fine
    ye = y.copy()
    ye[0], ye[1] = 0, V - 1
    out = orc.fwd_bwd(h, W, ye)
    assert out["n_valid"] == L - 1
    yc = np.where(ye == IGN, -1, ye)
    out_c = orc.fwd_bwd(h, W, yc, ignore_index=-1)
    assert out_c["n_valid"] == L - 1 and abs(out_c["loss"] - out["loss"]) <= 1e-12


# --------------------------------------------------------------------- subset helpers
def pin_row_helpers(orc):
    """rows_forward / rows_dh agree with the full-array functions row by row."""
    L, H, V = 25, 10, 60
    h, W, y = _case(L, H, V, seed=15, ignore=(1, 2))
    out = orc.fwd_bwd(h, W, y, grad=0.5)
    rows = np.array([0, 1, 7, 24])
    lse, nll = orc.rows_forward(h[rows], W, y[rows])
    assert np.max(np.abs(lse - out["lse"][rows])) <= 1e-12
    assert np.max(np.abs(nll - out["nll"][rows])) <= 1e-12
    dh = orc.rows_dh(h[rows], W, y[rows], out["n_valid"], grad=0.5)
    assert np.max(np.abs(dh - out["dh"][rows])) <= 1e-12


def pin_col_helper(orc):
    """cols_dW agrees with the full dW entry by entry: vocabulary entries that
    are the label of one or several rows, of an ignored row only, and of none,
    including the first and the last; blocks of rows that split the rows
    unevenly do not change it."""
    L, H, V = 37, 12, 50
    h, W, y = _case(L, H, V, seed=17, ignore=(3, 4, 30))
    y[[5, 6, 7]] = 11  # a label shared by three rows
    y[8] = V - 1
    y[9] = 0
    y[3] = -100
    out = orc.fwd_bwd(h, W, y, grad=0.75)
    never = [v for v in range(V) if v not in set(y.tolist())]
    cols = np.array([0, 11, V - 1, int(y[10]), never[0]])
    for block in (5, 8192):
        dW = orc.cols_dW(h, W[cols], y, cols, out["lse"], V, grad=0.75, block_rows=block)
        ref = out["dW"][cols]
        assert np.max(np.abs(dW - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    # no labelled row: zero
    yi = np.full(L, -100)
    assert not orc.cols_dW(h, W[cols], yi, cols, out["lse"], V).any()


ALL_PINS = [
    pin_zero_weights,
    pin_bruteforce_decimal,
    pin_torch_cross_entropy,
    pin_finite_differences,
    pin_chunk_independence,
    pin_ignored_rows,
    pin_invariants,
    pin_statistics,
    pin_label_range,
    pin_row_helpers,
    pin_col_helper,
]
