"""GPU parity at the full Qwen3 head workloads (4B 160k, 8B 1M-shard, 32B).

Each workload's seed-0 inputs are drawn on the CPU (their sha256 digests
must match those the golden files record) and copied bit for bit to the
device.  Both pairs of entry points (lmce_fwd + lmce_bwd, and the training
pair lmce_fwd_train + lmce_bwd_train that bench.py times) are then checked,
at full size, against values that only the fp64 CPU oracle computed:
  * the mean loss against the full-length oracle loss (relative <= 1e-3);
  * the lse of EVERY row against the full-length oracle lse (abs <= 2e-3);
  both stored in tests/golden/full_<workload>.{json,npy} by
  tests/golden/make_full_golden.py, which calls only the oracle;
  * dh on 512 sampled rows (row 0, the last row, ignored rows, random rows)
    against the oracle's rows_dh, computed here (relative Frobenius <= 1e-2;
    ignored rows exactly 0);
  * 24 sampled rows of dW (vocabulary entries 0, 1, 2 and V - 1, the labels
    of a few rows, random entries) against the oracle's cols_dW over all L
    rows, fed the oracle's full-length lse from the golden file (relative
    Frobenius <= 1e-2);
  * sum over the vocabulary of dW is ~0 (softmax minus one-hot sums to 0);
and a reduced instance (the first 1024 rows at full H and V) is compared with
the full oracle on every output, dW included.
"""

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import lm_head_chunked_amd as lm
from lm_head_chunked_amd import _lib, synth
from tests.golden.make_full_golden import LONG, digest, golden_paths
from tests.pairs import run_pair

pytestmark = pytest.mark.gpu

LOSS_REL = 1e-3
LSE_ABS = 2e-3
GRAD_REL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def np32(t):
    return t.detach().float().cpu().numpy()


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


_cache = {}


def cpu_inputs(name):
    """The workload's seed-0 CPU draw, checked against the golden digests (one workload kept at a time)."""
    if name not in _cache:
        _cache.clear()
        jp, npp = golden_paths(name)
        rec = json.load(open(jp))
        h, W, y = synth.make(synth.WORKLOADS[name])
        got = (digest(h), digest(W), digest(y))
        assert got == (rec["h_sha256"], rec["W_sha256"], rec["labels_sha256"]), \
            f"{name}: the CPU draw differs from the one the golden values were computed on"
        _cache[name] = (h, W, y, rec, np.load(npp))
    return _cache[name]


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
@pytest.mark.parametrize("name", LONG)
def test_full_size_against_full_oracle(name, train):
    wl = synth.WORKLOADS[name]
    say(f"[case] {name} full size L={wl.L} H={wl.H} V={wl.V} train={train}")
    h_c, W_c, y_c, rec, lse_ref = cpu_inputs(name)
    assert lse_ref.shape == (wl.L,) and rec["L"] == wl.L
    dev = torch.device("cuda:0")
    h, W, y = h_c.to(dev), W_c.to(dev), y_c.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(wl.L, wl.H, wl.V, 256), dtype=torch.uint8, device=dev)
    loss, lse, dh, dW = run_pair(train, h, W, y, -100, 256, ws)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    torch.cuda.synchronize()
    del ws
    say(f"[{name}] gpu done, loss {float(loss):.6f}")

    e_loss = abs(float(loss) - rec["loss"]) / abs(rec["loss"])
    lse_gpu = lse.cpu().numpy().astype(np.float64)
    e_lse = float(np.max(np.abs(lse_gpu - lse_ref)))
    say(f"[{name}] loss {float(loss):.7f} vs oracle {rec['loss']:.7f}: rel {e_loss:.2e}; "
        f"lse max abs err over all {wl.L} rows {e_lse:.2e}")
    assert e_loss <= LOSS_REL
    assert e_lse <= LSE_ABS

    g = torch.Generator().manual_seed(123)
    ign = torch.nonzero(y_c == -100).flatten()[:8]
    rnd = torch.randperm(wl.L, generator=g)[:512]
    rows = torch.unique(torch.cat([torch.tensor([0, wl.L - 1]), ign, rnd]))[:512]
    W_np = np32(W_c)
    n_valid = int((y_c != -100).sum())
    assert n_valid == rec["n_valid"]
    dh_ref = oracle.rows_dh(np32(h_c[rows]), W_np, y_c[rows].numpy(), n_valid)
    dh_gpu = dh[rows.to(dev)].cpu().numpy()
    e_dh = rel_fro(dh_gpu, dh_ref)
    say(f"[{name}] dh rel err on {len(rows)} sampled rows {e_dh:.2e}")
    assert e_dh <= GRAD_REL
    ignored = (y_c[rows] == -100).numpy()
    assert np.all(dh_gpu[ignored] == 0.0)

    gv = torch.Generator().manual_seed(321)
    cols = torch.cat([torch.tensor([0, 1, 2, wl.V - 1]), y_c[y_c != -100][:4],
                      torch.randperm(wl.V, generator=gv)[:24]])
    cols = torch.unique(cols)[:24]
    dW_ref = oracle.cols_dW(np32(h_c), np32(W_c[cols]), y_c.numpy(), cols.numpy(), lse_ref, wl.V)
    dW_gpu = dW[cols.to(dev)].cpu().numpy()
    e_dW = rel_fro(dW_gpu, dW_ref)
    say(f"[{name}] dW rel err on {len(cols)} sampled vocabulary rows over all {wl.L} rows {e_dW:.2e}")
    assert e_dW <= GRAD_REL

    colsum = dW.double().sum(0)
    ratio = float(colsum.norm() / dW.double().norm())
    say(f"[{name}] |sum_v dW| / |dW| = {ratio:.2e}")
    assert ratio <= 1e-2
    assert bool(torch.isfinite(dW).all()) and bool(torch.isfinite(dh).all())
    del dh, dW


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
@pytest.mark.parametrize("name", LONG)
def test_reduced_rows_full_parity(name, train):
    wl = synth.WORKLOADS[name]
    Lr = 1024
    say(f"[case] {name} first {Lr} rows at H={wl.H} V={wl.V} train={train} (oracle ~5-20 s)")
    dev = torch.device("cuda:0")
    h, W, y = synth.make(wl, device=dev)
    h = h[:Lr].contiguous()
    y = y[:Lr].contiguous()
    ws = torch.empty(lm.lmce_workspace_size(Lr, wl.H, wl.V, 256), dtype=torch.uint8, device=dev)
    loss, lse, dh, dW = run_pair(train, h, W, y, -100, 256, ws)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    torch.cuda.synchronize()
    ref = oracle.fwd_bwd(np32(h), np32(W), y.cpu().numpy())
    e = (abs(float(loss) - ref["loss"]) / abs(ref["loss"]), float(np.max(np.abs(lse.cpu().numpy() - ref["lse"]))),
         rel_fro(dh.cpu().numpy(), ref["dh"]), rel_fro(dW.cpu().numpy(), ref["dW"]))
    say(f"[{name} L={Lr}] loss rel {e[0]:.2e} lse abs {e[1]:.2e} dh rel {e[2]:.2e} dW rel {e[3]:.2e}")
    assert e[0] <= LOSS_REL and e[1] <= LSE_ABS and e[2] <= GRAD_REL and e[3] <= GRAD_REL
