"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (bf16 inputs, fp32 accumulation): mean loss relative error
<= 1e-3, per-row lse absolute error <= 2e-3 on every row, dh and dW relative
Frobenius error <= 1e-2.  Inputs are drawn once and copied bit-exactly to
both sides.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import lm_head_chunked_amd as lm
from lm_head_chunked_amd import _lib, synth
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
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def run_gpu(h, W, y, chunk_rows=256, grad=1.0, ignore_index=-100, train=False):
    """lmce_fwd + lmce_bwd, or (train=True) the training pair lmce_fwd_train + lmce_bwd_train."""
    dev = torch.device("cuda:0")
    h_d, W_d, y_d = h.to(dev), W.to(dev), y.to(dev)
    L, H = h.shape
    V = W.shape[0]
    ws = torch.empty(lm.lmce_workspace_size(L, H, V, chunk_rows), dtype=torch.uint8, device=dev)
    g = torch.tensor(grad, dtype=torch.float32, device=dev)
    loss, lse, dh, dW = run_pair(train, h_d, W_d, y_d, ignore_index, chunk_rows, ws, g)
    status = lm.lmce_read_status(ws)
    torch.cuda.synchronize()
    return {"loss": float(loss), "lse": lse.cpu().numpy(), "dh": dh.cpu().numpy(), "dW": dW.cpu().numpy(),
            "status": status}


def assert_parity(gpu, ref, what=""):
    loss_err = abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"])
    lse_err = float(np.max(np.abs(gpu["lse"] - ref["lse"])))
    dh_err = rel_fro(gpu["dh"], ref["dh"])
    dW_err = rel_fro(gpu["dW"], ref["dW"])
    say(f"[parity {what}] loss rel {loss_err:.2e} lse abs {lse_err:.2e} dh rel {dh_err:.2e} dW rel {dW_err:.2e}")
    assert gpu["status"] == _lib.LMCE_OK
    assert loss_err <= LOSS_REL, f"loss {gpu['loss']} vs {ref['loss']}"
    assert lse_err <= LSE_ABS
    assert dh_err <= GRAD_REL
    assert dW_err <= GRAD_REL
    return loss_err, lse_err, dh_err, dW_err


def test_tiny_workload_parity():
    say("[case] tiny workload L=512 H=256 V=4096")
    h, W, y = synth.make("tiny")
    gpu = run_gpu(h, W, y, chunk_rows=256)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    assert_parity(gpu, ref, "tiny")
    # ignored rows: exactly zero dh rows
    ign = (y == -100).numpy()
    assert np.all(gpu["dh"][ign] == 0.0)


RAGGED = [
    (300, 128, 700, 0.2),
    (129, 256, 257, 0.0),
    (1, 128, 1, 0.0),
    (77, 128, 4097, 0.5),
    (256, 384, 1000, 0.1),
    (1000, 512, 130, 0.05),
    (513, 640, 2000, 0.3),
]


@pytest.mark.parametrize("L,H,V,ign", RAGGED)
def test_ragged_shapes(L, H, V, ign):
    say(f"[case] ragged L={L} H={H} V={V} ignore={ign}")
    h, W, y = synth.random_case(L, H, V, seed=L + V, w_std=0.05, ignore_frac=ign)
    gpu = run_gpu(h, W, y, chunk_rows=96)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    if ref["n_valid"] == 0 or abs(ref["loss"]) < 1e-6:
        assert np.max(np.abs(gpu["lse"] - ref["lse"])) <= LSE_ABS
        return
    assert_parity(gpu, ref, f"L={L} H={H} V={V}")


# Wide hidden sizes (H % 256 == 0, H >= 1024) give each backward workgroup a
# 256-wide slice whose accumulator is parked between rounds, when the pass has
# at least one row block (dh) or vocabulary block (dW) per group: many rows
# exercise the dh pass that way, a large vocabulary the dW pass.
WIDE = [
    (5500, 3072, 2500, 0.1),
    (600, 3072, 5500, 0.1),
    (7000, 1024, 3000, 0.2),
    (900, 2560, 9000, 0.1),
]


@pytest.mark.parametrize("L,H,V,ign", WIDE)
def test_wide_slices(L, H, V, ign):
    say(f"[case] wide slices L={L} H={H} V={V} ignore={ign}")
    h, W, y = synth.random_case(L, H, V, seed=L + 7, w_std=0.02, ignore_frac=ign)
    gpu = run_gpu(h, W, y, chunk_rows=256)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    assert_parity(gpu, ref, f"L={L} H={H} V={V}")
    ign_rows = (y == -100).numpy()
    assert np.all(gpu["dh"][ign_rows] == 0.0)


# The training pair: one vocabulary sweep gives lse and O = sum_v softmax W_v;
# dh = g/N (O - W_y).  Same bar against the oracle, over the same edge cases.
TRAIN = [
    (512, 256, 4096, 0.1),
    (300, 128, 700, 0.2),
    (1, 128, 1, 0.0),
    (77, 128, 4097, 0.5),
    (513, 640, 2000, 0.3),
    (1000, 512, 130, 0.05),
    (5500, 3072, 2500, 0.1),
    (600, 3072, 5500, 0.1),
]


@pytest.mark.parametrize("L,H,V,ign", TRAIN)
def test_train_pair_parity(L, H, V, ign):
    say(f"[case] train pair L={L} H={H} V={V} ignore={ign}")
    h, W, y = synth.random_case(L, H, V, seed=L + V + 1, w_std=0.05, ignore_frac=ign)
    gpu = run_gpu(h, W, y, chunk_rows=256, grad=1.5, train=True)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=1.5)
    if ref["n_valid"] == 0 or abs(ref["loss"]) < 1e-6:
        assert np.max(np.abs(gpu["lse"] - ref["lse"])) <= LSE_ABS
        return
    assert_parity(gpu, ref, f"train L={L} H={H} V={V}")
    ign_rows = (y == -100).numpy()
    assert np.all(gpu["dh"][ign_rows] == 0.0)


def _max_jumps(z, tiles, jump=16.0):
    """(jumps, flat) counts of vocabulary rounds after the first in which some
    row's running maximum rises by more than `jump` (or by no more), on fp64
    logits z [L, V], with rows in 256-row blocks and rounds of `tiles`
    256-column tiles as in the fused training forward."""
    L, V = z.shape
    jumps = flat = 0
    for r0 in range(0, L, 256):
        zb = z[r0:r0 + 256]
        run = zb[:, :256 * tiles].max(axis=1)
        for v0 in range(256 * tiles, V, 256 * tiles):
            m = np.maximum(run, zb[:, v0:v0 + 256 * tiles].max(axis=1))
            if (m > run + jump).any():
                jumps += 1
            else:
                flat += 1
            run = m
    return jumps, flat


# (L, H, V): 128-wide slices (3 members, one tile each per round) and
# 256-wide slices (12 members, two tiles each per round)
JUMPS = [(600, 384, 6000), (300, 3072, 30000)]


@pytest.mark.parametrize("L,H,V", JUMPS)
def test_train_pair_parity_when_the_maximum_jumps(L, H, V):
    """Logits that grow along the vocabulary, so that in later rounds of the
    fused forward some rows' running maximum rises by more than 16 (O, the
    row sums and, with two tiles per round, the tile already in the exchange
    are then rescaled by less than exp(-16)), while in others it barely
    moves."""
    say(f"[case] train pair, growing logits L={L} H={H} V={V}")
    h, W, y = synth.random_case(L, H, V, seed=23, w_std=0.05, ignore_frac=0.1)
    scale = torch.ones(V)
    scale[V // 2:(3 * V) // 4] = 8.0
    scale[(3 * V) // 4:] = 20.0
    W = (W.float() * scale[:, None]).to(torch.bfloat16)
    z = np32(h).astype(np.float64) @ np32(W).astype(np.float64).T
    wide = H % 256 == 0 and H >= 1024
    tiles = (H // 256) * 2 if wide else H // 128
    jumps, flat = _max_jumps(z, tiles)
    assert jumps > 0 and flat > 0, (jumps, flat)
    a = run_gpu(h, W, y, grad=1.5, train=True)
    b = run_gpu(h, W, y, grad=1.5, train=True)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=1.5)
    assert_parity(a, ref, f"train growing logits L={L} H={H} V={V} (jumps {jumps}, flat {flat})")
    for k in ("lse", "dh", "dW"):
        assert np.array_equal(a[k], b[k]), k


def _random_shapes(n, seed=2024):
    """Seeded (L, H, V, ignore fraction, chunk_rows) draws: ragged L and V,
    H a multiple of 128 up to 4096 (so the 256-wide slices appear too), and
    every allowed kind of chunk_rows; sized for an fp64 oracle in seconds."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        H = int(rng.choice([128, 256, 384, 640, 1024, 1536, 3072, 4096]))
        L = int(rng.integers(1, 3000))
        V = int(rng.integers(1, 9000))
        if L * V * H > 2.5e10:
            continue
        out.append((L, H, V, float(rng.choice([0.0, 0.05, 0.3, 0.9])), int(rng.integers(1, 33)) * 32))
    return out


@pytest.mark.parametrize("L,H,V,ign,chunk", _random_shapes(10))
def test_random_shapes_both_pairs(L, H, V, ign, chunk):
    say(f"[case] random shape L={L} H={H} V={V} ignore={ign} chunk_rows={chunk}")
    h, W, y = synth.random_case(L, H, V, seed=L * 7 + V, w_std=0.05, ignore_frac=ign)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=0.75)
    for train in (False, True):
        gpu = run_gpu(h, W, y, chunk_rows=chunk, grad=0.75, train=train)
        if ref["n_valid"] == 0:
            assert math.isnan(gpu["loss"])
            assert np.max(np.abs(gpu["lse"] - ref["lse"])) <= LSE_ABS
            assert not gpu["dh"].any() and not gpu["dW"].any()
            continue
        assert_parity(gpu, ref, f"random L={L} H={H} V={V} train={train}")
        assert np.all(gpu["dh"][(y == -100).numpy()] == 0.0)


def test_train_pair_matches_plain_pair_and_is_deterministic():
    say("[case] train pair vs plain pair, qwen3_0.6b head")
    h, W, y = synth.make("qwen3_0.6b")
    a = run_gpu(h, W, y, train=True)
    b = run_gpu(h, W, y, train=True)
    c = run_gpu(h, W, y, train=False)
    for k in ("lse", "dh", "dW"):
        assert np.array_equal(a[k], b[k]), k
    assert a["loss"] == b["loss"]
    assert abs(a["loss"] - c["loss"]) <= 1e-5 * abs(c["loss"])
    assert np.max(np.abs(a["lse"] - c["lse"])) <= 1e-4
    assert rel_fro(a["dh"], c["dh"]) <= 5e-3
    # the same dW pass, fed the fused forward's lse (equal up to rounding)
    assert rel_fro(a["dW"], c["dW"]) <= 1e-3


# Repeated calls on the same inputs must agree bit for bit wherever the
# passes take 256-wide slices (the exchange, parking and statistics paths
# that only these shapes use): a run-to-run difference well inside the
# parity tolerance (0.3 % in dh) is still a bug.  One round per row block
# (V = 2500), many rounds (V = 40000), and H = 5120 (20 members per group).
REPEAT = [
    (5500, 3072, 2500),
    (2048, 4096, 40000),
    (1500, 5120, 9000),
]


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
@pytest.mark.parametrize("L,H,V", REPEAT)
def test_wide_slices_are_repeatable(L, H, V, train):
    say(f"[case] repeatability L={L} H={H} V={V} train={train}")
    h, W, y = synth.random_case(L, H, V, seed=3 * L + H, w_std=0.03, ignore_frac=0.1)
    runs = [run_gpu(h, W, y, train=train) for _ in range(3)]
    for r in runs[1:]:
        assert r["loss"] == runs[0]["loss"]
        for k in ("lse", "dh", "dW"):
            assert np.array_equal(r[k], runs[0][k]), k


def test_train_backward_without_train_forward_is_reported():
    say("[case] lmce_bwd_train after a plain lmce_fwd")
    h, W, y = synth.random_case(256, 128, 600, seed=11)
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(256, 128, 600), dtype=torch.uint8, device=dev)
    loss, lse = lm.lmce_fwd(hd, Wd, yd, workspace=ws)
    dh, dW = lm.lmce_bwd_train(hd, Wd, yd, lse, workspace=ws, dh_out=torch.empty(256, 128, device=dev))
    assert lm.lmce_read_status(ws) == _lib.LMCE_ERR_STATE
    assert torch.isnan(dh).all()
    # a training forward on the same workspace makes the pair valid again
    loss, lse, dh = lm.lmce_fwd_train(hd, Wd, yd, workspace=ws)
    dh, dW = lm.lmce_bwd_train(hd, Wd, yd, lse, workspace=ws, dh_out=dh)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    assert torch.isfinite(dh).all()
    # ... but only in the buffer the forward wrote O into
    loss, lse, dh = lm.lmce_fwd_train(hd, Wd, yd, workspace=ws)
    other = torch.zeros_like(dh)
    lm.lmce_bwd_train(hd, Wd, yd, lse, workspace=ws, dh_out=other)
    assert lm.lmce_read_status(ws) == _lib.LMCE_ERR_STATE
    assert torch.isnan(other).all()


def test_results_do_not_depend_on_chunk_rows():
    say("[case] chunk_rows independence L=700 H=256 V=3000")
    h, W, y = synth.random_case(700, 256, 3000, seed=5, ignore_frac=0.1)
    base = run_gpu(h, W, y, chunk_rows=256)
    for c in (32, 96, 128, 512, 1024):
        o = run_gpu(h, W, y, chunk_rows=c)
        assert o["loss"] == base["loss"], c
        assert np.array_equal(o["lse"], base["lse"]), c
        assert np.array_equal(o["dh"], base["dh"]), c
        assert np.array_equal(o["dW"], base["dW"]), c


def test_train_pair_does_not_depend_on_chunk_rows():
    say("[case] chunk_rows independence, training pair, L=700 H=3072 V=3000")
    h, W, y = synth.random_case(700, 3072, 3000, seed=6, ignore_frac=0.1)
    base = run_gpu(h, W, y, chunk_rows=256, train=True)
    for c in (32, 128, 1024):
        o = run_gpu(h, W, y, chunk_rows=c, train=True)
        assert o["loss"] == base["loss"], c
        for k in ("lse", "dh", "dW"):
            assert np.array_equal(o[k], base[k]), (c, k)


# Whatever the workspace holds before a call must not reach the results:
# every call writes all the workspace it reads (a row of h^T past L left
# unwritten once turned into NaN in dW, 0 * NaN, with a NaN-filled
# workspace).  Shapes with L % 128 in (0, 64], ignored rows (compaction on
# and off), 128- and 256-wide slices.
FILLED = [
    (2741, 256, 3237, 0.05),
    (700, 3072, 3000, 0.3),
    (321, 128, 5000, 0.5),
    (1000, 512, 900, 0.0),
]


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
@pytest.mark.parametrize("L,H,V,ign", FILLED)
def test_workspace_contents_do_not_matter(L, H, V, ign, train):
    say(f"[case] NaN-filled workspace L={L} H={H} V={V} ignore={ign} train={train}")
    h, W, y = synth.random_case(L, H, V, seed=L + 2 * V, w_std=0.05, ignore_frac=ign)
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((lm.lmce_workspace_size(L, H, V, 256),), fill, dtype=torch.uint8, device=dev)
        loss, lse, dh, dW = run_pair(train, hd, Wd, yd, -100, 256, ws)
        assert lm.lmce_read_status(ws) == _lib.LMCE_OK
        outs.append((float(loss), lse.cpu().numpy(), dh.cpu().numpy(), dW.cpu().numpy()))
    assert np.isfinite(outs[1][0]) and all(np.isfinite(x).all() for x in outs[1][1:])
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1:], outs[1][1:]):
        assert np.array_equal(a, b)


def test_plain_backward_between_train_calls_leaves_the_saved_forward():
    """A plain backward with other labels between lmce_fwd_train and
    lmce_bwd_train on one workspace: the plain dh pass keeps its own row order
    and flags, so the training backward still finds the forward's state.  Both
    label sets drop enough rows that each order is in use."""
    L, H, V = 1500, 512, 3000
    say(f"[case] plain backward between the training calls L={L} H={H} V={V}")
    h, W, y = synth.random_case(L, H, V, seed=91, w_std=0.05, ignore_frac=0.4)
    _, _, y2 = synth.random_case(L, H, V, seed=92, w_std=0.05, ignore_frac=0.6)
    dev = torch.device("cuda:0")
    hd, Wd, yd, y2d = h.to(dev), W.to(dev), y.to(dev), y2.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(L, H, V, 256), dtype=torch.uint8, device=dev)
    loss, lse, dh0 = lm.lmce_fwd_train(hd, Wd, yd, -100, 256, ws)
    dh_ref, dW_ref = lm.lmce_bwd_train(hd, Wd, yd, lse, None, -100, 256, ws, dh0)
    ref = (dh_ref.cpu().numpy(), dW_ref.cpu().numpy())
    loss, lse, dh1 = lm.lmce_fwd_train(hd, Wd, yd, -100, 256, ws)
    _, lse2 = lm.lmce_fwd(hd, Wd, y2d, -100, 256, torch.empty_like(ws))
    dh2, dW2 = lm.lmce_bwd(hd, Wd, y2d, lse2, None, -100, 256, ws)
    dh, dW = lm.lmce_bwd_train(hd, Wd, yd, lse, None, -100, 256, ws, dh1)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    assert np.array_equal(dh.cpu().numpy(), ref[0]) and np.array_equal(dW.cpu().numpy(), ref[1])
    # and the plain backward itself, on the other labels
    r2 = oracle.fwd_bwd(h.float().numpy(), W.float().numpy(), y2.numpy())
    assert rel_fro(dh2.cpu().numpy(), r2["dh"]) <= 1e-2 and rel_fro(dW2.cpu().numpy(), r2["dW"]) <= 1e-2
    assert np.all(dh2.cpu().numpy()[(y2 == -100).numpy()] == 0.0)


@pytest.mark.parametrize("L,H,V,ign", [(1300, 384, 2100, 0.45), (600, 3072, 1500, 0.6)])
def test_backward_halves_match_the_whole(L, H, V, ign):
    """lmce_bwd_dh and lmce_bwd_dW give bitwise the dh and dW of lmce_bwd, with
    enough ignored rows that the dh pass runs on its labelled-first order."""
    say(f"[case] backward halves L={L} H={H} V={V} ignore={ign}")
    h, W, y = synth.random_case(L, H, V, seed=L + V, w_std=0.05, ignore_frac=ign)
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(L, H, V, 256), dtype=torch.uint8, device=dev)
    _, lse = lm.lmce_fwd(hd, Wd, yd, -100, 256, ws)
    dh, dW = lm.lmce_bwd(hd, Wd, yd, lse, None, -100, 256, ws)
    dh1 = lm.lmce_bwd_dh(hd, Wd, yd, lse, None, -100, 256, ws)
    dW1 = lm.lmce_bwd_dW(hd, Wd, yd, lse, None, -100, 256, ws)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    assert np.array_equal(dh1.cpu().numpy(), dh.cpu().numpy())
    assert np.array_equal(dW1.cpu().numpy(), dW.cpu().numpy())
    ref = oracle.fwd_bwd(h.float().numpy(), W.float().numpy(), y.numpy())
    assert rel_fro(dh1.cpu().numpy(), ref["dh"]) <= 1e-2 and rel_fro(dW1.cpu().numpy(), ref["dW"]) <= 1e-2
    assert np.all(dh1.cpu().numpy()[(y == -100).numpy()] == 0.0)


def test_deterministic():
    say("[case] determinism tiny")
    h, W, y = synth.make("tiny")
    a = run_gpu(h, W, y)
    b = run_gpu(h, W, y)
    for k in ("lse", "dh", "dW"):
        assert np.array_equal(a[k], b[k])
    assert a["loss"] == b["loss"]


def test_zero_weights_give_ln_V():
    say("[case] W = 0")
    L, H, V = 200, 128, 4096
    h, _, y = synth.random_case(L, H, V, seed=3, ignore_frac=0.1)
    W = torch.zeros(V, H, dtype=torch.bfloat16)
    gpu = run_gpu(h, W, y)
    lnV = math.log(V)
    assert np.max(np.abs(gpu["lse"] - lnV)) <= 1e-5
    assert abs(gpu["loss"] - lnV) <= 1e-5
    assert np.all(gpu["dh"] == 0.0)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    assert rel_fro(gpu["dW"], ref["dW"]) <= GRAD_REL


def test_all_rows_ignored():
    say("[case] N_valid = 0")
    h, W, y = synth.random_case(130, 128, 500, seed=4)
    y[:] = -100
    gpu = run_gpu(h, W, y)
    assert math.isnan(gpu["loss"])
    assert np.all(np.isfinite(gpu["lse"]))
    assert np.all(gpu["dh"] == 0.0) and np.all(gpu["dW"] == 0.0)


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
def test_all_rows_ignored_wide_slices(train):
    """No labelled row at H = 3072: the dW pass (256-wide slices, accumulators
    parked between rounds) has no rows to sweep and must still write dW = 0."""
    say(f"[case] N_valid = 0, H = 3072, train={train}")
    h, W, y = synth.random_case(700, 3072, 3000, seed=9)
    y[:] = -100
    gpu = run_gpu(h, W, y, train=train)
    assert math.isnan(gpu["loss"])
    assert np.all(np.isfinite(gpu["lse"]))
    assert np.all(gpu["dh"] == 0.0) and np.all(gpu["dW"] == 0.0)


def test_out_of_range_label_is_reported():
    say("[case] bad label")
    h, W, y = synth.random_case(64, 128, 100, seed=6, ignore_frac=0.0)
    y[10] = 100
    gpu = run_gpu(h, W, y)
    assert gpu["status"] == _lib.LMCE_ERR_LABEL
    assert math.isnan(gpu["loss"])
    assert np.all(np.isfinite(gpu["dh"])) and np.all(np.isfinite(gpu["dW"]))


def test_custom_ignore_index_and_grad_scale():
    say("[case] ignore_index=7, grad=2.5")
    h, W, y = synth.random_case(256, 128, 600, seed=8, ignore_frac=0.0)
    y[::5] = 7  # label 7 is the ignore index here
    gpu = run_gpu(h, W, y, grad=2.5, ignore_index=7)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), ignore_index=7, grad=2.5)
    assert_parity(gpu, ref, "ignore_index=7 grad=2.5")


def test_autograd_binding():
    say("[case] autograd chunked_nll")
    h, W, y = synth.random_case(384, 256, 2048, seed=9)
    dev = torch.device("cuda:0")
    hd = h.to(dev).requires_grad_(True)
    Wd = W.to(dev).requires_grad_(True)
    loss = lm.chunked_nll(hd, Wd, y.to(dev))
    (loss * 0.5).backward()
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=0.5)
    assert abs(float(loss.detach()) - ref["loss"]) <= LOSS_REL * abs(ref["loss"])
    assert rel_fro(np32(hd.grad), ref["dh"]) <= GRAD_REL
    assert rel_fro(np32(Wd.grad), ref["dW"]) <= GRAD_REL


def test_qwen3_06b_head_full_parity():
    """Both pairs against the full oracle at the Qwen3-0.6B head: every output."""
    say("[case] qwen3_0.6b full L=8192 H=1024 V=151936, both pairs (oracle ~30 s)")
    h, W, y = synth.make("qwen3_0.6b")
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=1.25)
    for train in (False, True):
        gpu = run_gpu(h, W, y, grad=1.25, train=train)
        assert_parity(gpu, ref, f"qwen3_0.6b train={train}")
        assert np.all(gpu["dh"][(y == -100).numpy()] == 0.0)


def _with_spin_limit(value, fn):
    """Runs fn with the library's internal group-wait bound set to `value`
    (read by every call from LMCE_SPIN_LIMIT); 0 makes every wait that finds
    its group incomplete give up at once, and every kernel still exits."""
    import os

    old = os.environ.get("LMCE_SPIN_LIMIT")
    os.environ["LMCE_SPIN_LIMIT"] = str(value)
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["LMCE_SPIN_LIMIT"]
        else:
            os.environ["LMCE_SPIN_LIMIT"] = old


def test_failed_group_wait_survives_the_following_backward():
    """A training forward whose group waits give up (forced from the host) is
    reported by lmce_read_status after the following, clean lmce_bwd_train:
    the flags accumulate until read.  That forward's loss is NaN, and the
    backward, finding no complete forward, writes a NaN dh.  After the read
    clears the flags, a clean pair passes parity again."""
    L, H, V = 2048, 1024, 20000  # 8 row blocks, 8 members, 10 rounds of two waits
    say(f"[case] forced group-wait failure L={L} H={H} V={V}")
    h, W, y = synth.random_case(L, H, V, seed=31, w_std=0.05, ignore_frac=0.1)
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(L, H, V), dtype=torch.uint8, device=dev)
    loss, lse, dh = _with_spin_limit(0, lambda: lm.lmce_fwd_train(hd, Wd, yd, workspace=ws))
    torch.cuda.synchronize()
    dh, dW = lm.lmce_bwd_train(hd, Wd, yd, lse, workspace=ws, dh_out=dh)
    assert lm.lmce_read_status(ws) == _lib.LMCE_ERR_HIP
    assert math.isnan(float(loss))
    assert torch.isnan(dh).all()
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK  # the read cleared the flags
    loss, lse, dh = lm.lmce_fwd_train(hd, Wd, yd, workspace=ws)
    dh, dW = lm.lmce_bwd_train(hd, Wd, yd, lse, workspace=ws, dh_out=dh)
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    gpu = {"loss": float(loss), "lse": lse.cpu().numpy(), "dh": dh.cpu().numpy(), "dW": dW.cpu().numpy(),
           "status": _lib.LMCE_OK}
    assert_parity(gpu, ref, "after a forced wait failure")


def test_failed_wait_in_a_backward_pass_is_reported():
    """The plain backward's group waits give up: LMCE_ERR_HIP, then clear."""
    L, H, V = 1024, 512, 9000
    say(f"[case] forced group-wait failure in lmce_bwd L={L} H={H} V={V}")
    h, W, y = synth.random_case(L, H, V, seed=32, w_std=0.05, ignore_frac=0.1)
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(L, H, V), dtype=torch.uint8, device=dev)
    loss, lse = lm.lmce_fwd(hd, Wd, yd, workspace=ws)
    _with_spin_limit(0, lambda: lm.lmce_bwd(hd, Wd, yd, lse, workspace=ws))
    assert lm.lmce_read_status(ws) == _lib.LMCE_ERR_HIP
    assert math.isfinite(float(loss))
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK


def test_label_error_accumulates_until_read():
    """A bad label in one call stays reported after later clean calls on the
    same workspace; the later clean calls' own loss is not NaN."""
    say("[case] label error, then clean calls, then one read")
    h, W, y = synth.random_case(300, 128, 700, seed=33, ignore_frac=0.1)
    ybad = y.clone()
    ybad[17] = -5
    dev = torch.device("cuda:0")
    hd, Wd = h.to(dev), W.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(300, 128, 700), dtype=torch.uint8, device=dev)
    loss_bad, _ = lm.lmce_fwd(hd, Wd, ybad.to(dev), workspace=ws)
    loss, lse, dh = lm.lmce_fwd_train(hd, Wd, y.to(dev), workspace=ws)
    dh, dW = lm.lmce_bwd_train(hd, Wd, y.to(dev), lse, workspace=ws, dh_out=dh)
    assert lm.lmce_read_status(ws) == _lib.LMCE_ERR_LABEL
    assert math.isnan(float(loss_bad)) and math.isfinite(float(loss))
    assert torch.isfinite(dh).all() and torch.isfinite(dW).all()
    assert lm.lmce_read_status(ws) == _lib.LMCE_OK


@pytest.mark.parametrize("train", [False, True], ids=["plain", "train"])
def test_row_shards_compose_to_the_whole(train):
    """How the loss splits over GPUs by rows, on one GPU: each row shard runs
    on its own with the upstream gradient g * N_shard / N (so that its
    g / N_shard is the whole's g / N); the shards' dh rows are the whole's,
    their dW summed is the whole's dW, and the N-weighted mean of their
    losses is the whole's loss.  Checked against the oracle on the whole and,
    tighter, against one GPU call on the whole.  Unequal shards, one with few
    labels, and a 256-wide slice (H = 1024)."""
    L, H, V = 1500, 1024, 3000
    say(f"[case] row shards L={L} H={H} V={V} train={train}")
    h, W, y = synth.random_case(L, H, V, seed=34, w_std=0.05, ignore_frac=0.1)
    y[900:1340] = -100  # the second shard keeps few labels
    bounds = [(0, 700), (700, 1400), (1400, L)]
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    g = 0.75
    n_total = (yd != -100).sum()  # on the device, as a sharded run would all-reduce it
    dh_parts, dW_sum, loss_sum = [], None, torch.zeros((), dtype=torch.float32, device=dev)
    for r0, r1 in bounds:
        n_s = (yd[r0:r1] != -100).sum()
        g_s = (g * n_s.float() / n_total.float()).reshape(())
        ws = torch.empty(lm.lmce_workspace_size(r1 - r0, H, V), dtype=torch.uint8, device=dev)
        loss, _, dh, dW = run_pair(train, hd[r0:r1].contiguous(), Wd, yd[r0:r1].contiguous(), -100, 256, ws, g_s)
        assert lm.lmce_read_status(ws) == _lib.LMCE_OK
        dh_parts.append(dh)
        dW_sum = dW.clone() if dW_sum is None else dW_sum + dW
        loss_sum = loss_sum + loss * n_s.float()
    loss_c = float(loss_sum / n_total.float())
    dh_c = torch.cat(dh_parts).cpu().numpy()
    dW_c = dW_sum.cpu().numpy()
    whole = run_gpu(h, W, y, grad=g, train=train)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=g)
    e_ref = (abs(loss_c - ref["loss"]) / abs(ref["loss"]), rel_fro(dh_c, ref["dh"]), rel_fro(dW_c, ref["dW"]))
    e_gpu = (abs(loss_c - whole["loss"]) / abs(whole["loss"]), rel_fro(dh_c, whole["dh"]), rel_fro(dW_c, whole["dW"]))
    say(f"[shards] vs oracle: loss {e_ref[0]:.2e} dh {e_ref[1]:.2e} dW {e_ref[2]:.2e}; "
        f"vs one call: loss {e_gpu[0]:.2e} dh {e_gpu[1]:.2e} dW {e_gpu[2]:.2e}")
    assert e_ref[0] <= LOSS_REL and e_ref[1] <= GRAD_REL and e_ref[2] <= GRAD_REL
    assert e_gpu[0] <= 1e-5 and e_gpu[1] <= 1e-5 and e_gpu[2] <= 1e-5
    assert np.all(dh_c[(y == -100).numpy()] == 0.0)


def test_binding_rejects_bad_tensors_before_any_launch():
    """The Python binding's checks: host tensors, wrong dtypes, mismatched or
    non-contiguous shapes and a short workspace raise before the library is
    called (the C ABI's own checks are covered on the CPU)."""
    say("[case] binding argument checks")
    dev = torch.device("cuda:0")
    h, W, y = synth.random_case(64, 128, 300, seed=35)
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    bad = [
        ((h, Wd, yd), ValueError),                                 # host tensor
        ((hd.float(), Wd, yd), TypeError),                         # fp32 h
        ((hd, Wd, yd.int()), TypeError),                           # int32 labels
        ((hd, Wd[:, :64].contiguous(), yd), ValueError),           # H mismatch
        ((hd, Wd, yd[:32].contiguous()), ValueError),              # L mismatch
        ((hd.t().contiguous().t(), Wd, yd), ValueError),           # non-contiguous h
        ((hd[None], Wd, yd), ValueError),                          # 3-D h
    ]
    for args, exc in bad:
        with pytest.raises(exc):
            lm.lmce_fwd(*args)
    short = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):
        lm.lmce_fwd(hd, Wd, yd, workspace=short)
    loss, lse = lm.lmce_fwd(hd, Wd, yd)
    with pytest.raises(ValueError):
        lm.lmce_bwd(hd, Wd, yd, lse.double())                     # lse must be fp32
    x = torch.randn(32, 128, device=dev).to(torch.bfloat16)
    Wg = torch.randn(64, 128, device=dev).to(torch.bfloat16)
    with pytest.raises(TypeError):
        lm.lmce_mlp_fwd(x.float(), Wg, Wg, Wg.t().contiguous(), 32)
    with pytest.raises(ValueError):
        lm.lmce_mlp_fwd(x, Wg, Wg, Wg.contiguous(), 32)           # Wd must be [H, I]
    torch.cuda.synchronize()
