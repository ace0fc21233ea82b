"""GPU parity of the pages' own chunked formulation (lmce_chunked_fwd /
lmce_chunked_bwd): every chunk's logits materialised, then the plain loss and
its backward, chunk by chunk (TRL docs "Training Beyond 1M Tokens", section
"The massive logits matrix: chunk it").  Same oracle and bar as the fused
path: mean loss relative 1e-3, every row's lse absolute 2e-3, dh and dW
relative Frobenius 1e-2; ragged shapes, several chunk sizes, the edge cases,
and the Qwen3 heads (in full at 0.6B, the first 1024 rows at 8B and 32B)."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import lm_head_chunked_amd as lm
from lm_head_chunked_amd import _lib, synth

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def np32(t):
    return t.detach().float().cpu().numpy()


def rel_fro(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def run_chunked(h, W, y, chunk_rows=256, grad=1.0, ignore_index=-100):
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    L, H = h.shape
    V = W.shape[0]
    ws = torch.empty(lm.lmce_chunked_workspace_size(L, H, V, chunk_rows), dtype=torch.uint8, device=dev)
    loss, lse = lm.lmce_chunked_fwd(hd, Wd, yd, ignore_index, chunk_rows, ws)
    g = torch.tensor(grad, dtype=torch.float32, device=dev)
    dh, dW = lm.lmce_chunked_bwd(hd, Wd, yd, g, ignore_index, chunk_rows, ws)
    status = lm.lmce_read_status(ws)
    torch.cuda.synchronize()
    return {"loss": float(loss), "lse": lse.cpu().numpy(), "dh": dh.cpu().numpy(), "dW": dW.cpu().numpy(),
            "status": status}


def check(gpu, ref, what):
    e = (abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"]), float(np.max(np.abs(gpu["lse"] - ref["lse"]))),
         rel_fro(gpu["dh"], ref["dh"]), rel_fro(gpu["dW"], ref["dW"]))
    say(f"[chunked {what}] loss rel {e[0]:.2e} lse abs {e[1]:.2e} dh rel {e[2]:.2e} dW rel {e[3]:.2e}")
    assert gpu["status"] == _lib.LMCE_OK
    assert e[0] <= 1e-3 and e[1] <= 2e-3 and e[2] <= 1e-2 and e[3] <= 1e-2


CASES = [
    (512, 256, 4096, 0.1, 256),
    (300, 128, 700, 0.2, 256),
    (1, 128, 1, 0.0, 256),
    (77, 128, 4097, 0.5, 32),
    (1000, 512, 130, 0.05, 96),
    (513, 640, 2000, 0.3, 1000),
    (2100, 384, 3000, 0.1, 256),
    (600, 3072, 5500, 0.1, 4096),
]


@pytest.mark.parametrize("L,H,V,ign,chunk", CASES)
def test_chunked_parity(L, H, V, ign, chunk):
    say(f"[case] chunked L={L} H={H} V={V} ignore={ign} chunk_rows={chunk}")
    h, W, y = synth.random_case(L, H, V, seed=L + V + 5, w_std=0.05, ignore_frac=ign)
    gpu = run_chunked(h, W, y, chunk_rows=chunk, grad=1.5)
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy(), grad=1.5)
    if ref["n_valid"] == 0 or abs(ref["loss"]) < 1e-6:
        assert np.max(np.abs(gpu["lse"] - ref["lse"])) <= 2e-3
        return
    check(gpu, ref, f"L={L} H={H} V={V} chunk={chunk}")
    assert np.all(gpu["dh"][(y == -100).numpy()] == 0.0)


def test_chunked_edge_cases():
    say("[case] chunked: W = 0, no labelled row, a bad label")
    L, H, V = 200, 128, 4096
    h, _, y = synth.random_case(L, H, V, seed=3, ignore_frac=0.1)
    W = torch.zeros(V, H, dtype=torch.bfloat16)
    gpu = run_chunked(h, W, y)
    assert np.max(np.abs(gpu["lse"] - math.log(V))) <= 1e-5 and abs(gpu["loss"] - math.log(V)) <= 1e-5
    assert np.all(gpu["dh"] == 0.0)
    h, W, y = synth.random_case(130, 128, 500, seed=4)
    y[:] = -100
    gpu = run_chunked(h, W, y)
    assert math.isnan(gpu["loss"]) and np.all(np.isfinite(gpu["lse"]))
    assert np.all(gpu["dh"] == 0.0) and np.all(gpu["dW"] == 0.0)
    h, W, y = synth.random_case(64, 128, 100, seed=6, ignore_frac=0.0)
    y[10] = 100
    gpu = run_chunked(h, W, y)
    assert gpu["status"] == _lib.LMCE_ERR_LABEL and math.isnan(gpu["loss"])


def test_chunked_06b_head_full_parity():
    """Qwen3-0.6B head in full (8192 rows, 32 chunks) against the oracle."""
    say("[case] chunked vs oracle, qwen3_0.6b head")
    h, W, y = synth.make("qwen3_0.6b")
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    check(run_chunked(h, W, y), ref, "qwen3_0.6b")


@pytest.mark.parametrize("name", ["qwen3_8b_1m_shard", "qwen3_32b"])
def test_chunked_reduced_rows(name):
    wl = synth.WORKLOADS[name]
    Lr = 1024
    say(f"[case] chunked {name} first {Lr} rows at H={wl.H} V={wl.V}")
    h, W, y = synth.make(wl)
    h, y = h[:Lr].contiguous(), y[:Lr].contiguous()
    ref = oracle.fwd_bwd(np32(h), np32(W), y.numpy())
    check(run_chunked(h, W, y), ref, f"{name} L={Lr}")
