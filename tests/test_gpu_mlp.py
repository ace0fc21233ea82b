"""GPU parity of the sequence-tiled MLP block (lmce_mlp_fwd / lmce_mlp_bwd)
against the fp64 MLP oracle (TRL docs "Training Beyond 1M Tokens", section
"One GPU is not enough: split the sequence across many").

Bar: relative Frobenius error <= 1e-2 for y, dx, dWg, dWu and dWd.  The
kernels keep the four intermediates in bf16, as the model does (the page
prices each at 2 bytes per element), and accumulate in fp32; the oracle
rounds nothing, so the bar covers the bf16 rounding of the intermediates
(about 2^-9 relative per element).  Shapes: ragged rows and widths, chunk
sizes from 96 rows to past L, the Qwen3-4B MLP (2560 -> 9728) at 4096 rows
in full, and at its 262,144-row workload on sampled rows of y and dx plus the
chunk-size consistency of the weight gradients."""

import sys

import numpy as np
import pytest
import torch

import oracle
import lm_head_chunked_amd as lm
from lm_head_chunked_amd import synth

pytestmark = pytest.mark.gpu

REL = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def np32(t):
    return t.detach().float().cpu().numpy()


def rel_fro(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def run_mlp(x, Wg, Wu, Wd, dy, chunk_rows):
    dev = torch.device("cuda:0")
    xd, Wgd, Wud, Wdd, dyd = (t.to(dev) for t in (x, Wg, Wu, Wd, dy))
    L, H = x.shape
    I = Wg.shape[0]
    ws = torch.empty(lm.lmce_mlp_workspace_size(L, H, I, chunk_rows), dtype=torch.uint8, device=dev)
    y = lm.lmce_mlp_fwd(xd, Wgd, Wud, Wdd, chunk_rows, ws)
    dx, dWg, dWu, dWd = lm.lmce_mlp_bwd(xd, Wgd, Wud, Wdd, dyd, chunk_rows, ws)
    torch.cuda.synchronize()
    return {"y": y, "dx": dx, "dWg": dWg, "dWu": dWu, "dWd": dWd}


def check(gpu, ref, what):
    errs = {k: rel_fro(np32(gpu[k]), ref[k]) for k in ("y", "dx", "dWg", "dWu", "dWd")}
    say(f"[mlp {what}] " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= REL, (k, v)


CASES = [
    (512, 256, 768, 256),
    (1, 128, 64, 256),
    (300, 128, 192, 96),
    (1000, 384, 320, 128),
    (2100, 256, 1024, 1000),
    (700, 512, 640, 65536),
]


@pytest.mark.parametrize("L,H,I,chunk", CASES)
def test_mlp_parity(L, H, I, chunk):
    say(f"[case] mlp L={L} H={H} I={I} chunk_rows={chunk}")
    x, Wg, Wu, Wd, dy = synth.random_mlp_case(L, H, I, seed=L + I, w_std=0.05)
    gpu = run_mlp(x, Wg, Wu, Wd, dy, chunk)
    ref = oracle.mlp_fwd_bwd(*(np32(t) for t in (x, Wg, Wu, Wd, dy)))
    check(gpu, ref, f"L={L} H={H} I={I} chunk={chunk}")


def test_mlp_tiny_workload_and_chunk_independence():
    """The tiny workload; y and dx do not depend on the chunk size at all
    (each row's arithmetic is the same), the weight gradients only through
    the order of their fp32 sums."""
    say("[case] mlp_tiny, chunk sizes 128 / 256 / 512")
    x, Wg, Wu, Wd, dy = synth.make_mlp("mlp_tiny")
    ref = oracle.mlp_fwd_bwd(*(np32(t) for t in (x, Wg, Wu, Wd, dy)))
    runs = {c: run_mlp(x, Wg, Wu, Wd, dy, c) for c in (128, 256, 512)}
    check(runs[256], ref, "mlp_tiny")
    for c in (128, 512):
        assert torch.equal(runs[c]["y"], runs[256]["y"]) and torch.equal(runs[c]["dx"], runs[256]["dx"])
        for k in ("dWg", "dWu", "dWd"):
            assert rel_fro(np32(runs[c][k]), np32(runs[256][k])) <= 1e-5, (c, k)


def test_mlp_qwen3_4b_shape_full_oracle():
    wl = synth.MLP_WORKLOADS["qwen3_4b_mlp_256k"].with_rows(4096)
    say(f"[case] Qwen3-4B MLP L={wl.L} H={wl.H} I={wl.I}, chunk 1024 (oracle ~10 s)")
    x, Wg, Wu, Wd, dy = synth.make_mlp(wl)
    gpu = run_mlp(x, Wg, Wu, Wd, dy, 1024)
    ref = oracle.mlp_fwd_bwd(*(np32(t) for t in (x, Wg, Wu, Wd, dy)))
    check(gpu, ref, "qwen3_4b L=4096")


def test_mlp_qwen3_4b_full_workload_sampled():
    """262,144 rows at chunk 16384: y and dx of 512 sampled rows against the
    oracle's row helpers; the weight gradients of 8 sampled units over all
    rows against the oracle's unit helper, and in full against a run at chunk
    8192."""
    wl = synth.MLP_WORKLOADS["qwen3_4b_mlp_256k"]
    say(f"[case] Qwen3-4B MLP full workload L={wl.L} H={wl.H} I={wl.I}")
    dev = torch.device("cuda:0")
    x, Wg, Wu, Wd, dy = synth.make_mlp(wl, device=dev)
    a = run_mlp(x, Wg, Wu, Wd, dy, wl.chunk_rows)
    b = run_mlp(x, Wg, Wu, Wd, dy, wl.chunk_rows // 2)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["dx"], b["dx"])
    for k in ("dWg", "dWu", "dWd"):
        e = rel_fro(np32(a[k]), np32(b[k]))
        say(f"[mlp full] {k} chunk 16384 vs 8192: {e:.2e}")
        assert e <= 1e-4
        assert bool(torch.isfinite(a[k]).all())
    g = torch.Generator().manual_seed(7)
    rows = torch.unique(torch.cat([torch.tensor([0, wl.L - 1]), torch.randperm(wl.L, generator=g)[:510]]))
    rd = rows.to(dev)
    W_np = [np32(t) for t in (Wg, Wu, Wd)]
    y_ref = oracle.mlp_rows_forward(np32(x[rd]), *W_np)
    dx_ref = oracle.mlp_rows_dx(np32(x[rd]), *W_np, np32(dy[rd]))
    e_y, e_dx = rel_fro(np32(a["y"][rd]), y_ref), rel_fro(np32(a["dx"][rd]), dx_ref)
    say(f"[mlp full] sampled rows: y {e_y:.2e} dx {e_dx:.2e}")
    assert e_y <= REL and e_dx <= REL
    cols = torch.unique(torch.cat([torch.tensor([0, wl.I - 1]), torch.randperm(wl.I, generator=g)[:6]]))
    cd = cols.to(dev)
    dWg_ref, dWu_ref, dWd_ref = oracle.mlp_cols_grads(np32(x), *W_np, np32(dy), cols.numpy())
    errs = (rel_fro(np32(a["dWg"][cd]), dWg_ref), rel_fro(np32(a["dWu"][cd]), dWu_ref),
            rel_fro(np32(a["dWd"][:, cd]), dWd_ref))
    say(f"[mlp full] {len(cols)} sampled units over all rows: dWg {errs[0]:.2e} dWu {errs[1]:.2e} dWd {errs[2]:.2e}")
    assert max(errs) <= REL
