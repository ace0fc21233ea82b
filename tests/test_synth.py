"""CPU tests of the seeded input generator (no loss arithmetic lives there)."""

import numpy as np
import torch

from lm_head_chunked_amd import synth


def test_workload_table_shapes():
    w = synth.WORKLOADS
    assert (w["tiny"].L, w["tiny"].H, w["tiny"].V) == (512, 256, 4096)
    assert (w["qwen3_8b_1m_shard"].L, w["qwen3_8b_1m_shard"].H) == (131072, 4096)
    assert w["qwen3_8b_1m_shard"].L * 8 == 1048576
    assert w["qwen3_4b_160k"].L == 160 * 1024
    for wl in w.values():
        assert wl.chunk_rows == 256


def test_tiny_draw_is_seeded_and_bf16():
    h, W, y = synth.make("tiny")
    h2, W2, y2 = synth.make("tiny")
    assert h.dtype == torch.bfloat16 and W.dtype == torch.bfloat16 and y.dtype == torch.int64
    assert torch.equal(h, h2) and torch.equal(W, W2) and torch.equal(y, y2)
    assert int((y == -100).sum()) == round(0.1 * 512)
    valid = y[y != -100]
    assert int(valid.min()) >= 0 and int(valid.max()) < 4096
    assert abs(float(W.float().std()) - 0.02) < 0.001
    assert abs(float(h.float().std()) - 1.0) < 0.01


def test_zipf_labels_follow_the_law():
    wl = synth.WORKLOADS["qwen3_8b_1m_shard"].with_rows(200000)
    y = synth.draw_labels(wl)
    assert int(y[0]) == -100 and int((y == -100).sum()) == 1
    yv = y[1:].numpy()
    cdf = synth.zipf_cdf(wl.V, 1.1)
    # frequency of rank 1 and of the first ten ranks against the law
    p1 = cdf[0]
    p10 = cdf[9]
    assert abs((yv == 0).mean() - p1) < 5 * np.sqrt(p1 * (1 - p1) / yv.size)
    assert abs((yv < 10).mean() - p10) < 5 * np.sqrt(p10 * (1 - p10) / yv.size)
    assert yv.max() < wl.V


def test_shift_labels():
    t = torch.tensor([5, 6, 7, 8])
    assert synth.shift_labels(t).tolist() == [6, 7, 8, -100]


def test_mlp_draws_are_seeded_and_shaped():
    x, Wg, Wu, Wd, dy = synth.make_mlp("mlp_tiny")
    wl = synth.MLP_WORKLOADS["mlp_tiny"]
    assert x.shape == (wl.L, wl.H) and Wg.shape == (wl.I, wl.H) and Wu.shape == (wl.I, wl.H)
    assert Wd.shape == (wl.H, wl.I) and dy.shape == (wl.L, wl.H)
    assert all(t.dtype == torch.bfloat16 for t in (x, Wg, Wu, Wd, dy))
    x2 = synth.make_mlp("mlp_tiny")[0]
    assert torch.equal(x, x2)
    assert not torch.equal(Wg, Wu)  # separate generators
    assert abs(float(Wg.float().std()) - 0.02) < 0.002 and abs(float(x.float().std()) - 1.0) < 0.05
