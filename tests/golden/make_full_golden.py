#!/usr/bin/env python3
"""Writes full-length oracle values for the three long Qwen3 head workloads.

    python tests/golden/make_full_golden.py [workload ...]

For each workload (Qwen3-4B head at 160k rows, Qwen3-8B head at one GPU's
131072-row share of a 1,048,576-token sequence, Qwen3-32B head at 131072
rows) it draws the seed-0 inputs on the CPU with the shared input generator,
runs the fp64 CPU oracle's forward over EVERY row (full vocabulary, plain
log-softmax; TRL docs "Training Beyond 1M Tokens", section "The loss is the
first thing to break") and stores:

  full_<workload>.json   the mean loss (fp64), N_valid, the sha256 digests of
                         the bf16 bits of h and W and of the int64 labels, and
                         the command that wrote it
  full_<workload>.npy    lse of every row, float64 [L]

Only the oracle computes these values; the GPU path is never called here.
The GPU tests draw the same inputs on the CPU, check the digests, copy the
bits to the device and compare both pairs of entry points with these values.
"""

from __future__ import annotations

import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

LONG = ["qwen3_4b_160k", "qwen3_8b_1m_shard", "qwen3_32b"]


def digest(t) -> str:
    """sha256 of a CPU tensor's raw bytes (bf16 bits for h and W, int64 for labels)."""
    import torch

    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()


def golden_paths(name):
    return os.path.join(HERE, f"full_{name}.json"), os.path.join(HERE, f"full_{name}.npy")


def write(name):
    import numpy as np

    import oracle
    from lm_head_chunked_amd import synth

    wl = synth.WORKLOADS[name]
    t0 = time.time()
    h, W, y = synth.make(wl)  # CPU draw, seed 0
    rec = {"workload": name, "L": wl.L, "H": wl.H, "V": wl.V, "seed": 0,
           "h_sha256": digest(h), "W_sha256": digest(W), "labels_sha256": digest(y)}
    print(f"[{name}] inputs drawn in {time.time() - t0:.1f} s", flush=True)
    h_np = h.float().numpy()
    W_np = W.float().numpy()
    y_np = y.numpy()
    del h, W
    t1 = time.time()
    out = oracle.forward(h_np, W_np, y_np)
    dt = time.time() - t1
    rec.update({"loss": out["loss"], "n_valid": out["n_valid"], "oracle_seconds": round(dt, 1),
                "written_by": "python tests/golden/make_full_golden.py " + name,
                "values": "loss: fp64 mean NLL over non-ignored rows; full_<workload>.npy: fp64 lse of every row"})
    jp, npp = golden_paths(name)
    np.save(npp, out["lse"].astype(np.float64))
    with open(jp, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(f"[{name}] oracle forward over {wl.L} rows in {dt:.0f} s: loss {out['loss']:.9f}", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or LONG
    for n in names:
        if n not in LONG:
            raise SystemExit(f"unknown workload {n}; choose from {LONG}")
        write(n)
