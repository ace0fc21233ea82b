"""Seeded synthetic inputs for the LM-head + cross-entropy loss.

This module only draws random inputs.  It holds none of the loss arithmetic,
and it is the one module that both the CPU oracle's tests and the HIP path's
tests and benchmark share.

Shapes are the LM heads of the Qwen3 family (hidden size H, vocabulary
V = 151936).  Sequence lengths follow TRL docs "Training Beyond 1M Tokens":
163,840 tokens (160k) is the single-card reach of the chunked loss (section
"The massive logits matrix: chunk it"), and 131,072 rows is one GPU's share
of a 1,048,576-token sequence split over 8 GPUs (section "One GPU is not
enough: split the sequence across many").  The pages train on PG-19 books;
the labels here stand in for them: uniform, or a Zipf law (s = 1.1) over the
vocabulary, the usual shape of natural-text token frequencies.

Recipe (fixed, so that every run draws the same bits for a given seed):
  * each tensor is drawn from its own ``torch.Generator`` on ``device``,
    seeded with ``seed * 7919 + k`` (k = 0 h, 1 W, 2 labels, 3 ignored set);
  * h = h_scale * N(0, 1) drawn in float32, then rounded to bf16 (RNE);
  * W = 0.02 * N(0, 1) drawn in float32, then rounded to bf16 (RNE);
  * labels: uniform integers in [0, V), or truncated Zipf over ranks
    1..V with P(k) proportional to k^-s, label = rank - 1, drawn by inverse
    CDF from uniform draws;
  * exactly round(p * L) rows (a seeded permutation's first ones) get
    ignore_index = -100; the 8B-shaped workload ignores row 0 only.

Draws on a CUDA device and on the CPU give different bits for the same seed;
a test that compares the two paths draws once and copies the tensors.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

IGNORE_INDEX = -100
QWEN3_VOCAB = 151936


@dataclass(frozen=True)
class Workload:
    name: str
    L: int
    H: int
    V: int
    h_scale: float
    w_std: float
    labels: str  # "uniform" or "zipf"
    zipf_s: float
    ignore_frac: float
    ignore_first_only: bool
    chunk_rows: int

    def with_rows(self, L: int) -> "Workload":
        return replace(self, L=L)

    def n_ignored(self) -> int:
        if self.ignore_first_only:
            return 1 if self.L > 0 else 0
        return int(round(self.ignore_frac * self.L))

    def n_valid(self) -> int:
        return self.L - self.n_ignored()


WORKLOADS = {
    # tiny reference: a case the CPU oracle finishes in seconds
    "tiny": Workload("tiny", 512, 256, 4096, 1.0, 0.02, "uniform", 0.0, 0.10, False, 256),
    # Qwen3-0.6B head
    "qwen3_0.6b": Workload("qwen3_0.6b", 8192, 1024, QWEN3_VOCAB, 0.5, 0.02, "uniform", 0.0, 0.05, False, 256),
    # Qwen3-4B head, single-card 160k context
    "qwen3_4b_160k": Workload("qwen3_4b_160k", 163840, 2560, QWEN3_VOCAB, 1.0, 0.02, "zipf", 1.1, 0.0, False, 256),
    # Qwen3-8B head, one GPU's 131072-row share of a 1,048,576-token sequence
    "qwen3_8b_1m_shard": Workload("qwen3_8b_1m_shard", 131072, 4096, QWEN3_VOCAB, 1.0, 0.02, "zipf", 1.1, 0.0, True, 256),
    # Qwen3-32B head, wider logit range
    "qwen3_32b": Workload("qwen3_32b", 131072, 5120, QWEN3_VOCAB, 2.0, 0.02, "uniform", 0.0, 0.20, False, 256),
}


def _gen(device, seed, k):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 7919 + k)
    return g


def zipf_cdf(V: int, s: float) -> np.ndarray:
    """Normalised CDF of the truncated Zipf law over ranks 1..V (float64)."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def draw_labels(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    g = _gen(device, seed, 2)
    if wl.labels == "uniform":
        y = torch.randint(0, wl.V, (wl.L,), generator=g, device=device, dtype=torch.int64)
    elif wl.labels == "zipf":
        u = torch.rand(wl.L, generator=g, device=device, dtype=torch.float64)
        cdf = torch.from_numpy(zipf_cdf(wl.V, wl.zipf_s)).to(device)
        y = torch.searchsorted(cdf, u, right=True).clamp_(max=wl.V - 1)
    else:
        raise ValueError(wl.labels)
    n_ign = wl.n_ignored()
    if wl.ignore_first_only:
        if wl.L > 0:
            y[0] = IGNORE_INDEX
    elif n_ign > 0:
        gi = _gen(device, seed, 3)
        idx = torch.randperm(wl.L, generator=gi, device=device)[:n_ign]
        y[idx] = IGNORE_INDEX
    return y


def draw_h(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    g = _gen(device, seed, 0)
    h = torch.randn(wl.L, wl.H, generator=g, device=device, dtype=torch.float32)
    if wl.h_scale != 1.0:
        h.mul_(wl.h_scale)
    return h.to(torch.bfloat16)


def draw_W(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    g = _gen(device, seed, 1)
    W = torch.randn(wl.V, wl.H, generator=g, device=device, dtype=torch.float32)
    W.mul_(wl.w_std)
    return W.to(torch.bfloat16)


def make(wl, device="cpu", seed: int = 0):
    """(h bf16 [L,H], W bf16 [V,H], labels int64 [L]) for a workload or its name."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    return draw_h(wl, device, seed), draw_W(wl, device, seed), draw_labels(wl, device, seed)


def random_case(L, H, V, seed=0, h_scale=1.0, w_std=0.02, ignore_frac=0.1, device="cpu"):
    """A small ad-hoc case with uniform labels (for property and edge tests)."""
    wl = Workload("adhoc", L, H, V, h_scale, w_std, "uniform", 0.0, ignore_frac, False, 256)
    return make(wl, device, seed)


def shift_labels(tokens: torch.Tensor, ignore_index: int = IGNORE_INDEX) -> torch.Tensor:
    """Causal-LM shift: labels[i] = tokens[i + 1], the last row ignored.

    The library never shifts; a caller that holds input token ids uses this.
    """
    y = torch.empty_like(tokens)
    if tokens.numel() > 0:
        y[:-1] = tokens[1:]
        y[-1] = ignore_index
    return y
