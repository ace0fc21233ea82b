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

The MLP block of the same page's section "One GPU is not enough: split the
sequence across many" (down_proj(act_fn(gate_proj(x)) * up_proj(x)), an MLP
that widens each token from 2560 to 9728 in the Qwen3-4B model) gets its own
workloads: x = N(0, 1) (a normalised hidden state), the three weights
N(0, 0.02^2), the upstream gradient dy = N(0, 1), all rounded to bf16, each
from its own generator seeded with ``seed * 7919 + k`` (k = 10 x, 11 Wg,
12 Wu, 13 Wd, 14 dy).  The long one has 262,144 rows: one GPU's share of a
1,048,576-token sequence split over four GPUs, the page's own example.
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


@dataclass(frozen=True)
class MlpWorkload:
    name: str
    L: int
    H: int
    I: int
    x_scale: float
    w_std: float
    dy_scale: float
    chunk_rows: int

    def with_rows(self, L: int) -> "MlpWorkload":
        return replace(self, L=L)


MLP_WORKLOADS = {
    # small case the fp64 oracle finishes in well under a second
    "mlp_tiny": MlpWorkload("mlp_tiny", 512, 256, 768, 1.0, 0.02, 1.0, 256),
    # Qwen3-4B MLP (2560 -> 9728), one GPU's 262,144-row share of 1,048,576 tokens over 4 GPUs
    "qwen3_4b_mlp_256k": MlpWorkload("qwen3_4b_mlp_256k", 262144, 2560, 9728, 1.0, 0.02, 1.0, 16384),
}


def _draw_bf16(shape, scale, device, seed, k):
    t = torch.randn(*shape, generator=_gen(device, seed, k), device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(torch.bfloat16)


def make_mlp(wl, device="cpu", seed: int = 0):
    """(x [L,H], Wg [I,H], Wu [I,H], Wd [H,I], dy [L,H]), all bf16, for an MLP workload or its name."""
    if isinstance(wl, str):
        wl = MLP_WORKLOADS[wl]
    return (_draw_bf16((wl.L, wl.H), wl.x_scale, device, seed, 10),
            _draw_bf16((wl.I, wl.H), wl.w_std, device, seed, 11),
            _draw_bf16((wl.I, wl.H), wl.w_std, device, seed, 12),
            _draw_bf16((wl.H, wl.I), wl.w_std, device, seed, 13),
            _draw_bf16((wl.L, wl.H), wl.dy_scale, device, seed, 14))


def random_mlp_case(L, H, I, seed=0, w_std=0.02, device="cpu"):
    """A small ad-hoc MLP case (for property and edge tests)."""
    return make_mlp(MlpWorkload("adhoc", L, H, I, 1.0, w_std, 1.0, 256), device, seed)
