"""GPU parity at the library's documented maximum sizes.

The C ABI accepts 1 <= L, V <= 2^21 and 128 <= H <= 16384 (H a multiple of
128).  Each case below takes one dimension to its maximum and keeps the others
small, so that the fp64 oracle still computes every output exactly; both the
plain pair and the training pair are checked against it, with ignored rows.

  * H = 16384: groups of 64 (256-wide slices) or 128 (128-wide slices)
    members, the largest exchange slots;
  * V = 2^21: 8192 vocabulary tiles, a 512 MiB weight;
  * L = 2^21: 8192 row blocks, the label compaction over 2048 chunks.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import lm_head_chunked_amd as lm
from lm_head_chunked_amd import _lib, synth
from tests.pairs import run_pair

pytestmark = pytest.mark.gpu

LIMITS = [
    (600, 16384, 3000, 0.1),
    (300, 128, 1 << 21, 0.1),
    (1 << 21, 128, 300, 0.25),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("L,H,V,ign", LIMITS)
def test_maximum_sizes(L, H, V, ign):
    say(f"[case] limits L={L} H={H} V={V} ignore={ign}")
    h, W, y = synth.random_case(L, H, V, seed=17, w_std=0.05, ignore_frac=ign)
    ref = oracle.fwd_bwd(h.float().numpy(), W.float().numpy(), y.numpy())
    dev = torch.device("cuda:0")
    hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
    ws = torch.empty(lm.lmce_workspace_size(L, H, V, 256), dtype=torch.uint8, device=dev)
    for train, name in ((False, "plain"), (True, "train")):
        loss, lse, dh, dW = run_pair(train, hd, Wd, yd, -100, 256, ws)
        assert lm.lmce_read_status(ws) == _lib.LMCE_OK
        e = (abs(float(loss) - ref["loss"]) / abs(ref["loss"]),
             float(np.max(np.abs(lse.cpu().numpy() - ref["lse"]))),
             rel_fro(dh.cpu().numpy(), ref["dh"]), rel_fro(dW.cpu().numpy(), ref["dW"]))
        say(f"[{name} L={L} H={H} V={V}] loss rel {e[0]:.2e} lse abs {e[1]:.2e} dh rel {e[2]:.2e} dW rel {e[3]:.2e}")
        assert e[0] <= 1e-3 and e[1] <= 2e-3 and e[2] <= 1e-2 and e[3] <= 1e-2
        assert np.all(dh.cpu().numpy()[(y == -100).numpy()] == 0.0)
        del dh, dW
