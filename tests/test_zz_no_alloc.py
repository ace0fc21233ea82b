"""The allocation-free forward, lmce_fwd_noalloc, through the C ABI.

It runs the plain forward's kernels on the library's fixed device area
instead of a caller's workspace, for callers that cannot allocate.  Checked
against lmce_fwd on the same inputs (bitwise: the same kernels in the same
order) and against the fp64 oracle within the parity bar (loss relative
1e-3, every row's lse absolute 2e-3), on two calls in a row whose second is
smaller than the first, so that the area still holds the first call's
larger contents.
"""

import ctypes
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


def noalloc_via_abi(h, W, y, chunk_rows=256, ignore_index=-100):
    """Direct ctypes call of lmce_fwd_noalloc; outputs pre-allocated by the test."""
    L, H = h.shape
    V = W.shape[0]
    loss = torch.full((), float("inf"), dtype=torch.float32, device=h.device)
    lse = torch.full((L,), float("inf"), dtype=torch.float32, device=h.device)
    stream = torch.cuda.current_stream(h.device).cuda_stream
    st = _lib.load().lmce_fwd_noalloc(h.data_ptr(), W.data_ptr(), y.data_ptr(), L, H, V, ignore_index, chunk_rows,
                                      loss.data_ptr(), lse.data_ptr(), stream)
    return st, loss, lse


def test_noalloc_forward_matches_lmce_fwd_on_two_calls():
    dev = torch.device("cuda:0")
    cases = [(3000, 512, 9000, 0.1, 256), (700, 256, 3001, 0.3, 96)]  # the second call is smaller
    for L, H, V, ign, chunk in cases:
        say(f"[case] lmce_fwd_noalloc L={L} H={H} V={V} ignore={ign} chunk_rows={chunk}")
        h, W, y = synth.random_case(L, H, V, seed=L + V, w_std=0.05, ignore_frac=ign)
        hd, Wd, yd = h.to(dev), W.to(dev), y.to(dev)
        st, loss, lse = noalloc_via_abi(hd, Wd, yd, chunk)
        assert st == _lib.LMCE_OK, _lib.strerror(st)
        ws = torch.empty(lm.lmce_workspace_size(L, H, V, chunk), dtype=torch.uint8, device=dev)
        loss_ref, lse_ref = lm.lmce_fwd(hd, Wd, yd, -100, chunk, ws)
        assert lm.lmce_read_status(ws) == _lib.LMCE_OK
        torch.cuda.synchronize()
        assert float(loss) == float(loss_ref)
        assert torch.equal(lse, lse_ref)
        ref = oracle.forward(h.float().numpy(), W.float().numpy(), y.numpy())
        e_loss = abs(float(loss) - ref["loss"]) / abs(ref["loss"])
        e_lse = float(np.max(np.abs(lse.cpu().numpy() - ref["lse"])))
        say(f"[noalloc L={L}] loss rel {e_loss:.2e} lse abs {e_lse:.2e}")
        assert e_loss <= 1e-3 and e_lse <= 2e-3


def test_noalloc_forward_status_is_per_call():
    """A bad label gives a NaN loss in that call only: the next call on the
    same area starts from a cleared header."""
    dev = torch.device("cuda:0")
    h, W, y = synth.random_case(300, 128, 700, seed=41, ignore_frac=0.1)
    hd, Wd = h.to(dev), W.to(dev)
    ybad = y.clone()
    ybad[5] = 700
    st, loss_bad, _ = noalloc_via_abi(hd, Wd, ybad.to(dev))
    assert st == _lib.LMCE_OK
    st, loss, lse = noalloc_via_abi(hd, Wd, y.to(dev))
    assert st == _lib.LMCE_OK
    torch.cuda.synchronize()
    assert math.isnan(float(loss_bad))
    ref = oracle.forward(h.float().numpy(), W.float().numpy(), y.numpy())
    assert abs(float(loss) - ref["loss"]) <= 1e-3 * abs(ref["loss"])


def test_noalloc_forward_refuses_shapes_past_its_area():
    dev = torch.device("cuda:0")
    L = (1 << 20) + 256
    h = torch.zeros(L, 128, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(8, 128, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(L, dtype=torch.int64, device=dev)
    st, _, _ = noalloc_via_abi(h, W, y)
    assert st == _lib.LMCE_ERR_SCRATCH
