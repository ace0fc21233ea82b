"""Runs either pair of entry points of the loss on device tensors.

plain:  lmce_fwd, then lmce_bwd.
train:  lmce_fwd_train (O into the dh buffer), then lmce_bwd_train (dh formed
        in place in that buffer, and dW).
"""

import lm_head_chunked_amd as lm


def run_pair(train, h, W, y, ignore_index, chunk_rows, ws, grad=None):
    """(loss, lse, dh, dW) of one forward + backward on workspace ws."""
    if train:
        loss, lse, dh = lm.lmce_fwd_train(h, W, y, ignore_index, chunk_rows, ws)
        dh, dW = lm.lmce_bwd_train(h, W, y, lse, grad, ignore_index, chunk_rows, ws, dh)
    else:
        loss, lse = lm.lmce_fwd(h, W, y, ignore_index, chunk_rows, ws)
        dh, dW = lm.lmce_bwd(h, W, y, lse, grad, ignore_index, chunk_rows, ws)
    return loss, lse, dh, dW
