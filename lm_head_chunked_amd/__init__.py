"""MI355X-native fused LM-head + cross-entropy (chunked NLL) loss.

Python binding of the C ABI in ``include/lmce.h``.  PyTorch only allocates
device memory and supplies the current HIP stream; every step of the loss
runs in the HIP kernels of ``liblmce.so``.  There is no CPU or PyTorch
fallback: without the built library every call raises.

Page: TRL docs "Training Beyond 1M Tokens", sections "The loss is the first
thing to break" and "The massive logits matrix: chunk it" (256-row chunks by
default).
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import LmceError

IGNORE_INDEX = -100
DEFAULT_CHUNK_ROWS = 256

__all__ = [
    "lmce_workspace_size",
    "lmce_fwd",
    "lmce_bwd",
    "lmce_bwd_dh",
    "lmce_bwd_dW",
    "lmce_fwd_train",
    "lmce_bwd_train",
    "lmce_read_status",
    "lmce_fwd_noalloc",
    "lmce_chunked_workspace_size",
    "lmce_chunked_fwd",
    "lmce_chunked_bwd",
    "lmce_mlp_workspace_size",
    "lmce_mlp_fwd",
    "lmce_mlp_bwd",
    "chunked_nll",
    "LmceError",
    "IGNORE_INDEX",
    "DEFAULT_CHUNK_ROWS",
]


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check_inputs(h, W, labels):
    if not (h.is_cuda and W.is_cuda and labels.is_cuda):
        raise ValueError("h, W and labels must be device tensors")
    if h.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
        raise TypeError("h and W must be bfloat16")
    if labels.dtype != torch.int64:
        raise TypeError("labels must be int64")
    if h.dim() != 2 or W.dim() != 2 or labels.dim() != 1:
        raise ValueError("expected h [L, H], W [V, H], labels [L]")
    if h.shape[1] != W.shape[1] or labels.shape[0] != h.shape[0]:
        raise ValueError(f"shape mismatch: h {tuple(h.shape)}, W {tuple(W.shape)}, labels {tuple(labels.shape)}")
    if not (h.is_contiguous() and W.is_contiguous() and labels.is_contiguous()):
        raise ValueError("h, W and labels must be contiguous")
    return h.shape[0], h.shape[1], W.shape[0]


def lmce_workspace_size(L, H, V, chunk_rows=DEFAULT_CHUNK_ROWS) -> int:
    """Bytes of device workspace lmce_fwd / lmce_bwd need (never an L x V buffer)."""
    return _lib.workspace_size(L, H, V, chunk_rows)


def _workspace(L, H, V, chunk_rows, device, workspace):
    need = _lib.workspace_size(L, H, V, chunk_rows)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {need}")
    return workspace


def lmce_fwd(h, W, labels, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS, workspace=None,
             loss_out=None, lse_out=None):
    """Mean NLL loss (fp32 scalar tensor) and per-row logsumexp (fp32 [L])."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    ws = _workspace(L, H, V, chunk_rows, dev, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev) if loss_out is None else loss_out
    lse = torch.empty(L, dtype=torch.float32, device=dev) if lse_out is None else lse_out
    st = _lib.fwd(h.data_ptr(), W.data_ptr(), labels.data_ptr(), L, H, V, ignore_index, chunk_rows,
                  loss.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_fwd")
    return loss, lse


def lmce_fwd_noalloc(h, W, labels, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS, loss_out=None,
                     lse_out=None):
    """lmce_fwd on the library's fixed device area instead of a workspace
    (the C entry point allocates nothing; pass loss_out and lse_out to keep
    this wrapper from allocating them).  Calls that overlap on one device race."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    loss = torch.empty((), dtype=torch.float32, device=dev) if loss_out is None else loss_out
    lse = torch.empty(L, dtype=torch.float32, device=dev) if lse_out is None else lse_out
    st = _lib.fwd_noalloc(h.data_ptr(), W.data_ptr(), labels.data_ptr(), L, H, V, ignore_index, chunk_rows,
                          loss.data_ptr(), lse.data_ptr(), _stream(dev))
    _lib.check(st, "lmce_fwd_noalloc")
    return loss, lse


def lmce_fwd_train(h, W, labels, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS, workspace=None,
                   loss_out=None, lse_out=None, dh_out=None):
    """As lmce_fwd, and also writes into dh_out (fp32 [L, H], allocated if
    None) what lmce_bwd_train needs to form dh there without recomputing the
    logits.  Returns (loss, lse, dh_buffer); pass the same workspace and
    dh_buffer on to lmce_bwd_train."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    if workspace is None:
        raise ValueError("lmce_fwd_train needs an explicit workspace to hand to lmce_bwd_train")
    ws = _workspace(L, H, V, chunk_rows, dev, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev) if loss_out is None else loss_out
    lse = torch.empty(L, dtype=torch.float32, device=dev) if lse_out is None else lse_out
    dh = torch.empty(L, H, dtype=torch.float32, device=dev) if dh_out is None else dh_out
    if dh.dtype != torch.float32 or dh.shape != (L, H) or not dh.is_contiguous():
        raise ValueError("dh_out must be contiguous fp32 [L, H]")
    st = _lib.fwd_train(h.data_ptr(), W.data_ptr(), labels.data_ptr(), L, H, V, ignore_index, chunk_rows,
                        loss.data_ptr(), lse.data_ptr(), dh.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                        _stream(dev))
    _lib.check(st, "lmce_fwd_train")
    return loss, lse, dh


def lmce_bwd_train(h, W, labels, lse, grad_loss=None, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS,
                   workspace=None, dh_out=None, dW_out=None):
    """dh and dW like lmce_bwd, after lmce_fwd_train on the same inputs and
    workspace; dh_out must be the dh buffer that lmce_fwd_train returned (dh
    is formed in place there)."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    if lse.dtype != torch.float32 or lse.shape != (L,) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [L]")
    if workspace is None or dh_out is None:
        raise ValueError("lmce_bwd_train needs the workspace and the dh buffer of lmce_fwd_train")
    if grad_loss is None:
        grad_loss = torch.ones((), dtype=torch.float32, device=dev)
    grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    ws = _workspace(L, H, V, chunk_rows, dev, workspace)
    dh = dh_out
    if dh.dtype != torch.float32 or dh.shape != (L, H) or not dh.is_contiguous():
        raise ValueError("dh_out must be contiguous fp32 [L, H]")
    dW = torch.empty(V, H, dtype=torch.float32, device=dev) if dW_out is None else dW_out
    st = _lib.bwd_train(h.data_ptr(), W.data_ptr(), labels.data_ptr(), lse.data_ptr(), L, H, V, ignore_index,
                        chunk_rows, grad_loss.data_ptr(), dh.data_ptr(), dW.data_ptr(), ws.data_ptr(),
                        ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_bwd_train")
    return dh, dW


def lmce_bwd(h, W, labels, lse, grad_loss=None, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS,
             workspace=None, dh_out=None, dW_out=None):
    """dh (fp32 [L, H]) and dW (fp32 [V, H]) of grad_loss * loss (overwritten)."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    if lse.dtype != torch.float32 or lse.shape != (L,) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [L]")
    if grad_loss is None:
        grad_loss = torch.ones((), dtype=torch.float32, device=dev)
    grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    ws = _workspace(L, H, V, chunk_rows, dev, workspace)
    dh = torch.empty(L, H, dtype=torch.float32, device=dev) if dh_out is None else dh_out
    dW = torch.empty(V, H, dtype=torch.float32, device=dev) if dW_out is None else dW_out
    st = _lib.bwd(h.data_ptr(), W.data_ptr(), labels.data_ptr(), lse.data_ptr(), L, H, V, ignore_index, chunk_rows,
                  grad_loss.data_ptr(), dh.data_ptr(), dW.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                  _stream(dev))
    _lib.check(st, "lmce_bwd")
    return dh, dW


def _bwd_one(which, h, W, labels, lse, grad_loss, ignore_index, chunk_rows, workspace, out):
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    if lse.dtype != torch.float32 or lse.shape != (L,) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous fp32 [L]")
    if grad_loss is None:
        grad_loss = torch.ones((), dtype=torch.float32, device=dev)
    grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    ws = _workspace(L, H, V, chunk_rows, dev, workspace)
    rows = L if which == "dh" else V
    if out is None:
        out = torch.empty(rows, H, dtype=torch.float32, device=dev)
    fn = _lib.bwd_dh if which == "dh" else _lib.bwd_dW
    st = fn(h.data_ptr(), W.data_ptr(), labels.data_ptr(), lse.data_ptr(), L, H, V, ignore_index, chunk_rows,
            grad_loss.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, f"lmce_bwd_{which}")
    return out


def lmce_bwd_dh(h, W, labels, lse, grad_loss=None, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS,
                workspace=None, dh_out=None):
    """dh (fp32 [L, H]) alone, e.g. for a frozen LM head."""
    return _bwd_one("dh", h, W, labels, lse, grad_loss, ignore_index, chunk_rows, workspace, dh_out)


def lmce_bwd_dW(h, W, labels, lse, grad_loss=None, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS,
                workspace=None, dW_out=None):
    """dW (fp32 [V, H]) alone."""
    return _bwd_one("dW", h, W, labels, lse, grad_loss, ignore_index, chunk_rows, workspace, dW_out)


def lmce_chunked_workspace_size(L, H, V, chunk_rows=DEFAULT_CHUNK_ROWS) -> int:
    """Workspace bytes of the materialised-chunk comparison path (one chunk's fp32 logits and more)."""
    return _lib.chunked_workspace_size(L, H, V, chunk_rows)


def _chunked_ws(L, H, V, chunk_rows, device, workspace):
    need = _lib.chunked_workspace_size(L, H, V, chunk_rows)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {need}")
    return workspace


def lmce_chunked_fwd(h, W, labels, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS, workspace=None,
                     loss_out=None, lse_out=None):
    """The pages' chunked formulation: each chunk's logits materialised, loss and lse as lmce_fwd."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    ws = _chunked_ws(L, H, V, chunk_rows, dev, workspace)
    loss = torch.empty((), dtype=torch.float32, device=dev) if loss_out is None else loss_out
    lse = torch.empty(L, dtype=torch.float32, device=dev) if lse_out is None else lse_out
    st = _lib.chunked_fwd(h.data_ptr(), W.data_ptr(), labels.data_ptr(), L, H, V, ignore_index, chunk_rows,
                          loss.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_chunked_fwd")
    return loss, lse


def lmce_chunked_bwd(h, W, labels, grad_loss=None, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS,
                     workspace=None, dh_out=None, dW_out=None):
    """The pages' chunked formulation of the backward: dh and dW as lmce_bwd."""
    L, H, V = _check_inputs(h, W, labels)
    dev = h.device
    if grad_loss is None:
        grad_loss = torch.ones((), dtype=torch.float32, device=dev)
    grad_loss = grad_loss.to(device=dev, dtype=torch.float32).contiguous()
    ws = _chunked_ws(L, H, V, chunk_rows, dev, workspace)
    dh = torch.empty(L, H, dtype=torch.float32, device=dev) if dh_out is None else dh_out
    dW = torch.empty(V, H, dtype=torch.float32, device=dev) if dW_out is None else dW_out
    st = _lib.chunked_bwd(h.data_ptr(), W.data_ptr(), labels.data_ptr(), L, H, V, ignore_index, chunk_rows,
                          grad_loss.data_ptr(), dh.data_ptr(), dW.data_ptr(), ws.data_ptr(),
                          ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_chunked_bwd")
    return dh, dW


def _check_mlp(x, Wg, Wu, Wd, dy=None):
    ts = [x, Wg, Wu, Wd] + ([dy] if dy is not None else [])
    if not all(t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and t.dim() == 2 for t in ts):
        raise TypeError("x, Wg, Wu, Wd (and dy) must be contiguous 2-D bf16 device tensors")
    L, H = x.shape
    I = Wg.shape[0]
    if Wg.shape != (I, H) or Wu.shape != (I, H) or Wd.shape != (H, I) or (dy is not None and dy.shape != (L, H)):
        raise ValueError(f"shapes: x {tuple(x.shape)}, Wg {tuple(Wg.shape)}, Wu {tuple(Wu.shape)}, "
                         f"Wd {tuple(Wd.shape)}" + ("" if dy is None else f", dy {tuple(dy.shape)}"))
    return L, H, I


def lmce_mlp_workspace_size(L, H, I, chunk_rows) -> int:
    """Workspace bytes of the sequence-tiled MLP (packed weights and one chunk's intermediates)."""
    return _lib.mlp_workspace_size(L, H, I, chunk_rows)


def _mlp_ws(L, H, I, chunk_rows, device, workspace):
    need = _lib.mlp_workspace_size(L, H, I, chunk_rows)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {need}")
    return workspace


def lmce_mlp_fwd(x, Wg, Wu, Wd, chunk_rows=4096, workspace=None, y_out=None):
    """y = down_proj(silu(gate_proj(x)) * up_proj(x)) (fp32 [L, H]), chunk_rows rows at a time."""
    L, H, I = _check_mlp(x, Wg, Wu, Wd)
    dev = x.device
    ws = _mlp_ws(L, H, I, chunk_rows, dev, workspace)
    y = torch.empty(L, H, dtype=torch.float32, device=dev) if y_out is None else y_out
    st = _lib.mlp_fwd(x.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), L, H, I, chunk_rows, y.data_ptr(),
                      ws.data_ptr(), ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_mlp_fwd")
    return y


def lmce_mlp_bwd(x, Wg, Wu, Wd, dy, chunk_rows=4096, workspace=None, dx_out=None, dWg_out=None, dWu_out=None,
                 dWd_out=None):
    """(dx, dWg, dWu, dWd), fp32, for the upstream gradient dy (bf16 [L, H]) of y."""
    L, H, I = _check_mlp(x, Wg, Wu, Wd, dy)
    dev = x.device
    ws = _mlp_ws(L, H, I, chunk_rows, dev, workspace)
    f32 = dict(dtype=torch.float32, device=dev)
    dx = torch.empty(L, H, **f32) if dx_out is None else dx_out
    dWg = torch.empty(I, H, **f32) if dWg_out is None else dWg_out
    dWu = torch.empty(I, H, **f32) if dWu_out is None else dWu_out
    dWd = torch.empty(H, I, **f32) if dWd_out is None else dWd_out
    st = _lib.mlp_bwd(x.data_ptr(), Wg.data_ptr(), Wu.data_ptr(), Wd.data_ptr(), dy.data_ptr(), L, H, I, chunk_rows,
                      dx.data_ptr(), dWg.data_ptr(), dWu.data_ptr(), dWd.data_ptr(), ws.data_ptr(),
                      ws.numel() * ws.element_size(), _stream(dev))
    _lib.check(st, "lmce_mlp_bwd")
    return dx, dWg, dWu, dWd


def lmce_read_status(workspace) -> int:
    """Synchronises the current stream; the asynchronous status recorded by the last calls."""
    return _lib.read_status(workspace.data_ptr(), _stream(workspace.device))


class _ChunkedNLL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, h, W, labels, ignore_index, chunk_rows):
        L, H, V = _check_inputs(h, W, labels)
        ws = _workspace(L, H, V, chunk_rows, h.device, None)
        loss, lse, dh = lmce_fwd_train(h, W, labels, ignore_index, chunk_rows, ws)
        ctx.save_for_backward(h, W, labels, lse)
        ctx.ignore_index = ignore_index
        ctx.chunk_rows = chunk_rows
        ctx.ws = ws
        ctx.dh = dh
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        h, W, labels, lse = ctx.saved_tensors
        dh, dW = lmce_bwd_train(h, W, labels, lse, grad_loss, ctx.ignore_index, ctx.chunk_rows, ctx.ws, ctx.dh)
        ctx.ws = None
        ctx.dh = None
        return dh, dW, None, None, None


def chunked_nll(h, W, labels, ignore_index=IGNORE_INDEX, chunk_rows=DEFAULT_CHUNK_ROWS):
    """Differentiable mean NLL of log_softmax(h W^T) against labels (TRL's
    ``loss_type="chunked_nll"``), computed without an L x V logits buffer."""
    return _ChunkedNLL.apply(h, W, labels, ignore_index, chunk_rows)
