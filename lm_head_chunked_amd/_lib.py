"""ctypes loader for liblmce.so: argument marshalling for the C ABI only.

The library is found next to this file (built in-tree by ``build.py``).  There
is no fallback: if the library is missing or fails to load, every entry point
raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmce.so")

LMCE_OK = 0
LMCE_ERR_NULL = -1
LMCE_ERR_SHAPE = -2
LMCE_ERR_UNSUPPORTED = -3
LMCE_ERR_WORKSPACE = -4
LMCE_ERR_HIP = -5
LMCE_ERR_LABEL = -6
LMCE_ERR_STATE = -7
LMCE_ERR_SCRATCH = -8

# Every symbol the public header declares, with (restype, argtypes).
_c_i64 = ctypes.c_int64
_c_vp = ctypes.c_void_p
SIGNATURES = {
    "lmce_version": (ctypes.c_int, []),
    "lmce_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "lmce_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "lmce_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_bwd_dh": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                   _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_bwd_dW": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                   _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_fwd_train": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_bwd_train": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_read_status": (ctypes.c_int, [_c_vp, _c_vp]),
    "lmce_chunked_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "lmce_chunked_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_chunked_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_mlp_workspace_size": (ctypes.c_int, [_c_i64, _c_i64, _c_i64, _c_i64, ctypes.POINTER(ctypes.c_size_t)]),
    "lmce_mlp_fwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp,
                                    _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_mlp_bwd": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64,
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "lmce_fwd_noalloc": (ctypes.c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                        _c_vp, _c_vp, _c_vp]),
}

_lib = None


class LmceError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        msg = strerror(status) if _lib is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


def load(path: str = LIB_PATH):
    """Loads liblmce.so once and declares every signature; raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m lm_head_chunked_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    return load().lmce_strerror(int(status)).decode()


def check(status: int, what: str = ""):
    if status != LMCE_OK:
        raise LmceError(status, what)


def workspace_size(L, H, V, chunk_rows) -> int:
    n = ctypes.c_size_t(0)
    check(load().lmce_workspace_size(int(L), int(H), int(V), int(chunk_rows), ctypes.byref(n)), "lmce_workspace_size")
    return int(n.value)


def fwd(h_ptr, W_ptr, labels_ptr, L, H, V, ignore_index, chunk_rows, loss_ptr, lse_ptr, ws_ptr, ws_bytes, stream):
    return load().lmce_fwd(h_ptr, W_ptr, labels_ptr, int(L), int(H), int(V), int(ignore_index), int(chunk_rows),
                           loss_ptr, lse_ptr, ws_ptr, int(ws_bytes), stream)


def bwd(h_ptr, W_ptr, labels_ptr, lse_ptr, L, H, V, ignore_index, chunk_rows, grad_ptr, dh_ptr, dW_ptr, ws_ptr,
        ws_bytes, stream):
    return load().lmce_bwd(h_ptr, W_ptr, labels_ptr, lse_ptr, int(L), int(H), int(V), int(ignore_index),
                           int(chunk_rows), grad_ptr, dh_ptr, dW_ptr, ws_ptr, int(ws_bytes), stream)


def bwd_dh(h_ptr, W_ptr, labels_ptr, lse_ptr, L, H, V, ignore_index, chunk_rows, grad_ptr, dh_ptr, ws_ptr, ws_bytes,
           stream):
    return load().lmce_bwd_dh(h_ptr, W_ptr, labels_ptr, lse_ptr, int(L), int(H), int(V), int(ignore_index),
                              int(chunk_rows), grad_ptr, dh_ptr, ws_ptr, int(ws_bytes), stream)


def bwd_dW(h_ptr, W_ptr, labels_ptr, lse_ptr, L, H, V, ignore_index, chunk_rows, grad_ptr, dW_ptr, ws_ptr, ws_bytes,
           stream):
    return load().lmce_bwd_dW(h_ptr, W_ptr, labels_ptr, lse_ptr, int(L), int(H), int(V), int(ignore_index),
                              int(chunk_rows), grad_ptr, dW_ptr, ws_ptr, int(ws_bytes), stream)


def fwd_train(h_ptr, W_ptr, labels_ptr, L, H, V, ignore_index, chunk_rows, loss_ptr, lse_ptr, dh_ptr, ws_ptr,
              ws_bytes, stream):
    return load().lmce_fwd_train(h_ptr, W_ptr, labels_ptr, int(L), int(H), int(V), int(ignore_index),
                                 int(chunk_rows), loss_ptr, lse_ptr, dh_ptr, ws_ptr, int(ws_bytes), stream)


def bwd_train(h_ptr, W_ptr, labels_ptr, lse_ptr, L, H, V, ignore_index, chunk_rows, grad_ptr, dh_ptr, dW_ptr, ws_ptr,
              ws_bytes, stream):
    return load().lmce_bwd_train(h_ptr, W_ptr, labels_ptr, lse_ptr, int(L), int(H), int(V), int(ignore_index),
                                 int(chunk_rows), grad_ptr, dh_ptr, dW_ptr, ws_ptr, int(ws_bytes), stream)


def fwd_noalloc(h_ptr, W_ptr, labels_ptr, L, H, V, ignore_index, chunk_rows, loss_ptr, lse_ptr, stream):
    return load().lmce_fwd_noalloc(h_ptr, W_ptr, labels_ptr, int(L), int(H), int(V), int(ignore_index),
                                   int(chunk_rows), loss_ptr, lse_ptr, stream)


def chunked_workspace_size(L, H, V, chunk_rows) -> int:
    n = ctypes.c_size_t(0)
    check(load().lmce_chunked_workspace_size(int(L), int(H), int(V), int(chunk_rows), ctypes.byref(n)),
          "lmce_chunked_workspace_size")
    return int(n.value)


def chunked_fwd(h_ptr, W_ptr, labels_ptr, L, H, V, ignore_index, chunk_rows, loss_ptr, lse_ptr, ws_ptr, ws_bytes,
                stream):
    return load().lmce_chunked_fwd(h_ptr, W_ptr, labels_ptr, int(L), int(H), int(V), int(ignore_index),
                                   int(chunk_rows), loss_ptr, lse_ptr, ws_ptr, int(ws_bytes), stream)


def chunked_bwd(h_ptr, W_ptr, labels_ptr, L, H, V, ignore_index, chunk_rows, grad_ptr, dh_ptr, dW_ptr, ws_ptr,
                ws_bytes, stream):
    return load().lmce_chunked_bwd(h_ptr, W_ptr, labels_ptr, int(L), int(H), int(V), int(ignore_index),
                                   int(chunk_rows), grad_ptr, dh_ptr, dW_ptr, ws_ptr, int(ws_bytes), stream)


def mlp_workspace_size(L, H, I, chunk_rows) -> int:
    n = ctypes.c_size_t(0)
    check(load().lmce_mlp_workspace_size(int(L), int(H), int(I), int(chunk_rows), ctypes.byref(n)),
          "lmce_mlp_workspace_size")
    return int(n.value)


def mlp_fwd(x_ptr, Wg_ptr, Wu_ptr, Wd_ptr, L, H, I, chunk_rows, y_ptr, ws_ptr, ws_bytes, stream):
    return load().lmce_mlp_fwd(x_ptr, Wg_ptr, Wu_ptr, Wd_ptr, int(L), int(H), int(I), int(chunk_rows), y_ptr, ws_ptr,
                               int(ws_bytes), stream)


def mlp_bwd(x_ptr, Wg_ptr, Wu_ptr, Wd_ptr, dy_ptr, L, H, I, chunk_rows, dx_ptr, dWg_ptr, dWu_ptr, dWd_ptr, ws_ptr,
            ws_bytes, stream):
    return load().lmce_mlp_bwd(x_ptr, Wg_ptr, Wu_ptr, Wd_ptr, dy_ptr, int(L), int(H), int(I), int(chunk_rows),
                               dx_ptr, dWg_ptr, dWu_ptr, dWd_ptr, ws_ptr, int(ws_bytes), stream)


def read_status(ws_ptr, stream) -> int:
    return load().lmce_read_status(ws_ptr, stream)
