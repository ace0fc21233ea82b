"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before enqueuing anything (no GPU needed)."""

import ctypes
import json
import math
import os
import re
import subprocess

import pytest

from lm_head_chunked_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmce.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

# Aligned, non-NULL addresses that are never dereferenced: every call below
# fails argument validation before touching them.
FAKE = 0x100000


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lmce_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_abi():
    syms = declared_symbols()
    for s in ["lmce_fwd", "lmce_bwd", "lmce_workspace_size", "lmce_read_status", "lmce_strerror", "lmce_version"]:
        assert s in syms
    assert set(syms) == set(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lmce_\w+)$", out, flags=re.M))
    for s in declared_symbols():
        assert s in exported, f"{s} not exported"
        assert getattr(lib, s) is not None


def test_version_and_strerror(lib):
    assert lib.lmce_version() >= 100
    for code in range(-8, 1):
        assert len(_lib.strerror(code)) > 0
    assert _lib.strerror(12345) == "unknown status"


def test_workspace_size_errors(lib):
    n = ctypes.c_size_t(0)
    assert lib.lmce_workspace_size(0, 256, 4096, 256, ctypes.byref(n)) == _lib.LMCE_ERR_SHAPE
    assert lib.lmce_workspace_size(512, 256, 0, 256, ctypes.byref(n)) == _lib.LMCE_ERR_SHAPE
    assert lib.lmce_workspace_size(512, 100, 4096, 256, ctypes.byref(n)) == _lib.LMCE_ERR_UNSUPPORTED
    assert lib.lmce_workspace_size(512, 256, 4096, 100, ctypes.byref(n)) == _lib.LMCE_ERR_UNSUPPORTED
    assert lib.lmce_workspace_size(512, 256, 4096, 2048, ctypes.byref(n)) == _lib.LMCE_ERR_UNSUPPORTED
    assert lib.lmce_workspace_size(512, 256, 4096, 256, None) == _lib.LMCE_ERR_NULL
    assert lib.lmce_workspace_size(512, 256, 4096, 256, ctypes.byref(n)) == _lib.LMCE_OK
    assert n.value > 0


def test_workspace_never_holds_the_logits():
    """The pages' point: the L x V logits are the memory peak; the workspace
    holds no L x V array at any workload size."""
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    assert facts["default_chunk_rows"] == 256
    for wl in synth.WORKLOADS.values():
        ws = _lib.workspace_size(wl.L, wl.H, wl.V, wl.chunk_rows)
        # linear in L (per-segment row statistics, the dW pass's row
        # compaction, row orders), plus bounded exchange, parking and
        # partial-slice areas (at most 256 workgroups with 512 KiB of exchange
        # (two slots of two 256 x 256 bf16 tiles) and 256 KiB each of the
        # others: 256 MiB), and
        # an L x H bf16 area of gathered h rows only where the passes cannot
        # read h through the row order (128-wide slices, or h past 2^31
        # bytes); no transposed copy of h or W (the GEMMs read both in
        # place), never L * V, and no L x H fp32 array (the training
        # forward's O lives in the caller's dh)
        gathered = wl.H < 1024 or wl.H % 256 != 0 or wl.L * wl.H * 2 > 0x7ffff000
        bound = (2 * wl.L * wl.H if gathered else 0) + 96 * wl.L + (264 << 20)
        assert ws <= bound, (wl.name, ws, bound)
        if not gathered:
            assert ws <= 320 << 20, (wl.name, ws)
        if wl.V > 100000:
            assert ws < 0.1 * wl.L * wl.V * 4, (wl.name, ws)
    # 160k tokens of the Qwen3-4B head: the fp32 logits alone would need
    # ~92.7 GiB, more than the 80 GB card of the page; the workspace is tiny.
    wl = synth.WORKLOADS["qwen3_4b_160k"]
    assert wl.L == facts["qwen3_4b_chunked_reach_tokens"]
    assert wl.L * wl.V * 4 / 2**30 > facts["card_memory_gb"]
    assert _lib.workspace_size(wl.L, wl.H, wl.V, 256) < 2**30
    # Results never depend on chunk_rows, and the schedule inputs that do
    # (segments) are identical across the allowed chunk sizes.
    sizes = {_lib.workspace_size(8192, 1024, 151936, c) for c in (32, 128, 256, 512, 1024)}
    assert len(sizes) == 1


def _fwd(lib, h=FAKE, W=FAKE, y=FAKE, L=512, H=256, V=4096, ign=-100, chunk=256, loss=FAKE, lse=FAKE, ws=FAKE,
         wsb=1 << 40, stream=None):
    return lib.lmce_fwd(h, W, y, L, H, V, ign, chunk, loss, lse, ws, wsb, stream)


def _bwd(lib, h=FAKE, W=FAKE, y=FAKE, lse=FAKE, L=512, H=256, V=4096, ign=-100, chunk=256, g=FAKE, dh=FAKE,
         dW=FAKE, ws=FAKE, wsb=1 << 40, stream=None):
    return lib.lmce_bwd(h, W, y, lse, L, H, V, ign, chunk, g, dh, dW, ws, wsb, stream)


def test_fwd_rejects_bad_arguments(lib):
    E = _lib
    assert _fwd(lib, h=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, W=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, y=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, loss=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, lse=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, ws=None) == E.LMCE_ERR_NULL
    assert _fwd(lib, h=FAKE + 8) == E.LMCE_ERR_NULL  # misaligned
    assert _fwd(lib, ws=FAKE + 16) == E.LMCE_ERR_NULL
    assert _fwd(lib, L=0) == E.LMCE_ERR_SHAPE
    assert _fwd(lib, V=-1) == E.LMCE_ERR_SHAPE
    assert _fwd(lib, H=32) == E.LMCE_ERR_UNSUPPORTED
    assert _fwd(lib, H=200) == E.LMCE_ERR_UNSUPPORTED
    assert _fwd(lib, H=192) == E.LMCE_ERR_UNSUPPORTED  # a multiple of 64 but not of 128
    assert _fwd(lib, chunk=0) == E.LMCE_ERR_UNSUPPORTED
    assert _fwd(lib, chunk=250) == E.LMCE_ERR_UNSUPPORTED
    need = _lib.workspace_size(512, 256, 4096, 256)
    assert _fwd(lib, wsb=need - 1) == E.LMCE_ERR_WORKSPACE


def test_bwd_rejects_bad_arguments(lib):
    E = _lib
    for kw in ("h", "W", "y", "lse", "g", "dh", "dW", "ws"):
        assert _bwd(lib, **{kw: None}) == E.LMCE_ERR_NULL, kw
    assert _bwd(lib, dh=FAKE + 4) == E.LMCE_ERR_NULL
    assert _bwd(lib, L=-5) == E.LMCE_ERR_SHAPE
    assert _bwd(lib, H=96) == E.LMCE_ERR_UNSUPPORTED
    assert _bwd(lib, chunk=2048) == E.LMCE_ERR_UNSUPPORTED
    need = _lib.workspace_size(512, 256, 4096, 256)
    assert _bwd(lib, wsb=need - 1) == E.LMCE_ERR_WORKSPACE


def test_train_pair_rejects_bad_arguments(lib):
    E = _lib
    need = _lib.workspace_size(512, 256, 4096, 256)

    def fwd_t(h=FAKE, W=FAKE, y=FAKE, L=512, H=256, V=4096, loss=FAKE, lse=FAKE, dh=FAKE, ws=FAKE, wsb=1 << 40):
        return lib.lmce_fwd_train(h, W, y, L, H, V, -100, 256, loss, lse, dh, ws, wsb, None)

    def bwd_t(h=FAKE, W=FAKE, y=FAKE, lse=FAKE, L=512, H=256, V=4096, g=FAKE, dh=FAKE, dW=FAKE, ws=FAKE,
              wsb=1 << 40):
        return lib.lmce_bwd_train(h, W, y, lse, L, H, V, -100, 256, g, dh, dW, ws, wsb, None)

    for kw in ("h", "W", "y", "loss", "lse", "dh", "ws"):
        assert fwd_t(**{kw: None}) == E.LMCE_ERR_NULL, kw
    assert fwd_t(dh=FAKE + 4) == E.LMCE_ERR_NULL
    assert fwd_t(L=0) == E.LMCE_ERR_SHAPE
    assert fwd_t(H=192) == E.LMCE_ERR_UNSUPPORTED
    assert fwd_t(wsb=need - 1) == E.LMCE_ERR_WORKSPACE
    for kw in ("h", "W", "y", "lse", "g", "dh", "dW", "ws"):
        assert bwd_t(**{kw: None}) == E.LMCE_ERR_NULL, kw
    assert bwd_t(dW=FAKE + 4) == E.LMCE_ERR_NULL
    assert bwd_t(V=0) == E.LMCE_ERR_SHAPE
    assert bwd_t(wsb=need - 1) == E.LMCE_ERR_WORKSPACE
    assert _lib.strerror(E.LMCE_ERR_STATE).startswith("lmce_bwd_train")


def test_read_status_rejects_bad_workspace(lib):
    assert lib.lmce_read_status(None, None) == _lib.LMCE_ERR_NULL
    assert lib.lmce_read_status(FAKE + 4, None) == _lib.LMCE_ERR_NULL


def test_golden_facts_cite_the_pages():
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    for key, val in facts.items():
        if key.startswith("_"):
            continue
        assert key in facts["_cite"], f"{key} has no citation"
    assert math.isclose(facts["card_memory_gb"], 80)


def test_noalloc_forward_rejects_before_enqueuing(lib):
    """lmce_fwd_noalloc: shape and pointer errors as lmce_fwd, and shapes past
    its fixed area (L > 2^20 rows) are refused before any device call."""
    f = lib.lmce_fwd_noalloc
    assert f(FAKE, FAKE, FAKE, 0, 256, 4096, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_SHAPE
    assert f(FAKE, FAKE, FAKE, 512, 100, 4096, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_UNSUPPORTED
    assert f(None, FAKE, FAKE, 512, 256, 4096, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_NULL
    assert f(FAKE + 2, FAKE, FAKE, 512, 256, 4096, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_NULL
    assert f(FAKE, FAKE, FAKE, 512, 256, 4096, -100, 256, FAKE, None, None) == _lib.LMCE_ERR_NULL
    assert f(FAKE, FAKE, FAKE, (1 << 20) + 1, 256, 151936, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_SCRATCH
    assert f(FAKE, FAKE, FAKE, 1 << 21, 128, 1, -100, 256, FAKE, FAKE, None) == _lib.LMCE_ERR_SCRATCH


def test_binding_refuses_host_tensors():
    """The torch-level entry points take device tensors only: host tensors
    raise before anything reaches the library (there is no CPU path)."""
    import torch

    import lm_head_chunked_amd as lm

    h = torch.zeros(8, 128, dtype=torch.bfloat16)
    W = torch.zeros(16, 128, dtype=torch.bfloat16)
    y = torch.zeros(8, dtype=torch.int64)
    for call in (lambda: lm.lmce_fwd(h, W, y), lambda: lm.lmce_fwd_train(h, W, y),
                 lambda: lm.lmce_bwd(h, W, y, torch.zeros(8)), lambda: lm.lmce_chunked_fwd(h, W, y)):
        try:
            call()
        except ValueError as e:
            assert "device" in str(e)
            continue
        raise AssertionError("a host tensor was accepted")
    x = torch.zeros(8, 128, dtype=torch.bfloat16)
    try:
        lm.lmce_mlp_fwd(x, W, W, W.t().contiguous(), 8)
    except TypeError as e:
        assert "device" in str(e)
    else:
        raise AssertionError("a host tensor was accepted by the MLP")
