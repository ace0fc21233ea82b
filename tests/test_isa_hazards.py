"""The gfx950 assembly of the kernels keeps every wide store's data intact.

A buffer store of more than 8 bytes whose scalar offset is an SGPR gets no
wait state from the compiler before a VALU write of its data registers, and
on gfx950 such a write can reach the data before the store has read it: a
training-forward build that reused the registers at once wrote wrong exchange
tiles, differently on every run.  The library therefore gives its wide buffer
stores a constant scalar offset (the compiler then separates store and write
itself).  This test builds the device code to assembly (hipcc cross-compiles
without a GPU) and checks, in every kernel:
  * every buffer store of 12 or 16 bytes has a constant scalar offset;
  * no store of 12 or 16 bytes is followed at once by a VALU instruction that
    writes one of its data registers.
"""

import os
import re
import subprocess
import tempfile

import pytest

from lm_head_chunked_amd import build

WIDE_STORE = re.compile(r"^(buffer|global|scratch|flat)_store_(dwordx3|dwordx4|b96|b128)\b")


def vregs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bv(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def kernel_instructions(asm):
    """(kernel, instruction) in program order, labels and directives dropped."""
    kern, out = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kern = m.group(1)
            continue
        s = line.split(";")[0].strip()
        if kern is None or not s or s.endswith(":") or s.startswith("."):
            continue
        out.append((kern, s))
    return out


def wide_store_problems(asm):
    insts = kernel_instructions(asm)
    problems, n = [], 0
    for i, (kern, s) in enumerate(insts):
        op = s.split()[0]
        if not WIDE_STORE.match(op):
            continue
        n += 1
        args = [a.strip() for a in s[len(op):].split(",")]
        # buffer_store vdata, vaddr, srsrc, soffset ...; global/flat/scratch: vaddr, vdata, ...
        data = vregs(args[0]) if op.startswith("buffer") else vregs(args[1])
        if op.startswith("buffer") and re.match(r"^s(\d+|\[)", args[3].split()[0]):
            problems.append(f"{kern}: SGPR scalar offset on a wide buffer store: {s}")
        j = i + 1
        while j < len(insts) and insts[j][1].startswith("s_nop"):
            j += 1
        if j < len(insts) and j == i + 1:
            nxt = insts[j][1]
            nop = nxt.split()[0]
            if nop.startswith("v_") and vregs(nxt[len(nop):].split(",")[0]) & data:
                problems.append(f"{kern}: data registers of '{s}' written at once by '{nxt}'")
    return n, problems


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not available")
    texts = {}
    with tempfile.TemporaryDirectory() as tmp:
        for src in ("lmce_fwd.hip", "lmce_bwd.hip"):
            out = os.path.join(tmp, src + ".s")
            cmd = [build.hipcc(), *[f for f in build.flags() if f != "-fPIC"], "--cuda-device-only", "-S",
                   os.path.join(build.CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-2000:]
            texts[src] = open(out).read()
    return texts


def test_wide_stores_keep_their_data(device_asm):
    total = 0
    for src, asm in device_asm.items():
        n, problems = wide_store_problems(asm)
        total += n
        assert not problems, "\n".join(problems)
    assert total > 0  # the exchange writes are 16-byte stores


def test_checker_flags_the_hazard():
    """The scanner itself: an SGPR-offset wide store whose data is overwritten at once."""
    asm = "\n".join([
        "_Zkernel:",
        "\tbuffer_store_dwordx4 v[12:15], v17, s[84:87], s72 offen sc1",
        "\tv_xor_b32_e32 v12, v7, v0",
        "\tbuffer_store_dwordx4 v[20:23], v18, s[84:87], 0 offen sc1",
        "\tv_mov_b32_e32 v30, v1",
    ])
    n, problems = wide_store_problems(asm)
    assert n == 2
    assert len(problems) == 2  # the SGPR offset and the immediate overwrite of the first store
    assert all("v[12:15]" in p for p in problems)
