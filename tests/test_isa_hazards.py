"""The gfx950 assembly of the kernels keeps every wide store's data intact,
and no instruction touches the registers of an LDS fragment read in flight.

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

The GEMM engine reads its MFMA fragments from LDS with inline-asm ds_read_b128
and waits for them later with its own s_waitcnt lgkmcnt.  The compiler takes
an inline-asm output as written when the asm statement ends, so it could copy,
spill or reuse such a register while the read is still in flight, and the late
read would then overwrite whatever the register holds by then (an address, for
instance).  The engine keeps reads in flight across its K-loop's back edge, so
the scan follows every branch: from each path state it tracks the reads not yet
retired by an lgkmcnt wait and fails on any other instruction that reads or
writes one of their registers.
"""

import os
import re
import subprocess
import tempfile

import pytest

from lm_head_chunked_amd import build

# Scalar-memory operations: counted by lgkmcnt like LDS operations, but their
# results return out of order.
SMEM_OPS = ("s_load", "s_buffer_load", "s_memtime", "s_memrealtime", "s_dcache", "s_scratch_load", "s_atc_probe")
WIDE_STORE = re.compile(r"^(buffer|global|scratch|flat)_store_(dwordx3|dwordx4|b96|b128)\b")


def regs_va(text):
    """VGPR and AGPR names an operand list mentions (v7, a[4:7], ...)."""
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", text):
        out |= {f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"\b([va])(\d+)\b", text):
        out.add(m.group(1) + m.group(2))
    return out


def kernel_programs(asm):
    """{kernel: (instructions [(text, from inline asm)], {label: index})}."""
    progs, kern, inasm = {}, None, False
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kern = m.group(1)
            progs[kern] = ([], {})
            continue
        if kern is None:
            continue
        if ";;#ASMSTART" in line:
            inasm = True
            continue
        if ";;#ASMEND" in line:
            inasm = False
            continue
        m = re.match(r"^(\.L\w+):", line)
        if m:
            progs[kern][1][m.group(1)] = len(progs[kern][0])
            continue
        s = line.split(";")[0].strip()
        if s and not s.startswith("."):
            progs[kern][0].append((s, inasm))
    return progs


def inflight_problems(insts, labels, depth=16):
    """Instructions that touch a register of an inline-asm LDS read still in flight, on any path.

    A path state is (instruction index, queue of outstanding LDS operations),
    where an inline-asm ds_read carries its destination registers and any other
    LDS operation none; s_waitcnt lgkmcnt(n) keeps the newest n.  LDS
    operations complete in order.  Scalar-memory operations (s_load,
    s_memtime, ...) also count in lgkmcnt but complete out of order, so they
    are not queued: with one outstanding, lgkmcnt(n) may be met while the
    newest n LDS operations are still in flight, which is what keeping the
    newest n LDS entries models."""
    problems, seen, work = set(), set(), [(0, ())]
    while work:
        i, q = work.pop()
        while i < len(insts) and (i, q) not in seen:
            seen.add((i, q))
            s, inasm = insts[i]
            op = s.split()[0]
            args = s[len(op):]
            if op == "s_waitcnt" and "lgkmcnt" in s:
                n = int(re.search(r"lgkmcnt\((\d+)\)", s).group(1))
                q = q[len(q) - n:] if len(q) > n else q
                i += 1
                continue
            live = set().union(*map(set, q)) if q else set()
            if op.startswith("ds_read") and inasm:
                dst, src = args.split(",")[0], ",".join(args.split(",")[1:])
                if regs_va(src) & live:
                    problems.add(f"address of '{s}' still being loaded")
                q = q + (tuple(sorted(regs_va(dst))),)
            else:
                if regs_va(args) & live:
                    problems.add(f"'{s}' touches {sorted(regs_va(args) & live)[:4]} while a fragment read is in flight")
                if op.startswith("ds_"):
                    q = q + ((),)
            q = q[-depth:]
            if op == "s_endpgm":
                break
            if op.startswith(("s_branch", "s_cbranch", "s_setpc")):
                tgt = args.strip().split(",")[-1].strip()
                if tgt in labels:
                    work.append((labels[tgt], q))
                if op.startswith("s_branch"):
                    break
            i += 1
    return problems, len(seen)


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
        for src in ("lmce_fwd.hip", "lmce_bwd.hip", "lmce_gemm.hip"):
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


def test_fragment_reads_in_flight_are_left_alone(device_asm):
    kernels = 0
    for src, asm in device_asm.items():
        for kern, (insts, labels) in kernel_programs(asm).items():
            if not any(inasm and s.startswith("ds_read") for s, inasm in insts):
                continue
            kernels += 1
            problems, states = inflight_problems(insts, labels)
            assert states > len(insts) // 2, kern
            assert not problems, kern + ":\n" + "\n".join(sorted(problems)[:10])
    assert kernels >= 10  # the group passes, the plain forward and the GEMM kernels use the engine


def test_inflight_checker_follows_the_back_edge():
    """The scanner itself: a read issued at the end of a loop body and waited for
    at the top of the next iteration, with a register reuse in between that only
    the back edge reaches."""
    asm = "\n".join([
        "_Zkernel:",
        "\ts_mov_b32 s0, 0",
        ".LBB0_1:",
        "\tv_add_u32_e32 v8, 1, v8",            # reached from the back edge with the read in flight
        "\ts_waitcnt lgkmcnt(0)",
        "\tv_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], v[4:7], v[16:31]",
        "\t;;#ASMSTART",
        "\tds_read_b128 v[4:7], v9",
        "\t;;#ASMEND",
        "\tv_mov_b32_e32 v10, v1",               # unrelated: fine
        "\ts_cbranch_scc1 .LBB0_1",
        "\ts_waitcnt lgkmcnt(0)",
        "\ts_endpgm",
    ])
    insts, labels = kernel_programs(asm)["_Zkernel"]
    problems, _ = inflight_problems(insts, labels)
    assert problems == set()  # v8 is not a fragment register
    insts[1] = ("v_add_u32_e32 v5, 1, v5", False)  # now the loop top reuses a register of the read
    problems, _ = inflight_problems(insts, labels)
    assert len(problems) == 1 and "v5" in next(iter(problems))


def test_inflight_checker_treats_scalar_loads_as_out_of_order():
    """The scanner itself: an s_memtime issued after a fragment read does not
    let lgkmcnt(1) retire that read (the scalar result may have come back
    first), so touching the read's registers after that wait is a problem;
    after lgkmcnt(0) it is not."""
    body = [
        "_Zkernel:",
        "\t;;#ASMSTART",
        "\tds_read_b128 v[4:7], v9",
        "\t;;#ASMEND",
        "\ts_memtime s[2:3]",
        "\ts_waitcnt lgkmcnt(1)",
        "\tv_mov_b32_e32 v5, v1",
        "\ts_endpgm",
    ]
    insts, labels = kernel_programs("\n".join(body))["_Zkernel"]
    problems, _ = inflight_problems(insts, labels)
    assert len(problems) == 1 and "v5" in next(iter(problems))
    body[5] = "\ts_waitcnt lgkmcnt(0)"
    insts, labels = kernel_programs("\n".join(body))["_Zkernel"]
    problems, _ = inflight_problems(insts, labels)
    assert problems == set()
